"""Pins of the oracle's E4M3 / E2M1 / NVFP4 codecs (CPU only).

The pins are independent of the oracle's own code: PyTorch's float8_e4m3fn
conversion (a library routine), the OCP format anchors and the E2M1 rounding
table worked by hand (tests/golden), and properties the formats fix.
"""
import math

import numpy as np
import pytest
import torch

from conftest import read_golden


def _torch_e4m3_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_decode_all_codes_matches_torch(oracle):
    got = oracle.e4m3_value(np.arange(256))
    want = _torch_e4m3_values()
    same = (got == want) | (np.isnan(got) & np.isnan(want))
    assert same.all()
    assert (np.signbit(got) == np.signbit(want))[~np.isnan(want)].all()


def test_e4m3_anchor_values(oracle):
    for code, val in read_golden("e4m3_anchors.txt"):
        got = float(oracle.e4m3_value([int(code, 16)])[0])
        want = float(val)
        if math.isnan(want):
            assert math.isnan(got)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_e4m3_structure(oracle):
    v = oracle.e4m3_value(np.arange(128))
    finite = v[:127]
    assert np.all(np.diff(finite) > 0), "non-negative codes 0x00..0x7E must increase strictly"
    assert np.isnan(v[127])
    neg = oracle.e4m3_value(np.arange(128, 256))
    assert np.array_equal(neg[:127], -finite)
    assert (np.isnan(oracle.e4m3_value(np.arange(256)))).sum() == 2


def _e4m3_encode_inputs():
    vals = _torch_e4m3_values()[:127]
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(0)
    pts = np.concatenate([
        vals, mids,
        np.nextafter(mids.astype(np.float32), np.float32(0)).astype(np.float64),
        np.nextafter(mids.astype(np.float32), np.float32(1e9)).astype(np.float64),
        rng.uniform(0, 464, 4000), np.exp(rng.uniform(-16, 6.1, 4000)),
    ]).astype(np.float32)
    pts = pts[pts <= 464.0]
    return np.concatenate([pts, -pts])


def test_e4m3_encode_rne_matches_torch(oracle):
    x = _e4m3_encode_inputs()
    got = oracle.e4m3_encode(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), int(got[i]), int(want[i])) for i in bad[:10]]


def test_e4m3_encode_saturates_and_nan(oracle):
    big = np.array([448.0, 464.0, 464.01, 480.0, 1e6, 1e30, np.inf], dtype=np.float32)
    assert (oracle.e4m3_encode(big) == 0x7E).all()
    assert (oracle.e4m3_encode(-big) == 0xFE).all()
    assert oracle.e4m3_encode([np.nan])[0] & 0x7F == 0x7F
    assert oracle.e4m3_encode([-0.0])[0] == 0x80


def test_e2m1_table(oracle):
    for code, val in read_golden("e2m1_table.txt"):
        got = float(oracle.e2m1_value([int(code, 16)])[0])
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), code


def test_e2m1_rounding_table(oracle):
    for x, code in read_golden("e2m1_rounding.txt"):
        assert int(oracle.e2m1_encode([float(x)])[0]) == int(code, 16), x


def test_e2m1_encode_is_nearest(oracle):
    """Any input maps to a grid point at least as close as every other one."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    x = np.random.default_rng(1).uniform(-7, 7, 20000).astype(np.float32)
    codes = oracle.e2m1_encode(x)
    vals = oracle.e2m1_value(codes)
    ax = np.minimum(np.abs(x.astype(np.float64)), 6.0)
    best = np.min(np.abs(grid[None, :] - ax[:, None]), axis=1)
    assert np.all(np.abs(np.abs(vals) - ax) <= best + 0.0)
    assert np.all((np.signbit(vals)) == np.signbit(x))


# ------------------------------------------------------------------ NVFP4
def test_nvfp4_product_table_exhaustive(oracle):
    """All 16 E2M1 codes x 256 E4M3 scales: the value is the exact product, it
    has at most 6 significant bits, and lies in [2^-10, 2688] when nonzero."""
    e2m1 = oracle.e2m1_value(np.arange(16))
    e4m3 = _torch_e4m3_values()
    L = oracle.lib()
    n_exact = 0
    for s in range(256):
        if np.isnan(e4m3[s]):
            continue
        for c in range(16):
            v = L.ref_nvfp4_value(c, s, 1.0)
            assert v == e2m1[c] * e4m3[s]
            if v != 0:
                m, e = math.frexp(abs(v))
                assert (m * 64) == int(m * 64), "more than 6 significant bits"
                assert 2.0 ** -10 <= abs(v) <= 2688.0
                # exact in float16 (11 significant bits, range to 65504)
                assert float(np.float16(v)) == v
            n_exact += 1
    assert n_exact == 254 * 16


def test_page_table_counts(oracle):
    facts = {r[0]: int(r[1]) for r in read_golden("page_facts.txt")}
    # 256 scales x 8 magnitudes x 1 byte = the pages' 2 KB lookup table
    assert facts["e4m3_scale_values"] * facts["e2m1_magnitudes"] == facts["lds_table_bytes"]
    assert len(set(np.abs(oracle.e2m1_value(np.arange(16))))) == facts["e2m1_magnitudes"]


def test_nvfp4_byte_cost_matches_pages(oracle):
    """16 elements -> 8 code bytes + 1 scale byte = 0.5625 B/element, the pages' 34,560/61,440."""
    facts = {r[0]: int(r[1]) for r in read_golden("page_facts.txt")}
    codes, scales = oracle.nvfp4_quantize(np.ones((1, 16), np.float32), 1.0)
    per_elem = (codes.size + scales.size) / 16
    assert per_elem == facts["nvfp4_kv_bytes_per_token"] / facts["fp8_kv_bytes_per_token"]
    assert 10000 - 10000 * per_elem == facts["saving_percent_x100"]
    # K+V of 4 heads x 128 dims per layer at 0.5625 B = 576 B; 34,560 / 576 = 60 layers
    assert facts["nvfp4_kv_bytes_per_token"] % int(2 * 4 * 128 * per_elem) == 0


def _deq(oracle, codes, scales, ts):
    e2m1 = oracle.e2m1_value(np.arange(16))
    e4m3 = _torch_e4m3_values()
    lo = codes & 0xF
    hi = codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (16,))
    return e2m1[c] * e4m3[scales][..., None] * ts


def test_nvfp4_zero_block(oracle):
    codes, scales = oracle.nvfp4_quantize(np.zeros((3, 16), np.float32), 0.01)
    assert (codes == 0).all() and (scales == 0).all()
    tiny = np.full((1, 16), 1e-30, np.float32)
    codes, scales = oracle.nvfp4_quantize(tiny, 1.0)
    assert (codes == 0).all() and (scales == 0).all()


def test_nvfp4_roundtrip_of_representable_blocks(oracle):
    """A block whose values are c * s * ts with some |c| = 6 quantises back to the same bytes."""
    rng = np.random.default_rng(2)
    e4m3 = _torch_e4m3_values()
    ts = float(np.float32(8 / (6 * 448)))
    for _ in range(300):
        c = rng.integers(0, 16, 16).astype(np.uint8)
        c[rng.integers(0, 16)] = 7 | (8 * rng.integers(0, 2))
        s = int(rng.integers(8, 0x7E))  # normal scales
        vals = (oracle.e2m1_value(c) * e4m3[s] * ts).astype(np.float32)
        codes, scales = oracle.nvfp4_quantize(vals, ts)
        got_vals = _deq(oracle, codes, scales, ts)[0]
        assert scales[0] == s
        # +0 and -0 may differ only where the value is zero
        assert np.array_equal(got_vals, oracle.e2m1_value(c) * e4m3[s] * ts)
        nz = oracle.e2m1_value(c) != 0
        lo = codes[0] & 0xF
        hi = codes[0] >> 4
        got_c = np.stack([lo, hi], -1).reshape(16)
        assert np.array_equal(got_c[nz], c[nz])


def test_nvfp4_error_bound(oracle):
    """|x - q(x)| is at most half an E2M1 grid step (1, 0.5 or 0.25 scaled by s*ts), unless saturated."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2000, 16)).astype(np.float32)
    ts = float(np.float32(8 / (6 * 448)))
    codes, scales = oracle.nvfp4_quantize(x, ts)
    codes, scales = codes.reshape(2000, 8), scales.reshape(2000)
    e4m3 = _torch_e4m3_values()
    deq = _deq(oracle, codes, scales, ts)
    step = e4m3[scales][:, None] * ts
    y = np.abs(x / step)
    half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0))
    sat = y > 6
    err = np.abs(deq - x)
    assert np.all(err[~sat] <= half[~sat] * step.repeat(16, 1)[~sat] * (1 + 1e-6))
    # amax maps close to 6: the scale is the E4M3 rounding of amax/6/ts
    amax = np.abs(x).max(1)
    assert np.all(np.abs(e4m3[scales] - amax / 6 / ts) <= e4m3[scales] / 16 + 1e-12)


def test_nvfp4_saturation(oracle):
    x = np.full((1, 16), 1e6, np.float32)
    x[0, 3] = -1e6
    codes, scales = oracle.nvfp4_quantize(x, 1.0)
    assert scales[0] == 0x7E
    lo = codes[0] & 0xF
    hi = codes[0] >> 4
    c = np.stack([lo, hi], -1).reshape(16)
    assert (c[np.arange(16) != 3] == 7).all() and c[3] == 0xF


def test_queries_e4m3(oracle):
    x = np.random.default_rng(4).standard_normal(5000).astype(np.float32)
    got = oracle.quantize_queries(x, 1.0)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    dec = oracle.decode_queries(got, oracle.FP8_E4M3, 0.5)
    assert np.array_equal(dec, torch.from_numpy(want).view(torch.float8_e4m3fn).double().numpy() * 0.5)


# ---------------------------------------------------------------- FP8 cache elements
def test_fp8_byte_cost_matches_pages(oracle):
    """One byte per element: 128 B of index keys and 1,024 B of K+V (4 heads x 128 dims) per
    token and layer, the pages' FP8 figures; 61,440 B per token is 60 such layers, the same
    layer count as NVFP4's 34,560 B at 576 B per layer."""
    facts = {r[0]: int(r[1]) for r in read_golden("page_facts.txt")}
    idx = oracle.OracleCache(oracle.FP8_E4M3, oracle.TOKEN_MAJOR, 1, 1, 1.0)
    assert idx.bytes.size // 128 == facts["index_bytes_per_token_fp8"]
    kv = oracle.OracleCache(oracle.FP8_E4M3, oracle.TOKEN_MAJOR, facts["kv_heads"], 1, 1.0)
    assert 2 * kv.bytes.size // 128 == facts["dense_kv_bytes_per_token_fp8"]
    layers = facts["fp8_kv_bytes_per_token"] // facts["dense_kv_bytes_per_token_fp8"]
    assert layers * facts["dense_kv_bytes_per_token_fp8"] == facts["fp8_kv_bytes_per_token"]
    assert layers * 576 == facts["nvfp4_kv_bytes_per_token"]


def test_fp8_quantize_matches_torch(oracle):
    """In range, an FP8 cache code is PyTorch's float8_e4m3fn rounding of the FP32 quotient x / ts."""
    rng = np.random.default_rng(21)
    ts = float(np.float32(8 / 448))
    x = np.clip(rng.standard_normal(20000).astype(np.float32) * 2, -7.9, 7.9).astype(np.float32)
    x[:50] = 0.0
    x[50:100] = rng.standard_normal(50).astype(np.float32) * 1e-4  # E4M3 subnormals
    got = oracle.fp8_quantize(x, ts)
    y = torch.from_numpy(x) / torch.tensor(ts, dtype=torch.float32)
    want = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)
    vals = _torch_e4m3_values()
    assert np.array_equal(np.array([oracle.fp8_value(int(c), ts) for c in got[:200]]), vals[got[:200]] * ts)


def test_fp8_quantize_rounds_even_saturates_and_keeps_nan(oracle):
    ts = 0.25  # a power of two: x / ts is exact, so the rounding seen is the E4M3 one
    vals = _torch_e4m3_values()
    for c in range(0, 0x7E):  # consecutive finite non-negative codes c, c + 1
        mid = (vals[c] + vals[c + 1]) / 2
        want = c if c % 2 == 0 else c + 1
        assert oracle.fp8_quantize(np.float32(mid * ts), ts) == want
        assert oracle.fp8_quantize(np.float32(-mid * ts), ts) == (want | 0x80)
    for big in (449.0 * ts, 1e6, 3e38):
        assert oracle.fp8_quantize(np.float32(big), ts) == 0x7E
        assert oracle.fp8_quantize(np.float32(-big), ts) == 0xFE
    assert oracle.fp8_quantize(np.float32(np.nan), ts) & 0x7F == 0x7F
    assert oracle.fp8_quantize(np.float32(-0.0), ts) == 0x80


def test_fp8_layouts_hold_the_same_values(oracle):
    """Token-major [tok][dim] and dim-major [dim][tok] slabs: the same bytes at transposed
    offsets, and each value is E4M3(x / ts) * ts."""
    rng = np.random.default_rng(22)
    ts = float(np.float32(8 / 448))
    x = rng.standard_normal((40, 4, 128)).astype(np.float32)
    slots = rng.choice(3 * 128, size=40, replace=False)
    tm = oracle.OracleCache(oracle.FP8_E4M3, oracle.TOKEN_MAJOR, 4, 3, ts)
    dm = oracle.OracleCache(oracle.FP8_E4M3, oracle.DIM_MAJOR, 4, 3, ts)
    hr = oracle.OracleCache(oracle.FP8_E4M3, oracle.HALF_ROWS, 4, 3, ts)
    tm.write(slots, x)
    dm.write(slots, x)
    hr.write(slots, x)
    a = tm.bytes.reshape(3, 4, 128, 128)
    b = dm.bytes.reshape(3, 4, 128, 128)
    assert np.array_equal(a, np.swapaxes(b, -1, -2))
    # half rows: 16-token chunks, each as two 1 KB halves (dims 0..63, then 64..127)
    h = hr.bytes.reshape(3, 4, 8, 2, 16, 64)
    assert np.array_equal(a.reshape(3, 4, 8, 16, 2, 64), np.transpose(h, (0, 1, 2, 4, 3, 5)))
    codes = oracle.fp8_quantize(x, ts)
    for i, s in enumerate(slots):
        assert np.array_equal(a[s // 128, :, s % 128, :], codes[i])
    vals = _torch_e4m3_values()
    for i, s in enumerate(slots[:5]):
        for h in range(4):
            for d in (0, 17, 127):
                for c in (tm, dm, hr):
                    assert c.value(int(s // 128), h, int(s % 128), d) == vals[codes[i, h, d]] * ts


# ---------------------------------------------------------------- NVFP4 page placement
def _nvfp4_expected_pool(codes, scales, slots, heads, num_pages, dim_major):
    """Bytes of an NVFP4 page pool holding the given per-element E2M1 codes [n][heads][128] and
    per-group E4M3 scale codes [n][heads][8] at `slots`, placed by the slab layouts the C ABI
    defines (9,216 B per (page, head): 8,192 B of codes, then 1,024 B of scales).
    Token-major: codes [tok][64 B], byte i = dim 2i (low nibble) | dim 2i+1 (high); scales [tok][8].
    Dim-major: codes [dim][64 B], byte i = token 2i (low) | token 2i+1 (high); scales [8][tok]."""
    pool = np.zeros((num_pages, heads, 9216), np.uint8)
    for i, s in enumerate(slots):
        p, t = int(s) // 128, int(s) % 128
        for h in range(heads):
            slab = pool[p, h]
            for d in range(128):
                c = int(codes[i, h, d])
                if dim_major:
                    byte, shift = d * 64 + t // 2, 4 * (t % 2)
                else:
                    byte, shift = t * 64 + d // 2, 4 * (d % 2)
                slab[byte] |= np.uint8(c << shift)
            for j in range(8):
                slab[8192 + (j * 128 + t if dim_major else t * 8 + j)] = scales[i, h, j]
    return pool.reshape(-1)


@pytest.mark.parametrize("heads,layout", [(4, "token_major"), (1, "token_major"), (4, "dim_major")])
def test_nvfp4_cache_bytes_sit_where_the_layout_puts_them(oracle, heads, layout):
    """The oracle's NVFP4 cache writer against the layout definition, with no quantiser or
    decoder in the comparison.  Rows are built from drawn E2M1 codes and E4M3 scale codes as
    e2m1 * e4m3 * ts with a power-of-two ts and one magnitude-6 element per 16-dim group, so
    every FP32 step of the amax recipe is exact: the scale is the drawn one and each code
    comes back.  The rows go to shuffled slots of a 3-page pool (token pairs sharing a
    dim-major byte included); every byte of the pool must equal the layout's placement of the
    drawn codes and zero elsewhere.  Keys (4 heads) and index keys (1 head) are token-major,
    values dim-major."""
    rng = np.random.default_rng(31 + heads + (layout == "dim_major"))
    e4m3 = _torch_e4m3_values()
    ts = 2.0 ** -8
    n, num_pages = 150, 3
    codes = rng.choice(np.array([c for c in range(16) if c != 8], np.uint8), size=(n, heads, 128))
    sixes = rng.integers(0, 16, size=(n, heads, 8))
    g = codes.reshape(n, heads, 8, 16)
    np.put_along_axis(g, sixes[..., None], (7 | (8 * rng.integers(0, 2, size=(n, heads, 8, 1)))).astype(np.uint8),
                      axis=-1)
    codes = g.reshape(n, heads, 128)
    scales = rng.integers(8, 0x7E, size=(n, heads, 8)).astype(np.uint8)  # normal E4M3 scales
    x = oracle.e2m1_value(codes) * np.repeat(e4m3[scales], 16, axis=-1) * ts
    x = x.astype(np.float32)
    assert np.array_equal(x.astype(np.float64), oracle.e2m1_value(codes) * np.repeat(e4m3[scales], 16, -1) * ts)
    slots = rng.choice(num_pages * 128, size=n, replace=False)
    dm = layout == "dim_major"
    cache = oracle.OracleCache(oracle.NVFP4, oracle.DIM_MAJOR if dm else oracle.TOKEN_MAJOR, heads, num_pages, ts)
    cache.write(slots, x if heads > 1 else x[:, 0])
    want = _nvfp4_expected_pool(codes, scales, slots, heads, num_pages, dm)
    assert np.array_equal(cache.bytes, want)


@pytest.mark.parametrize("layout", ["token_major", "dim_major"])
def test_nvfp4_cache_values_stay_within_a_grid_step_of_their_source(oracle, layout):
    """N(0,1) rows written at shuffled slots, read back by the tests' own decoder of the
    documented layout (helpers.decode_pages_f64): every (slot, head, dim) lies within one E2M1
    grid step of its source value, and every slot not written reads as zero.  The step bound
    is independent of the oracle: a group's E4M3 scale s is amax/6/ts rounded to 3 mantissa
    bits (relative error at most 2^-4), and the error is at most half a grid step of at most
    2 * s * ts, or the saturation distance past 6 * s * ts, both below s * ts <= (amax/6) *
    (1 + 2^-4).  A row or group written to the wrong place would be off by O(1)."""
    from helpers import decode_pages_f64

    rng = np.random.default_rng(41 + (layout == "dim_major"))
    ts = float(np.float32(8 / (6 * 448)))
    n, num_pages, heads = 200, 3, 4
    x = rng.standard_normal((n, heads, 128)).astype(np.float32)
    slots = rng.choice(num_pages * 128, size=n, replace=False)
    dm = layout == "dim_major"
    cache = oracle.OracleCache(oracle.NVFP4, oracle.DIM_MAJOR if dm else oracle.TOKEN_MAJOR, heads, num_pages, ts)
    cache.write(slots, x)
    vals = decode_pages_f64(cache.bytes, True, dm, heads, num_pages, ts)  # [page][head][tok][dim]
    got = vals[slots // 128, :, slots % 128, :]  # [n][heads][128]
    amax = np.abs(x.astype(np.float64)).reshape(n, heads, 8, 16).max(-1)
    bound = np.repeat(amax / 6 * (1 + 2.0 ** -4), 16, axis=-1)
    err = np.abs(got - x)
    assert np.all(err <= bound * (1 + 1e-9))
    assert err.max() > 0.1 * bound.max()  # the values did go through the quantiser
    unused = np.setdiff1d(np.arange(num_pages * 128), slots)
    assert not vals[unused // 128, :, unused % 128, :].any()
