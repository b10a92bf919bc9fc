"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same
seeded inputs.

Bars (spec criteria, restated in each test):
  * cache bytes, FP8 query bytes and dequantised values: bit-exact;
  * selected block sets: identical wherever the oracle's (topk-1)-th and
    topk-th candidate scores differ by more than 1e-3 relative; inside that
    band the GPU set must be a valid top set of the band (tests/helpers.py);
  * attention output: per (request, row, head) vector, max |o - o_ref| /
    max |o_ref| <= 2e-3;
  * index scores (no bar is stated; derived): |s - s_ref| <= 2e-4 *
    sum_k |q_k K_k|.  The matrix-core FP8 x FP4 product accumulates its 16
    products with fewer than FP32's bits (measured on gfx950 at up to
    8e-5 of the sum of |terms| for wide exponent ranges); the E4M3 scales
    and FP32 sums add about 1e-7.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workload as W
from helpers import (decode_pages_f64, oracle_batch, oracle_caches, oracle_queries, row_positions,
                     selection_guard_ok)

pytestmark = pytest.mark.gpu

SCORE_TOL = 2e-4
OUT_TOL = 2e-3


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_attention_index_amd as M

    return M


def _dev(x, dt=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return t if dt is None else t.to(dt)


def gpu_setup(M, wl, hold_new=False, shared=True, owner=False):
    """Device caches holding the workload's rows.  hold_new: leave out each request's
    last R positions (the step's new tokens) and return their rows, request-major
    [B*R], as a fourth value (k, v, idx, slots); rows of positions below 0 are zero
    with slot -1 (no token).  shared: declare the workload's shared prefix pages in
    the batch (the indexer then scores them once for all requests).  owner: the
    batch carries the owner map msa_page_owner builds (physical-order scan)."""
    from block_sparse_attention_index_amd.decoder import MsaDecoder, make_caches

    dtype = {"nvfp4": M.MSA_NVFP4, "fp8": M.MSA_FP8_E4M3, "f32": M.MSA_F32}[wl.cache]
    k, v, idx = make_caches(dtype, wl.num_pages, wl.tensor_scale)
    batch = M.Batch(_dev(wl.block_table), _dev(wl.lengths), wl.R, wl.prefix_pages if shared else 0)
    if owner:
        own = M.msa_page_owner(batch, wl.num_pages)
        batch = M.Batch(batch.block_table, batch.ctx_lens, wl.R, batch.struct.shared_prefix_pages, page_owner=own)
    dec = MsaDecoder(batch, k, v, idx, wl.topk)
    n_new = wl.B * wl.R
    nk = np.zeros((n_new, 4, 128), np.float32)
    nv = np.zeros((n_new, 4, 128), np.float32)
    ni = np.zeros((n_new, 128), np.float32)
    nslots = np.full(n_new, -1, np.int64)
    # one request at a time, so that full-size caches never sit in host memory at once
    if wl.prefix_tokens:
        pos = np.arange(wl.prefix_tokens, dtype=np.int64)
        xi, xk, xv = W.prefix_rows(wl)
        dec.insert(_dev(xk), _dev(xv), _dev(xi), _dev(wl.slots(0, pos)))
    for b in range(wl.B):
        pos = wl.own_positions(b)
        if pos.shape[0]:
            xi, xk, xv = W.request_rows(wl, b)
            keep = pos < int(wl.lengths[b]) - wl.R if hold_new else np.ones(pos.shape[0], bool)
            if keep.any():
                dec.insert(_dev(xk[keep]), _dev(xv[keep]), _dev(xi[keep]), _dev(wl.slots(b, pos[keep])))
            if hold_new:
                for r in range(wl.R):
                    p_ = int(wl.lengths[b]) - wl.R + r
                    if p_ >= wl.prefix_tokens:
                        j = p_ - wl.prefix_tokens
                        nk[b * wl.R + r], nv[b * wl.R + r], ni[b * wl.R + r] = xk[j], xv[j], xi[j]
                        nslots[b * wl.R + r] = wl.slots(b, np.array([p_]))[0]
        if wl.num_pages > 4096 and b % 8 == 7:
            print(f"  inserted requests 0..{b}", flush=True)
    qi32, q32 = W.queries(wl)
    if wl.cache != "f32":
        q_idx = M.msa_quantize_e4m3(_dev(qi32), wl.q_scale)
        q = M.msa_quantize_e4m3(_dev(q32), wl.q_scale)
    else:
        q_idx, q = _dev(qi32), _dev(q32)
    torch.cuda.synchronize()
    if hold_new:
        return dec, q_idx, q, (_dev(nk), _dev(nv), _dev(ni), _dev(nslots))
    return dec, q_idx, q


def _print_case(name, wl):
    print(f"[case] {name}: {wl.name} B={wl.B} R={wl.R} lens={wl.lengths.tolist()[:6]} pages={wl.num_pages}",
          flush=True)


CASES = {
    "cfg1_f32": lambda: W.make_workload(1, seed=0),
    "cfg2_small": lambda: W.make_workload(2, seed=1, B=3, len_div=16),
    "cfg3_small": lambda: W.make_workload(3, seed=2, B=4, len_div=48),
    "cfg4_small": lambda: W.make_workload(4, seed=3, B=3, len_div=64),
    "cfg5_small": lambda: W.make_workload(5, seed=4, B=4, len_div=64),
    "ragged": lambda: W.make_workload(3, seed=5, lengths=[1, 127, 128, 129, 2047, 2048, 2049, 5000], R=1),
    "ragged_r4": lambda: W.make_workload(4, seed=6, lengths=[0, 2, 3, 4, 131, 2051, 2052, 7000], R=4),
    "r3": lambda: W.make_workload(4, seed=7, B=2, len_div=64, R=3),
    # shared prefix of 32 pages (4,096 tokens); 70 requests x 4 groups = 280 index queries span
    # several query tiles of the prefix kernel, the last one partial
    "prefix_wide": lambda: W.make_workload(5, seed=9, B=70, len_div=64),
    # shared-prefix decode with the scan fused into the prefix launch (one row per request):
    # 70 requests (unpacked scan ids, two query tiles) and 32 requests (packed ids), both with
    # workgroups that run two scan chunk ids; contexts shorter than the prefix on the fused path
    "prefix_fused_wide": lambda: W.make_workload(5, seed=37, B=70, len_div=16),
    "prefix_fused_b32": lambda: W.make_workload(5, seed=38, B=32, len_div=32),
    "prefix_short_r1": lambda: W.make_workload(5, seed=39, len_div=64, R=1,
                                               lengths=[64 * n for n in (0, 1, 100, 4095, 4096, 4097, 4200, 4500)]),
    # 65 requests (unpacked scan ids) whose suffixes fit one chunk: fewer scan chunk ids (65) than
    # fused workgroups (128), so most workgroups run no chunk
    "prefix_fused_sparse_ids": lambda: W.make_workload(5, seed=40, len_div=8, R=1, lengths=[8 * 32868] * 65),
    # contexts shorter than, equal to and just past the shared prefix, two rows each
    "prefix_short": lambda: W.make_workload(5, seed=10, len_div=64, R=2,
                                            lengths=[64 * n for n in (0, 1, 100, 4095, 4096, 4097, 4200, 9000)]),
    # prefill chunks: many causal rows per request (the dense matrix-core indexer)
    "prefill_r512": lambda: W.make_workload(6, seed=15, lengths=[8192], R=512),
    "prefill_ragged": lambda: W.make_workload(6, seed=16, lengths=[3000, 5000, 200], R=300),
    # FP8 caches (E4M3 per element, FP32 tensor scale)
    "fp8_cfg3_small": lambda: W.make_workload(3, seed=11, B=4, len_div=48, cache="fp8"),
    "fp8_ragged": lambda: W.make_workload(3, seed=12, lengths=[1, 127, 128, 129, 2047, 2048, 2049, 5000], R=1,
                                          cache="fp8"),
    "fp8_ragged_r4": lambda: W.make_workload(4, seed=13, lengths=[0, 2, 3, 4, 131, 2051, 2052, 7000], R=4,
                                             cache="fp8"),
    "fp8_r8": lambda: W.make_workload(4, seed=14, B=2, len_div=64, R=8, cache="fp8"),
    # prefill chunks in FP8 caches
    "fp8_prefill": lambda: W.make_workload(6, seed=17, lengths=[3000, 1000, 130], R=300, cache="fp8"),
    "fp8_prefill_r512": lambda: W.make_workload(6, seed=20, lengths=[8192], R=512, cache="fp8"),
    "r8": lambda: W.make_workload(4, seed=8, B=2, len_div=64, R=8),
    # batches whose B*R*4 workgroup rows exceed the 256 CUs: attention walks row-group unions
    # (two query tiles for R=4, one for R=2) instead of one workgroup per row
    "union_r4": lambda: W.make_workload(4, seed=18, B=20, len_div=64, R=4),
    "union_r2": lambda: W.make_workload(4, seed=19, B=40, len_div=128, R=2),
    # more than 64 requests: the scan's grid is not packed to the contexts (the per-lane map covers 64)
    "many_reqs": lambda: W.make_workload(3, seed=21, B=80, len_div=256),
    "fp8_many_reqs": lambda: W.make_workload(3, seed=22, B=80, len_div=256, cache="fp8"),
    # 5, 6 and 7 rows: the index scan's second FP16 query tile is partial (40, 48, 56 of 64 index
    # queries), and attention's two-tile row groups end with a partial group
    # (r6 and fp8_r6: 11 x 6 x 4 = 264 workgroup rows, so attention takes row groups of 4 + 2 rows;
    # r5, r7: one workgroup per row)
    "r5": lambda: W.make_workload(4, seed=23, B=2, len_div=64, R=5),
    "r6": lambda: W.make_workload(4, seed=24, B=11, len_div=64, R=6),
    "r7": lambda: W.make_workload(4, seed=25, lengths=[3, 900, 6000], R=7),
    "union_r7": lambda: W.make_workload(4, seed=36, B=10, len_div=64, R=7),
    "fp8_r5": lambda: W.make_workload(4, seed=26, B=2, len_div=64, R=5, cache="fp8"),
    "fp8_r6": lambda: W.make_workload(4, seed=27, B=11, len_div=64, R=6, cache="fp8"),
    "fp8_r7": lambda: W.make_workload(4, seed=28, lengths=[3, 900, 6000], R=7, cache="fp8"),
    # 3 rows on the row-group union path: 24 x 3 x 4 = 288 workgroup rows exceed the 256 CUs
    "union_r3": lambda: W.make_workload(4, seed=29, B=24, len_div=32, R=3),
    # other selection sizes through the index scan, the fused selection and attention
    "topk8": lambda: W.make_workload(3, seed=30, B=4, len_div=24, topk=8),
    "topk32": lambda: W.make_workload(3, seed=31, B=4, len_div=12, topk=32),
    "topk32_r4": lambda: W.make_workload(4, seed=32, B=3, len_div=24, R=4, topk=32),
    # the largest and smallest selections: 64 blocks (the whole union when a context has at most 64)
    # and the latest block alone
    "topk64": lambda: W.make_workload(3, seed=41, B=4, len_div=6, topk=64),
    "topk1": lambda: W.make_workload(3, seed=42, B=4, len_div=48, topk=1),
    "fp8_topk8": lambda: W.make_workload(3, seed=33, B=3, len_div=24, topk=8, cache="fp8"),
    # a block table wider than 3,072 entries (short contexts): the selection reads its scores from
    # memory on demand and attention reads the table row from memory instead of LDS
    "wide_table": lambda: W.make_workload(3, seed=34, B=3, len_div=32, table_width=3100),
    "wide_table_r4": lambda: W.make_workload(4, seed=35, B=2, len_div=32, R=4, table_width=3100),
    # pools with pages no request uses, scattered among the used ones (the physical-order scan
    # reads them and drops them)
    "spare_pool": lambda: W.make_workload(3, seed=43, B=6, len_div=40, spare_pages=333),
    "spare_pool_r4": lambda: W.make_workload(4, seed=44, lengths=[0, 1, 4, 127, 128, 131, 2052, 5000], R=4,
                                             spare_pages=77),
    # two rows: new rows on one page, across a page boundary (129: positions 127 and 128), and
    # contexts shorter than the rows
    "prefill_topk64": lambda: W.make_workload(6, seed=48, lengths=[9000, 3000], R=200, topk=64),
    "prefill_topk1": lambda: W.make_workload(6, seed=49, lengths=[5000, 140], R=150, topk=1),
    "prefill_wide_table": lambda: W.make_workload(6, seed=50, lengths=[4000, 2000], R=100, table_width=8300),
    "fp8_spare_pool": lambda: W.make_workload(3, seed=46, B=5, len_div=40, spare_pages=211, cache="fp8"),
    "fp8_spare_pool_r3": lambda: W.make_workload(4, seed=47, lengths=[0, 2, 3, 127, 128, 130, 2051, 4000], R=3,
                                                 spare_pages=97, cache="fp8"),
    "ragged_r2": lambda: W.make_workload(4, seed=45, lengths=[0, 1, 2, 128, 129, 130, 2049, 5000], R=2,
                                         spare_pages=19),
    # more workgroup rows than half the 256 CUs, at most all of them: one workgroup per row, whose
    # waves take two blocks each; 144-256 rows, with 8, 48 and from-memory candidate counts per
    # lane, and FP8 caches
    "cus_b48": lambda: W.make_workload(3, seed=51, B=48, len_div=48),
    "cus_r4": lambda: W.make_workload(4, seed=52, B=16, len_div=32, R=4),
    "cus_ragged": lambda: W.make_workload(3, seed=53, lengths=[1, 127, 128, 129, 2047, 2048, 2049, 5000] * 5, R=1),
    "cus_wide": lambda: W.make_workload(3, seed=54, B=36, len_div=32, table_width=1600),
    "cus_wide_mem": lambda: W.make_workload(3, seed=55, B=36, len_div=32, table_width=3100),
    "fp8_cus": lambda: W.make_workload(3, seed=56, B=40, len_div=48, cache="fp8"),
    "fp8_cus_wide": lambda: W.make_workload(3, seed=57, B=36, len_div=32, table_width=1600, cache="fp8"),
    # the same batch shape with 32 blocks per row (four per wave) and with 8
    "cus_topk32": lambda: W.make_workload(3, seed=58, B=48, len_div=24, topk=32),
    "cus_topk8": lambda: W.make_workload(3, seed=59, B=48, len_div=48, topk=8),
}

CUS_CASES = ["cus_b48", "cus_r4", "cus_ragged", "cus_wide", "cus_wide_mem", "fp8_cus", "fp8_cus_wide",
             "cus_topk32", "cus_topk8"]


# ---------------------------------------------------------------- step 0 / codecs
@pytest.mark.parametrize("case", ["cfg2_small", "cfg4_small", "cfg5_small", "cfg1_f32", "fp8_cfg3_small"])
def test_insert_bytes_bitexact(M, oracle, case):
    wl = CASES[case]()
    _print_case(case, wl)
    dec, _, _ = gpu_setup(M, wl)
    ci, ck, cv = oracle_caches(oracle, wl)
    assert np.array_equal(dec.idx.pages.cpu().numpy(), ci.bytes)
    assert np.array_equal(dec.k.pages.cpu().numpy(), ck.bytes)
    assert np.array_equal(dec.v.pages.cpu().numpy(), cv.bytes)


@pytest.mark.parametrize("n,consecutive", [(300, False), (512, False), (1030, True)])
def test_insert_special_values_bitexact(M, oracle, n, consecutive):
    """Groups spanning subnormal scales, saturation, exact zeros, -0 and E2M1 ties.  Below 512
    tokens the insert quantises on a 16-lane row per group, from 512 on with one lane per group;
    consecutive slots (a prompt chunk) write value bytes of token pairs whole."""
    print(f"[case] insert special values n={n} consecutive={consecutive}", flush=True)
    rng = np.random.default_rng(11 + n)
    x = rng.standard_normal((n, 4, 128)).astype(np.float32)
    x *= (2.0 ** rng.integers(-24, 14, size=(n, 4, 8, 1))).repeat(16, -1).reshape(n, 4, 128).astype(np.float32)
    x[::7, :, :16] = 0.0
    x[1::7, :, 16:32] = -0.0
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], np.float32)
    x[2::7, :, 32:48] = np.tile(np.concatenate([ties, -ties]), 1)  # amax 6 -> scale = E4M3(1/ts)
    xi = x[:, 0, :].copy()
    ts = float(np.float32(1.0))
    from block_sparse_attention_index_amd.decoder import make_caches

    npg = n // 128 + 1
    k, v, idx = make_caches(True, npg, ts)
    slots = (np.arange(n) + 3) if consecutive else rng.permutation(npg * 128)[:n]
    slots = slots.astype(np.int64)
    M.msa_kv_insert(_dev(x), _dev(x), _dev(xi), _dev(slots), k, v, idx)
    torch.cuda.synchronize()
    ok = O.OracleCache(O.NVFP4, O.TOKEN_MAJOR, 4, npg, ts)
    ov = O.OracleCache(O.NVFP4, O.DIM_MAJOR, 4, npg, ts)
    oi = O.OracleCache(O.NVFP4, O.TOKEN_MAJOR, 1, npg, ts)
    ok.write(slots, x), ov.write(slots, x), oi.write(slots, xi)
    assert np.array_equal(k.pages.cpu().numpy(), ok.bytes)
    assert np.array_equal(v.pages.cpu().numpy(), ov.bytes)
    assert np.array_equal(idx.pages.cpu().numpy(), oi.bytes)


def test_insert_fp8_special_values_bitexact(M, oracle):
    """FP8 cache bytes: E4M3(x / ts) over subnormals, exact midpoints, saturation, zeros, -0 and NaN."""
    print("[case] insert fp8 special values", flush=True)
    rng = np.random.default_rng(12)
    n = 384
    ts = 0.25
    vals = O.e4m3_value(np.arange(127))
    mids = (vals[:-1] + vals[1:]) / 2
    pool = np.concatenate([vals, mids, [449.0, 464.0, 500.0, 1e6, 0.0, -0.0, np.nan, 2.0 ** -10]]) * ts
    x = rng.choice(np.concatenate([pool, -pool]), size=(n, 4, 128)).astype(np.float32)
    x[: n // 2] = (rng.standard_normal((n // 2, 4, 128)) * 2.0 ** rng.integers(-12, 9, (n // 2, 4, 1))).astype(
        np.float32)
    xi = x[:, 1, :].copy()
    from block_sparse_attention_index_amd.decoder import make_caches

    npg = n // 128 + 1
    k, v, idx = make_caches(M.MSA_FP8_E4M3, npg, ts)
    slots = rng.permutation(npg * 128)[:n].astype(np.int64)
    M.msa_kv_insert(_dev(x), _dev(x), _dev(xi), _dev(slots), k, v, idx)
    torch.cuda.synchronize()
    ok = O.OracleCache(O.FP8_E4M3, O.TOKEN_MAJOR, 4, npg, ts)
    ov = O.OracleCache(O.FP8_E4M3, O.DIM_MAJOR, 4, npg, ts)
    oi = O.OracleCache(O.FP8_E4M3, O.HALF_ROWS, 1, npg, ts)
    ok.write(slots, x), ov.write(slots, x), oi.write(slots, xi)
    assert np.array_equal(k.pages.cpu().numpy(), ok.bytes)
    assert np.array_equal(v.pages.cpu().numpy(), ov.bytes)
    assert np.array_equal(idx.pages.cpu().numpy(), oi.bytes)


@pytest.mark.parametrize("layout", ["token_major", "dim_major", "half_rows"])
def test_debug_dequant_fp8_all_codes(M, oracle, layout):
    """Every E4M3 byte in the three FP8 slab layouts, bit-exact against the oracle (NaN codes give NaN)."""
    print(f"[case] fp8 dequant {layout}", flush=True)
    npg = 2
    raw = (np.arange(npg * 16384) * 7 % 256).astype(np.uint8)
    lay = {"token_major": (M.MSA_TOKEN_MAJOR, O.TOKEN_MAJOR), "dim_major": (M.MSA_DIM_MAJOR, O.DIM_MAJOR),
           "half_rows": (M.MSA_HALF_ROWS, O.HALF_ROWS)}[layout]
    c = M.Cache(_dev(raw), M.MSA_FP8_E4M3, lay[0], 1, npg, 0.3)
    oc = O.OracleCache(O.FP8_E4M3, lay[1], 1, npg, 0.3)
    oc.bytes[:] = raw
    want = oc.dequant_pages(np.arange(npg))
    for mode in (0, 1):
        out = torch.empty((npg, 1, 128, 128), dtype=torch.float32, device="cuda")
        M.msa_debug_dequant(c, _dev(np.arange(npg, dtype=np.int32)), mode, out)
        got = out.cpu().numpy()
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], want[~nan])


def test_quantize_e4m3_bitexact(M, oracle):
    print("[case] e4m3 query quantiser", flush=True)
    vals = O.e4m3_value(np.arange(127))
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(3)
    x = np.concatenate([vals, mids, rng.standard_normal(20000) * 4, np.exp(rng.uniform(-18, 7, 5000)),
                        [448, 463.9, 464, 464.1, 500, 1e30, np.inf, 0.0, -0.0, 2.0 ** -10, 2.0 ** -11 * 3]])
    x = np.concatenate([x, -x]).astype(np.float32)
    for scale in (1.0, 0.37):
        got = M.msa_quantize_e4m3(_dev(x), scale).cpu().numpy()
        want = O.quantize_queries(x, scale)
        assert np.array_equal(got, want), scale
    xn = np.array([np.nan], np.float32)
    assert M.msa_quantize_e4m3(_dev(xn), 1.0).cpu().numpy()[0] & 0x7F == 0x7F


@pytest.mark.parametrize("layout", ["token_major", "dim_major"])
@pytest.mark.parametrize("mode", [0, 1])
def test_debug_dequant_exhaustive(M, oracle, layout, mode):
    """Every E4M3 scale code against every E2M1 code, bit-exact (NaN scales give NaN)."""
    print(f"[case] dequant {layout} mode {mode}", flush=True)
    rng = np.random.default_rng(1)
    npg = 4
    raw = rng.integers(0, 256, size=npg * 9216, dtype=np.uint8)
    slabs = raw.reshape(npg, 9216)
    # scales: page p uses codes (p*1024 + i) % 256 -> all 256 codes appear in every page
    slabs[:, 8192:] = (np.arange(npg * 1024).reshape(npg, 1024) % 256).astype(np.uint8)
    # codes: row (token or dim) x, element e holds nibble (x + e) % 16, so every 16-element
    # group holds all 16 E2M1 codes, each next to every scale code over the pages
    rr, ii = np.meshgrid(np.arange(128), np.arange(64), indexing="ij")
    codes = ((2 * ii + rr) % 16) | (((2 * ii + 1 + rr) % 16) << 4)
    slabs[:, :8192] = codes.reshape(-1).astype(np.uint8)[None, :]
    dm = layout == "dim_major"
    dev_pages = _dev(raw)
    c = M.Cache(dev_pages, M.MSA_NVFP4, M.MSA_DIM_MAJOR if dm else M.MSA_TOKEN_MAJOR, 1, npg, 0.3)
    out = torch.empty((npg, 1, 128, 128), dtype=torch.float32, device="cuda")
    M.msa_debug_dequant(c, _dev(np.arange(npg, dtype=np.int32)), mode, out)
    got = out.cpu().numpy()
    oc = O.OracleCache(O.NVFP4, O.DIM_MAJOR if dm else O.TOKEN_MAJOR, 1, npg, 0.3)
    oc.bytes[:] = raw
    want = oc.dequant_pages(np.arange(npg))
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    exact = decode_pages_f64(raw, True, dm, 1, npg, 0.3)
    assert np.array_equal(np.isnan(exact), nan)


# ---------------------------------------------------------------- steps 1+2
@pytest.mark.parametrize("case", ["cfg1_f32", "cfg2_small", "cfg3_small", "cfg4_small", "cfg5_small", "ragged",
                                  "ragged_r4", "r3", "r8", "prefix_wide", "prefix_short", "fp8_cfg3_small",
                                  "fp8_ragged", "fp8_ragged_r4", "fp8_r8", "prefill_r512", "prefill_ragged",
                                  "fp8_prefill", "fp8_prefill_r512", "many_reqs", "fp8_many_reqs", "r5", "r6", "r7",
                                  "fp8_r5", "fp8_r6", "fp8_r7", "union_r3", "wide_table", "wide_table_r4",
                                  "prefix_fused_wide", "prefix_fused_b32", "prefix_short_r1",
                                  "prefix_fused_sparse_ids"])
def test_index_scores(M, oracle, case):
    wl = CASES[case]()
    _print_case(case, wl)
    dec, q_idx, _ = gpu_setup(M, wl)
    T = wl.max_pages * 128
    tok = torch.empty((wl.B, wl.R, 4, T), dtype=torch.float32, device="cuda")
    dec.index(q_idx, wl.q_scale, tok)
    got_tok = tok.cpu().numpy().astype(np.float64)
    got_blk = dec.block_scores.cpu().numpy().astype(np.float64)
    ci, _, _ = oracle_caches(oracle, wl)
    _, _, qi, _ = oracle_queries(oracle, wl)
    bt = oracle_batch(oracle, wl)
    ref_tok, ref_abs = oracle.index_scores(bt, qi, ci, with_abs=True)
    ref_blk = oracle.block_maxpool(bt, ref_tok)
    inv = np.isneginf(ref_tok)
    assert np.array_equal(np.isneginf(got_tok), inv)
    err = np.abs(got_tok[~inv] - ref_tok[~inv])
    bound = SCORE_TOL * ref_abs[~inv] + 1e-30
    ratio = float((err / bound).max()) if err.size else 0.0
    print(f"  token score error / bound max = {ratio:.3f}; max err/sum|terms| = "
          f"{float((err / (ref_abs[~inv] + 1e-30)).max()) if err.size else 0:.2e}", flush=True)
    assert ratio <= 1.0
    # block scores are the max-pool of the token scores
    binv = np.isneginf(ref_blk)
    assert np.array_equal(np.isneginf(got_blk), binv)
    pooled = got_tok.reshape(got_tok.shape[:3] + (wl.max_pages, 128)).max(-1)
    assert np.array_equal(got_blk, pooled)
    # same kernel without the token-score output (which packs its grid to the contexts and
    # writes the -inf of the pages past them separately): every entry must be rewritten
    dec.block_scores.fill_(3.0)
    dec.index(q_idx, wl.q_scale, None)
    assert np.array_equal(dec.block_scores.cpu().numpy().astype(np.float64), got_blk)


@pytest.mark.parametrize("case", ["prefix_wide", "prefill_ragged", "cfg4_small", "fp8_cfg3_small"])
def test_nan_index_query(M, oracle, case):
    """An index query holding a NaN (the E4M3 NaN byte 0x7F in one dim) scores NaN on every token,
    and the max-pool skips NaN on both sides, so its blocks score -inf; the other queries are
    untouched.  Through the shared-prefix indexer (matrix cores, FP16), the prefill indexer, the
    FP16 multi-row scan and the FP8 scan; the selection of the NaN rows is then the tie rule's:
    the latest block and the lowest others."""
    wl = CASES[case]()
    _print_case(f"nan index query {case}", wl)
    dec, q_idx, _ = gpu_setup(M, wl)
    bi = oracle.quantize_queries(W.queries(wl)[0], wl.q_scale)
    nan_rows = [(0, 0, 1), (wl.B - 1, wl.R - 1, 3)] + ([(1, wl.R // 2, 0)] if wl.B > 1 else [])
    for (b, r, g) in nan_rows:
        bi[b, r, g, 5] = 0x7F
    q_idx.copy_(_dev(bi))
    T = wl.max_pages * 128
    tok = torch.empty((wl.B, wl.R, 4, T), dtype=torch.float32, device="cuda")
    dec.index(q_idx, wl.q_scale, tok)
    dec.select()
    torch.cuda.synchronize()
    got_tok = tok.cpu().numpy().astype(np.float64)
    got_blk = dec.block_scores.cpu().numpy().astype(np.float64)
    ci, _, _ = oracle_caches(oracle, wl)
    bt = oracle_batch(oracle, wl)
    qi = oracle.decode_queries(bi, oracle.FP8_E4M3, wl.q_scale)
    ref_tok, ref_abs = oracle.index_scores(bt, qi, ci, with_abs=True)
    ref_blk = oracle.block_maxpool(bt, ref_tok)
    nan = np.isnan(ref_tok)
    assert nan.any()
    assert np.array_equal(np.isnan(got_tok), nan)
    inv = np.isneginf(ref_tok)
    assert np.array_equal(np.isneginf(got_tok), inv)
    ok = ~nan & ~inv
    assert (np.abs(got_tok[ok] - ref_tok[ok]) <= SCORE_TOL * ref_abs[ok] + 1e-30).all()
    binv = np.isneginf(ref_blk)
    for (b, r, g) in nan_rows:
        assert binv[b, r, g].all()
    assert np.array_equal(np.isneginf(got_blk), binv)
    fin = ~binv
    pooled = np.where(np.isnan(got_tok), -np.inf, got_tok).reshape(got_tok.shape[:3] + (wl.max_pages, 128)).max(-1)
    assert np.array_equal(got_blk[fin], pooled[fin])
    rs, rc = oracle.select(bt, ref_blk, wl.topk)
    g_sel, g_cnt = dec.sel.cpu().numpy(), dec.cnt.cpu().numpy()
    for (b, r, g) in nan_rows:
        assert g_cnt[b, r, g] == rc[b, r, g] and np.array_equal(g_sel[b, r, g], rs[b, r, g])


# ---------------------------------------------------------------- step 3
@pytest.mark.parametrize("topk,P", [(1, 300), (4, 300), (16, 300), (64, 300), (16, 1400), (16, 2500), (16, 4000)])
def test_topk_exact_on_shared_scores(M, oracle, topk, P):
    """Same FP32 scores on both sides: the selection must be identical, ties and NaN included.
    P covers each register-capacity variant of the kernel and the rescan-from-memory one."""
    print(f"[case] topk={topk} P={P}", flush=True)
    rng = np.random.default_rng(topk + P)
    B, R = 6, 2
    lens = np.array([0, 1, 128, 129, P * 128, 20000], np.int32)
    table = np.zeros((B, P), np.int32)
    scores = rng.integers(-4, 5, size=(B, R, 4, P)).astype(np.float32)
    scores[4, 0, 1, :40] = rng.standard_normal(40).astype(np.float32)
    scores[4, 1, 2, :8] = [-0.0, 0.0, -0.0, 0.0, np.nan, np.nan, -np.inf, np.inf]
    scores[5, 1, 3, 100:150] = np.nan
    batch = M.Batch(_dev(table), _dev(lens), R)
    sel = torch.empty((B, R, 4, topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, R, 4), dtype=torch.int32, device="cuda")
    M.msa_block_maxpool_topk(batch, _dev(scores), 0, topk, sel, cnt)
    bt = oracle.OracleBatch(table, lens, R)
    rs, rc = oracle.select(bt, scores.astype(np.float64), topk)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(sel.cpu().numpy(), rs)
    # token-level route: max-pool first
    tok = np.repeat(scores, 128, axis=-1) - rng.integers(0, 3, size=(B, R, 4, P * 128)).astype(np.float32)
    M.msa_block_maxpool_topk(batch, _dev(tok), 1, topk, sel, cnt)
    rs2, rc2 = oracle.select(bt, oracle.block_maxpool(bt, tok.astype(np.float64)), topk)
    assert np.array_equal(cnt.cpu().numpy(), rc2)
    assert np.array_equal(sel.cpu().numpy(), rs2)


@pytest.mark.parametrize("topk,P", [(16, 300), (16, 1400), (16, 2500), (16, 4000), (64, 300), (64, 1400)])
def test_topk_lane_periodic_scores(M, oracle, topk, P):
    """Scores that depend only on the block index modulo 64 (one register lane of the
    selection), so whole lanes tie: every key of the best lanes is a candidate, which
    fills the candidate buffer and, past its capacity, takes the round-based path."""
    print(f"[case] lane-periodic topk={topk} P={P}", flush=True)
    B, R = 3, 1
    lens = np.array([P * 128, P * 128 - 77, 64 * 128 * 3 + 5], np.int32)
    table = np.zeros((B, P), np.int32)
    j = np.arange(P)
    base = (100.0 - (j % 64)).astype(np.float32)
    scores = np.broadcast_to(base, (B, R, 4, P)).copy()
    scores[1] = np.broadcast_to((j % 64).astype(np.float32), (R, 4, P))  # increasing with the lane
    scores[2, 0, 1] = np.float32(1.0)  # all equal: the lowest block indices win
    batch = M.Batch(_dev(table), _dev(lens), R)
    sel = torch.empty((B, R, 4, topk), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, R, 4), dtype=torch.int32, device="cuda")
    M.msa_block_maxpool_topk(batch, _dev(scores), 0, topk, sel, cnt)
    bt = oracle.OracleBatch(table, lens, R)
    rs, rc = oracle.select(bt, scores.astype(np.float64), topk)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    assert np.array_equal(sel.cpu().numpy(), rs)


# ---------------------------------------------------------------- step 4
def _out_err(got, ref):
    return np.abs(got - ref).max(-1) / np.maximum(np.abs(ref).max(-1), 1e-30)


@pytest.mark.parametrize("case", ["cfg1_f32", "cfg2_small", "cfg3_small", "cfg4_small", "cfg5_small",
                                  "ragged", "ragged_r4", "r3", "r8", "fp8_cfg3_small", "fp8_ragged_r4", "fp8_r8",
                                  "prefill_ragged", "fp8_prefill", "r5", "r7", "fp8_r6", "union_r3", "topk8",
                                  "topk32", "topk32_r4", "fp8_topk8", "wide_table"] + CUS_CASES)
def test_sparse_decode_on_oracle_selection(M, oracle, case):
    wl = CASES[case]()
    _print_case(case, wl)
    dec, q_idx, q = gpu_setup(M, wl)
    ci, ck, cv = oracle_caches(oracle, wl)
    _, _, qi, qd = oracle_queries(oracle, wl)
    bt = oracle_batch(oracle, wl)
    sel, cnt = oracle.select(bt, oracle.block_maxpool(bt, oracle.index_scores(bt, qi, ci)), wl.topk)
    dec.sel.copy_(_dev(sel))
    dec.cnt.copy_(_dev(cnt))
    dec.attend(q, wl.q_scale, wl.sm_scale)
    got = dec.out.cpu().numpy().astype(np.float64)
    ref = oracle.attention(bt, qd, wl.sm_scale, ck, cv, sel, cnt)
    err = _out_err(got, ref)
    empty = np.repeat(cnt == 0, 8, axis=2)
    assert (got[empty] == 0).all()
    print(f"  max per-vector relative error {err[~empty].max() if (~empty).any() else 0:.3e}", flush=True)
    assert err[~empty].max(initial=0.0) <= OUT_TOL


# ---------------------------------------------------------------- whole step
def _check_full_step(M, oracle, wl, sample=None, fused=True, new_rows=False, owner=False, workspace=True):
    """workspace=False (fused only): msa_select_decode without a workspace (no split rows, and
    prefill chunks in the per-row form instead of the block-major one)."""
    if new_rows:  # the step itself inserts each request's last R rows
        dec, q_idx, q, new = gpu_setup(M, wl, hold_new=True, owner=owner)
        if not workspace:
            dec.workspace = None
        dec.step(q_idx, q, wl.q_scale, wl.sm_scale, new_tokens=new, fused=fused)
    else:
        dec, q_idx, q = gpu_setup(M, wl, owner=owner)
        if not workspace:
            dec.workspace = None
        dec.step(q_idx, q, wl.q_scale, wl.sm_scale, fused=fused)
    torch.cuda.synchronize()
    g_sel, g_cnt = dec.sel.cpu().numpy(), dec.cnt.cpu().numpy()
    g_out = dec.out.cpu().numpy().astype(np.float64)
    g_bs = dec.block_scores.cpu().numpy().astype(np.float64)
    rows = np.arange(wl.B) if sample is None else np.asarray(sample)
    ci, ck, cv = oracle_caches(oracle, wl) if sample is None else _sampled_caches(oracle, wl, rows)
    _, _, qi, qd = oracle_queries(oracle, wl)
    bt = oracle.OracleBatch(wl.block_table[rows], wl.lengths[rows], wl.R)
    # the oracle's steps 1-4 in order (its decode_step), the index scores taken once with their
    # sums of |terms| for the score bound
    ts, ab = oracle.index_scores(bt, qi[rows], ci, with_abs=True)
    res = {"block_scores": oracle.block_maxpool(bt, ts)}
    res["sel"], res["cnt"] = oracle.select(bt, res["block_scores"], wl.topk)
    res["out"] = oracle.attention(bt, qd[rows], wl.sm_scale, ck, cv, res["sel"], res["cnt"])
    # block scores (max-pooled) against the oracle's, with the derived bound
    absmax = ab.reshape(ab.shape[:3] + (wl.max_pages, 128)).max(-1)
    fin = np.isfinite(res["block_scores"])
    assert np.array_equal(np.isfinite(g_bs[rows]), fin)
    assert (np.abs(g_bs[rows][fin] - res["block_scores"][fin]) <= SCORE_TOL * absmax[fin] + 1e-30).all()
    p = row_positions(wl)[rows]
    guarded = mism = 0
    for bi_, b in enumerate(rows):
        for r in range(wl.R):
            for g in range(4):
                ok, gd = selection_guard_ok(res["block_scores"][bi_, r, g], res["sel"][bi_, r, g],
                                            res["cnt"][bi_, r, g], g_sel[b, r, g], g_cnt[b, r, g], p[bi_, r],
                                            wl.topk)
                guarded += gd
                mism += not ok
    print(f"  selections: {rows.size * wl.R * 4} compared, {guarded} inside the 1e-3 guard band, "
          f"{mism} invalid", flush=True)
    assert mism == 0
    # outputs: against oracle attention on the GPU's (validated) selection, and on the oracle's where equal
    same = np.array([[[set(g_sel[b, r, g, :g_cnt[b, r, g]]) == set(res["sel"][i, r, g, :res["cnt"][i, r, g]])
                       for g in range(4)] for r in range(wl.R)] for i, b in enumerate(rows)])
    same_h = np.repeat(same, 8, axis=2)
    # (where every set is the oracle's, the oracle's output on its own selection is that reference)
    ref_own = res["out"] if same.all() else oracle.attention(bt, qd[rows], wl.sm_scale, ck, cv, g_sel[rows],
                                                               g_cnt[rows])
    err = _out_err(g_out[rows], ref_own)
    print(f"  max per-vector relative error {err.max():.3e}", flush=True)
    assert err.max() <= OUT_TOL
    err2 = _out_err(g_out[rows], res["out"])
    assert err2[same_h].max(initial=0.0) <= OUT_TOL
    return dec


def _sampled_caches(oracle, wl, rows):
    """Oracle caches holding only the pages of the sampled requests (and the shared prefix)."""
    dt = {"f32": oracle.F32, "nvfp4": oracle.NVFP4, "fp8": oracle.FP8_E4M3}[wl.cache]
    ci = oracle.OracleCache(dt, oracle.TOKEN_MAJOR, 1, wl.num_pages, wl.tensor_scale)
    ck = oracle.OracleCache(dt, oracle.TOKEN_MAJOR, 4, wl.num_pages, wl.tensor_scale)
    cv = oracle.OracleCache(dt, oracle.TOKEN_MAJOR if dt == oracle.F32 else oracle.DIM_MAJOR, 4, wl.num_pages,
                            wl.tensor_scale)
    if wl.prefix_tokens:
        pos = np.arange(wl.prefix_tokens, dtype=np.int64)
        xi, xk, xv = W.prefix_rows(wl)
        s = wl.slots(0, pos)
        ci.write(s, xi), ck.write(s, xk), cv.write(s, xv)
    for b in rows:
        pos = wl.own_positions(b)
        xi, xk, xv = W.request_rows(wl, b)
        s = wl.slots(b, pos)
        ci.write(s, xi), ck.write(s, xk), cv.write(s, xv)
    return ci, ck, cv


FULL_STEP_CASES = ["cfg1_f32", "cfg2_small", "cfg3_small", "cfg4_small", "cfg5_small", "ragged", "ragged_r4", "r3",
                   "r8", "prefix_wide", "prefix_short", "fp8_cfg3_small", "fp8_ragged", "fp8_ragged_r4", "fp8_r8",
                   "union_r4", "union_r2", "r5", "r6", "r7", "fp8_r5", "fp8_r6", "fp8_r7", "union_r3", "union_r7",
                   "topk8", "topk32", "topk32_r4", "fp8_topk8", "wide_table", "wide_table_r4", "topk64", "topk1"]
# Prefill chunks given a workspace run the same kernels fused or not (the top-k launch, then the
# block-major route), and the wide-batch cases' separate route is covered on the oracle's
# selection: both run fused only.
FUSED_ONLY_CASES = ["prefill_r512", "prefill_ragged", "fp8_prefill", "fp8_prefill_r512"] + CUS_CASES


@pytest.mark.parametrize("case,fused", [(c, f) for c in FULL_STEP_CASES for f in (True, False)]
                         + [(c, True) for c in FUSED_ONLY_CASES])
def test_full_step(M, oracle, case, fused):
    """Steps 0-4 (insert, index, selection, attention); fused = selection and attention in one launch."""
    wl = CASES[case]()
    _print_case(f"{case} fused={fused}", wl)
    _check_full_step(M, oracle, wl, fused=fused)


@pytest.mark.parametrize("case", ["cfg2_small", "cfg3_small", "cfg4_small", "cfg5_small", "ragged", "ragged_r4", "r8",
                                  "prefix_wide", "fp8_cfg3_small", "fp8_ragged", "fp8_ragged_r4", "fp8_r8", "r5",
                                  "r6", "r7", "fp8_r5", "fp8_r7", "union_r3", "topk32", "prefix_fused_b32",
                                  "cus_r4", "cus_ragged", "fp8_cus"])
@pytest.mark.parametrize("fused", [True, False])
def test_full_step_with_new_rows(M, oracle, case, fused):
    """The step inserts each request's R new rows itself (fused: insert + index in one
    launch), then indexes, selects and attends; checked against the oracle on all rows."""
    wl = CASES[case]()
    _print_case(f"{case} new rows fused={fused}", wl)
    _check_full_step(M, oracle, wl, fused=fused, new_rows=True)


@pytest.mark.parametrize("case", ["cfg3_small", "cfg4_small", "ragged", "ragged_r4", "r3", "r8", "many_reqs", "r5",
                                  "r6", "r7", "fp8_r7", "union_r3", "cfg5_small", "prefix_fused_wide",
                                  "prefix_fused_b32", "prefix_short_r1", "prefix_fused_sparse_ids"])
def test_insert_index_equals_separate_calls(M, oracle, case):
    """msa_insert_index_score: the caches bitwise as msa_kv_insert_nvfp4 writes them (and as
    the oracle writes them), and bitwise the block scores of msa_index_score after that insert."""
    wl = CASES[case]()
    _print_case(case, wl)
    dec_a, q_idx, _, (nk, nv, ni, ns) = gpu_setup(M, wl, hold_new=True)
    dec_b, _, _, _ = gpu_setup(M, wl, hold_new=True)
    dec_a.insert(nk, nv, ni, ns)
    dec_a.index(q_idx, wl.q_scale)
    dec_b.block_scores.fill_(3.0)
    dec_b.insert_index(nk, nv, ni, q_idx, wl.q_scale)
    torch.cuda.synchronize()
    ci, ck, cv = oracle_caches(oracle, wl)
    for ca, cb, co in ((dec_a.idx, dec_b.idx, ci), (dec_a.k, dec_b.k, ck), (dec_a.v, dec_b.v, cv)):
        assert torch.equal(ca.pages, cb.pages)
        assert np.array_equal(cb.pages.cpu().numpy(), co.bytes)
    assert torch.equal(dec_a.block_scores.view(torch.int32), dec_b.block_scores.view(torch.int32))


@pytest.mark.parametrize("case", ["cfg3_small", "cfg4_small", "ragged_r4", "r8", "union_r4", "union_r2", "r5", "r6",
                                  "r7", "fp8_r6", "union_r3", "union_r7", "topk8", "topk32", "topk32_r4",
                                  "fp8_topk8", "wide_table", "wide_table_r4", "topk64", "topk1"] + CUS_CASES)
def test_select_decode_equals_separate_calls(M, oracle, case):
    """msa_select_decode: same selection as msa_block_maxpool_topk and bitwise the same
    output as msa_sparse_decode on that selection."""
    wl = CASES[case]()
    _print_case(case, wl)
    dec, q_idx, q = gpu_setup(M, wl)
    dec.index(q_idx, wl.q_scale)
    dec.select()
    dec.attend(q, wl.q_scale, wl.sm_scale)
    sel_a, cnt_a, out_a = dec.sel.clone(), dec.cnt.clone(), dec.out.clone()
    dec.sel.fill_(-5), dec.cnt.fill_(-5), dec.out.fill_(7.0)
    dec.select_attend(q, wl.q_scale, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(dec.cnt, cnt_a) and torch.equal(dec.sel, sel_a)
    assert torch.equal(dec.out.view(torch.int32), out_a.view(torch.int32))


@pytest.mark.parametrize("case", ["prefill_ragged", "fp8_prefill"])
def test_prefill_select_decode_on_oracle_scores(M, oracle, case):
    """Prefill chunks (one row per workgroup): from the oracle's block scores rounded to FP32,
    the fused selection + attention equals msa_block_maxpool_topk + msa_sparse_decode bitwise,
    the selection equals the oracle's on the same FP32 scores, and the output matches the
    oracle's attention on it."""
    wl = CASES[case]()
    _print_case(case, wl)
    dec, q_idx, q = gpu_setup(M, wl)
    ci, ck, cv = oracle_caches(oracle, wl)
    _, _, qi, qd = oracle_queries(oracle, wl)
    bt = oracle_batch(oracle, wl)
    bs32 = oracle.block_maxpool(bt, oracle.index_scores(bt, qi, ci)).astype(np.float32)
    dec.block_scores.copy_(_dev(bs32))
    dec.select()
    dec.attend(q, wl.q_scale, wl.sm_scale)
    sel_a, cnt_a, out_a = dec.sel.clone(), dec.cnt.clone(), dec.out.clone()
    dec.sel.fill_(-5), dec.cnt.fill_(-5), dec.out.fill_(7.0)
    dec.select_attend(q, wl.q_scale, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(dec.cnt, cnt_a) and torch.equal(dec.sel, sel_a)
    assert torch.equal(dec.out.view(torch.int32), out_a.view(torch.int32))
    rs, rc = oracle.select(bt, bs32.astype(np.float64), wl.topk)
    assert np.array_equal(cnt_a.cpu().numpy(), rc) and np.array_equal(sel_a.cpu().numpy(), rs)
    ref = oracle.attention(bt, qd, wl.sm_scale, ck, cv, rs, rc)
    got = out_a.cpu().numpy().astype(np.float64)
    empty = np.repeat(rc == 0, 8, axis=2)
    assert (got[empty] == 0).all()
    err = _out_err(got, ref)
    print(f"  max per-vector relative error {err[~empty].max() if (~empty).any() else 0:.3e}", flush=True)
    assert err[~empty].max(initial=0.0) <= OUT_TOL


@pytest.mark.parametrize("case", ["prefill_ragged", "prefill_r512", "fp8_prefill"])
def test_prefill_row_route(M, oracle, case):
    """Prefill chunks through msa_select_decode without a workspace: the per-row form (one
    workgroup per row) instead of the block-major one, against the oracle."""
    wl = CASES[case]()
    _print_case(f"{case} per-row route", wl)
    _check_full_step(M, oracle, wl, fused=True, workspace=False)


@pytest.mark.parametrize("case,fused", [("prefill_topk64", True), ("prefill_topk1", True),
                                        ("prefill_wide_table", True), ("prefill_wide_table", False)])
def test_prefill_more_cases(M, oracle, case, fused):
    """Prefill chunks at the edges of the block-major route: 64 ranks per row (the merge's
    groups of 16 ranks four times), one rank per row, and a block table wider than the route
    counts in LDS (8,300 pages: the workspace size is 0 and the per-row form runs, whose fused
    selection differs from the separate one; the block-major route runs the same kernels
    either way)."""
    wl = CASES[case]()
    _print_case(f"{case} fused={fused}", wl)
    if case == "prefill_wide_table":
        assert M.msa_workspace_bytes(M.Batch(_dev(wl.block_table), _dev(wl.lengths), wl.R), wl.topk) == 0
    _check_full_step(M, oracle, wl, fused=fused)


def _hand_selection_check(M, oracle, wl, names, distinct=False):
    """msa_sparse_decode with hand-made selections through the workspace call and the
    no-allocation call (names: what each route is), both against the oracle's attention on
    the same sets with the absent entries left out.  distinct: a block named again within a
    row is replaced by -1 (the selection never repeats a block; a row group's union attends
    each block once per row, so repeats are only compared on one-row routes)."""
    dec, q_idx, q = gpu_setup(M, wl)
    rng = np.random.default_rng(5)
    p = row_positions(wl)
    nb = np.maximum(p // 128 + 1, 0)
    shape = (wl.B, wl.R, 4, wl.topk)
    cnt = rng.integers(0, wl.topk + 1, size=shape[:3]).astype(np.int32)
    odd = rng.random(shape[:3])
    cnt[odd < 0.03] = wl.topk + 3
    cnt[(odd >= 0.03) & (odd < 0.06)] = -2
    cnt[p < 0] = 0
    ids = np.floor(rng.random(shape) * nb[:, :, None, None]).astype(np.int32)
    k = np.arange(wl.topk)[None, None, None, :]
    inside = k < cnt[..., None]
    absent = inside & (rng.random(shape) < 0.05)
    if distinct:  # later repeats within a row become absent entries
        for idx in np.ndindex(*shape[:3]):
            _, first = np.unique(ids[idx], return_index=True)
            rep = np.ones(wl.topk, bool)
            rep[first] = False
            absent[idx] |= rep & inside[idx]
    sel_gpu = np.where(inside, ids, -1).astype(np.int32)
    sel_gpu[absent] = np.where(rng.random(int(absent.sum())) < 0.5, -1, wl.max_pages + 3)
    sel_ref = np.full(shape, -1, np.int32)
    cnt_ref = np.zeros(shape[:3], np.int32)
    keep = inside & ~absent
    for idx in np.ndindex(*shape[:3]):
        v = ids[idx][keep[idx]]
        sel_ref[idx][:v.size] = v
        cnt_ref[idx] = v.size
    dec.sel.copy_(_dev(sel_gpu))
    dec.cnt.copy_(_dev(cnt))
    dec.attend(q, wl.q_scale, wl.sm_scale)
    out_ws = dec.out.clone()
    out_na = torch.full_like(dec.out, 7.0)
    M.msa_sparse_decode_noalloc(dec.batch, q, dec.q_dtype, wl.q_scale, wl.sm_scale, dec.k, dec.v, dec.sel, dec.cnt,
                                wl.topk, out_na)
    torch.cuda.synchronize()
    _, ck, cv = oracle_caches(oracle, wl)
    _, _, _, qd = oracle_queries(oracle, wl)
    ref = oracle.attention(oracle_batch(oracle, wl), qd, wl.sm_scale, ck, cv, sel_ref, cnt_ref)
    empty = np.repeat(cnt_ref == 0, 8, axis=2)
    for name, got_t in zip(names, (out_ws, out_na)):
        got = got_t.cpu().numpy().astype(np.float64)
        assert (got[empty] == 0).all(), name
        err = _out_err(got, ref)
        print(f"  {name}: max per-vector relative error {err[~empty].max(initial=0.0):.3e}", flush=True)
        assert err[~empty].max(initial=0.0) <= OUT_TOL, name
    return dec


@pytest.mark.parametrize("case", ["prefill_ragged", "prefill_r512", "prefill_topk64", "fp8_prefill"])
def test_prefill_hand_selections_both_routes(M, oracle, case):
    """msa_sparse_decode on a prefill chunk with hand-made selections: blocks named twice,
    ranks in no order, counts from 0 to topk (a few above topk, which read as topk, and a few
    negative, which read as 0), and entries inside the count that name no block (-1, or past
    the table), which count as absent.  Through the block-major route (the workspace) and the
    per-row route (the no-allocation call, whose scratch array is too small for the
    block-major partials), each against the oracle's attention on the same sets with the
    absent entries left out."""
    wl = CASES[case]()
    _print_case(f"{case} hand-made selections", wl)
    wl_batch = M.Batch(_dev(wl.block_table), _dev(wl.lengths), wl.R)
    assert M.msa_workspace_bytes(wl_batch, wl.topk) > M.MSA_NOALLOC_SCRATCH_BYTES
    _hand_selection_check(M, oracle, wl, ("block-major", "per-row"))


@pytest.mark.parametrize("case", ["cfg1_f32", "cfg2_small", "cfg3_small", "ragged_r4", "union_r4", "fp8_cfg3_small",
                                  "cus_b48", "topk32"])
def test_decode_hand_selections(M, oracle, case):
    """The same hand-made selections through the decode forms: FP32 per-block partials, rows
    split over 4 and 2 workgroups, one workgroup per row, row-group unions, FP8, through the
    workspace call and the no-allocation call (the same kernels, its scratch array in place
    of the workspace)."""
    wl = CASES[case]()
    _print_case(f"{case} hand-made selections", wl)
    _hand_selection_check(M, oracle, wl, ("workspace", "no-allocation"), distinct=case == "union_r4")


def test_full_step_deterministic(M, oracle):
    wl = CASES["cfg4_small"]()
    _print_case("determinism", wl)
    dec, q_idx, q = gpu_setup(M, wl)
    dec.step(q_idx, q, wl.q_scale, wl.sm_scale)
    a = (dec.block_scores.clone(), dec.sel.clone(), dec.out.clone())
    dec.step(q_idx, q, wl.q_scale, wl.sm_scale)
    assert torch.equal(a[0], dec.block_scores) and torch.equal(a[1], dec.sel)
    assert torch.equal(a[2].view(torch.int32), dec.out.view(torch.int32))


@pytest.mark.parametrize("case", ["cfg3_small", "fp8_cfg3_small", "prefix_wide", "prefill_r512"])
@pytest.mark.parametrize("new_rows", [False, True])
def test_graph_replay_matches_eager(M, oracle, case, new_rows):
    """The step has no memset nodes and no host sync: capture it and replay it several
    times (with new rows, every replay inserts the same rows again, which is idempotent).
    NVFP4, FP8, a shared prefix and a prefill chunk (separate insert, dense indexer)."""
    wl = CASES[case]()
    _print_case(f"graph replay {case} new_rows={new_rows}", wl)
    if new_rows:
        dec, q_idx, q, new = gpu_setup(M, wl, hold_new=True)
    else:
        (dec, q_idx, q), new = gpu_setup(M, wl), None
    dec.step(q_idx, q, wl.q_scale, wl.sm_scale, new_tokens=new)
    torch.cuda.synchronize()
    eager = dec.out.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dec.step(q_idx, q, wl.q_scale, wl.sm_scale, new_tokens=new)
    for _ in range(3):
        dec.out.zero_()
        dec.sel.fill_(-7)
        dec.block_scores.fill_(1.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dec.out.view(torch.int32), eager.view(torch.int32))
        x = torch.randn(1000, device="cuda").sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        del x


# ---------------------------------------------------------------- physical-order scan (owner map)

def _owner_np(wl, lengths):
    """The owner map of a table and lengths, built by hand: b * max_pages + j at page
    table[b][j] for j < ceil(L_b / 128), -1 elsewhere."""
    own = np.full(wl.num_pages, -1, np.int32)
    for b in range(wl.B):
        for j in range(-(-int(lengths[b]) // 128)):
            own[wl.block_table[b, j]] = b * wl.max_pages + j
    return own


OWNER_CASES = ["cfg2_small", "cfg3_small", "cfg4_small", "ragged", "ragged_r2", "union_r2", "ragged_r4", "r3", "r5",
               "r7", "r8", "many_reqs", "wide_table", "wide_table_r4", "spare_pool", "spare_pool_r4", "topk64",
               "fp8_cfg3_small", "fp8_ragged", "fp8_ragged_r4", "fp8_r5", "fp8_r7", "fp8_r8", "fp8_many_reqs",
               "fp8_spare_pool", "fp8_spare_pool_r3"]


@pytest.mark.parametrize("case", ["cfg3_small", "ragged", "wide_table", "spare_pool", "spare_pool_r4"])
def test_page_owner_builds_the_inverse_table(M, oracle, case):
    """msa_page_owner: bitwise the map built by hand from the table and lengths."""
    wl = CASES[case]()
    _print_case(case, wl)
    batch = M.Batch(_dev(wl.block_table), _dev(wl.lengths), wl.R)
    out = torch.full((wl.num_pages,), 12345, dtype=torch.int32, device="cuda")
    M.msa_page_owner(batch, wl.num_pages, out)
    assert np.array_equal(out.cpu().numpy(), _owner_np(wl, wl.lengths))


@pytest.mark.parametrize("case", OWNER_CASES)
@pytest.mark.parametrize("insert", [False, True])
def test_owned_scan_equals_table_scan(M, oracle, case, insert):
    """The scan in physical page order: bitwise the block scores of the chunk-mapped scan
    (and, with the fused insert, bitwise the same cache bytes).  Its owner map is the one
    the previous step left (lengths L_b - R: the pages of the step's new rows may be
    missing), and every other entry holds junk, some of it naming real blocks whose table
    entries point elsewhere.  Afterwards the map holds the pages of the new rows too."""
    wl = CASES[case]()
    _print_case(f"{case} insert={insert}", wl)
    dec_a, q_idx, _, (nk, nv, ni, ns) = gpu_setup(M, wl, hold_new=True)
    dec_b, _, _, _ = gpu_setup(M, wl, hold_new=True)
    prev = np.maximum(wl.lengths.astype(np.int64) - wl.R, 0)
    own = _owner_np(wl, prev)
    rng = np.random.default_rng(7)
    junk = own < 0
    own[junk] = rng.integers(-3, wl.B * wl.max_pages + 3, size=int(junk.sum()), dtype=np.int32)
    own_t = _dev(own)
    dec_b.batch = M.Batch(dec_b.batch.block_table, dec_b.batch.ctx_lens, wl.R, page_owner=own_t)
    dec_a.insert(nk, nv, ni, ns)
    dec_a.index(q_idx, wl.q_scale)
    dec_b.block_scores.fill_(3.0)
    if insert:
        dec_b.insert_index(nk, nv, ni, q_idx, wl.q_scale)
    else:
        dec_b.insert(nk, nv, ni, ns)
        dec_b.index(q_idx, wl.q_scale)
    torch.cuda.synchronize()
    for ca, cb in ((dec_a.idx, dec_b.idx), (dec_a.k, dec_b.k), (dec_a.v, dec_b.v)):
        assert torch.equal(ca.pages, cb.pages)
    assert torch.equal(dec_a.block_scores.view(torch.int32), dec_b.block_scores.view(torch.int32))
    after = own_t.cpu().numpy()
    full = _owner_np(wl, wl.lengths)
    used = full >= 0
    assert np.array_equal(after[used], full[used])
    assert np.array_equal(after[~used], own[~used])  # only the new rows' pages are written


@pytest.mark.parametrize("case", ["cfg3_small", "ragged_r2", "ragged_r4", "r8", "spare_pool", "topk64",
                                  "fp8_ragged_r4", "fp8_spare_pool", "fp8_spare_pool_r3", "fp8_topk8"])
@pytest.mark.parametrize("new_rows", [False, True])
def test_full_step_owned_scan(M, oracle, case, new_rows):
    """Steps 0-4 with the physical-order scan (fused launches), against the oracle."""
    wl = CASES[case]()
    _print_case(f"{case} owner map new_rows={new_rows}", wl)
    _check_full_step(M, oracle, wl, new_rows=new_rows, owner=True)


def test_graph_replay_owned_scan(M, oracle):
    """The physical-order step captured and replayed (the owner-map writes repeat the same
    values): every replay bitwise the eager result."""
    wl = CASES["spare_pool"]()
    _print_case("graph replay owner map", wl)
    dec, q_idx, q, new = gpu_setup(M, wl, hold_new=True, owner=True)
    dec.step(q_idx, q, wl.q_scale, wl.sm_scale, new_tokens=new)
    torch.cuda.synchronize()
    eager, eager_bs = dec.out.clone(), dec.block_scores.clone()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        dec.step(q_idx, q, wl.q_scale, wl.sm_scale, new_tokens=new)
    for _ in range(3):
        dec.out.zero_()
        dec.block_scores.fill_(1.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dec.out.view(torch.int32), eager.view(torch.int32))
        assert torch.equal(dec.block_scores.view(torch.int32), eager_bs.view(torch.int32))
        x = torch.randn(1000, device="cuda").sum()
        torch.cuda.synchronize()
        del x


def _random_case(seed):
    """A seeded random small batch: B, R, ragged lengths (empty contexts included), topk, cache
    format, spare pool pages, owner map, new rows."""
    rng = np.random.default_rng([seed, 99])
    R = int(rng.choice([1, 1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 13))
    lengths = rng.integers(0, 3200, size=B)
    lengths[rng.random(B) < 0.15] = 0
    lengths[rng.random(B) < 0.15] = rng.integers(1, 5)
    topk = int(rng.choice([1, 4, 16, 16, 32, 64]))
    cache = "fp8" if rng.random() < 0.3 else "nvfp4"
    spare = int(rng.integers(0, 50))
    owner = rng.random() < 0.6
    new_rows = bool(rng.random() < 0.6)
    wl = W.make_workload(4 if R > 1 else 3, seed=seed, lengths=lengths.tolist(), R=R, topk=topk, cache=cache,
                         spare_pages=spare)
    return wl, owner, new_rows


@pytest.mark.parametrize("seed", list(range(500, 572)))
def test_random_small_batches(M, oracle, seed):
    """Seeded random small batches through the whole step (fused launches), against the oracle."""
    wl, owner, new_rows = _random_case(seed)
    _print_case(f"random seed={seed} owner={owner} new_rows={new_rows} topk={wl.topk} cache={wl.cache}", wl)
    _check_full_step(M, oracle, wl, new_rows=new_rows, owner=owner)


@pytest.mark.parametrize("seed", list(range(600, 612)))
def test_random_prefill_chunks(M, oracle, seed):
    """Seeded random prompt chunks (9 to 300 causal rows per request, 1 to 3 requests) through the
    dense indexer, the selection and the prefill attention, against the oracle."""
    rng = np.random.default_rng([seed, 98])
    B = int(rng.integers(1, 4))
    R = int(rng.integers(9, 301))
    lengths = rng.integers(R, R + 4000, size=B)
    topk = int(rng.choice([4, 16, 32]))
    cache = "fp8" if rng.random() < 0.3 else "nvfp4"
    wl = W.make_workload(6, seed=seed, lengths=lengths.tolist(), R=R, topk=topk, cache=cache)
    _print_case(f"random prefill seed={seed} topk={topk} cache={cache}", wl)
    _check_full_step(M, oracle, wl, new_rows=bool(rng.random() < 0.5))


@pytest.mark.parametrize("seed", list(range(700, 706)))
def test_random_shared_prefix(M, oracle, seed):
    """Seeded random shared-prefix batches (the prefix shrunk to 16-64 pages, 1 to 80 requests,
    1 to 4 rows) through the prefix product, the fused scan and the rest of the step."""
    rng = np.random.default_rng([seed, 97])
    wl = W.make_workload(5, seed=seed, B=int(rng.integers(1, 81)), len_div=int(rng.choice([32, 64, 128])),
                         R=int(rng.choice([1, 1, 2, 4])))
    new_rows = bool(rng.random() < 0.6)
    _print_case(f"random shared prefix seed={seed} new_rows={new_rows}", wl)
    _check_full_step(M, oracle, wl, new_rows=new_rows)


def _table_order_step_equal(M, wl, dec):
    """The step again in block-table order (no owner map), on the caches the physical-order
    step left with its new rows written: bitwise the same block scores, selections and outputs."""
    from block_sparse_attention_index_amd.decoder import MsaDecoder

    b = dec.batch
    dec2 = MsaDecoder(M.Batch(b.block_table, b.ctx_lens, wl.R), dec.k, dec.v, dec.idx, wl.topk)
    qi32, q32 = W.queries(wl)
    q_idx = M.msa_quantize_e4m3(_dev(qi32), wl.q_scale)
    q = M.msa_quantize_e4m3(_dev(q32), wl.q_scale)
    dec2.block_scores.fill_(3.0), dec2.sel.fill_(-5), dec2.cnt.fill_(-5), dec2.out.fill_(7.0)
    dec2.step(q_idx, q, wl.q_scale, wl.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(dec2.block_scores.view(torch.int32), dec.block_scores.view(torch.int32))
    assert torch.equal(dec2.cnt, dec.cnt) and torch.equal(dec2.sel, dec.sel)
    assert torch.equal(dec2.out.view(torch.int32), dec.out.view(torch.int32))


def test_full_size_config3_owned_sampled(M, oracle):
    """Configuration 3 at full size (B=32, 64K-192K tokens) through the physical-order scan,
    the step inserting its new rows (the benchmark's launch configuration); three sampled
    requests end to end against the oracle, then the whole batch in block-table order bitwise."""
    wl = W.make_workload(3, seed=0)
    _print_case("config 3 full size, owner map", wl)
    rows = [int(np.argmin(wl.lengths)), int(np.argmax(wl.lengths)), 7]
    dec = _check_full_step(M, oracle, wl, sample=rows, new_rows=True, owner=True)
    _table_order_step_equal(M, wl, dec)


def test_full_size_config3_fp8_owned_sampled(M, oracle):
    """The 128K-context batch in FP8 caches at full size through the physical-order scan,
    the step inserting its new rows; three sampled requests end to end against the oracle,
    then the whole batch in block-table order bitwise."""
    wl = W.make_workload(3, seed=0, cache="fp8")
    _print_case("config 3 fp8 full size, owner map", wl)
    rows = [int(np.argmin(wl.lengths)), int(np.argmax(wl.lengths)), 11]
    dec = _check_full_step(M, oracle, wl, sample=rows, new_rows=True, owner=True)
    _table_order_step_equal(M, wl, dec)


def test_full_size_config2_sampled(M, oracle):
    """Configuration 2 at full size (B=8, 32K tokens): rows split over 4 attention workgroups."""
    wl = W.make_workload(2, seed=0)
    _print_case("config 2 full size", wl)
    _check_full_step(M, oracle, wl, sample=[0, 6])


def test_full_size_config7_sampled(M, oracle):
    """The forced-dense configuration at full size (B=32, 8K tokens, top-64 of 64 blocks): every
    block is selected, so attention covers each whole context."""
    wl = W.make_workload(7, seed=0)
    _print_case("config 7 full size", wl)
    _check_full_step(M, oracle, wl, sample=[0, 17, 31])


def test_full_size_config4_sampled(M, oracle):
    wl = W.make_workload(4, seed=0)
    _print_case("config 4 full size", wl)
    _check_full_step(M, oracle, wl, sample=[0, 5])


def test_full_size_config5_sampled(M, oracle):
    """The shared-prefix workload at full size (64 requests on one 262,144-token
    prefix + 1K-8K private tokens each), with the step inserting its new rows, in
    the bench's launch configuration; the oracle checks two sampled requests."""
    wl = W.make_workload(5, seed=0)
    _print_case("config 5 full size", wl)
    rows = [int(np.argmin(wl.lengths)), int(np.argmax(wl.lengths))]
    _check_full_step(M, oracle, wl, sample=rows, new_rows=True)



def test_full_size_config6_sampled(M, oracle):
    """The prefill workload at full size (4 prompts of 64K tokens, the last 2,048 of each a
    chunk of causal rows), the step inserting the chunk's rows, in the bench's launch
    configuration.  The oracle checks 12 sampled rows of one request, each as a one-row
    request of its own: context p + 1 for the row at position p (it sees tokens 0..p, as in
    the chunk), the same block-table row and caches."""
    wl = W.make_workload(6, seed=0)
    _print_case("config 6 full size", wl)
    dec, q_idx, q, new = gpu_setup(M, wl, hold_new=True)
    dec.step(q_idx, q, wl.q_scale, wl.sm_scale, new_tokens=new)
    torch.cuda.synchronize()
    g_sel, g_cnt = dec.sel.cpu().numpy(), dec.cnt.cpu().numpy()
    g_out = dec.out.cpu().numpy().astype(np.float64)
    g_bs = dec.block_scores.cpu().numpy().astype(np.float64)
    b = 1
    rows = np.array([0, 1, 127, 128, 500, 1023, 1024, 1500, 1919, 1920, 2046, 2047])
    ci, ck, cv = _sampled_caches(oracle, wl, np.array([b]))
    _, _, qi, qd = oracle_queries(oracle, wl)
    p = int(wl.lengths[b]) - wl.R + rows  # positions of the sampled rows
    n = rows.size
    table = np.repeat(wl.block_table[b:b + 1], n, axis=0)
    bt = oracle.OracleBatch(table, (p + 1).astype(np.int32), 1)
    qi_s, qd_s = qi[b, rows][:, None], qd[b, rows][:, None]  # [n][1][4][128], [n][1][32][128]
    res = oracle.decode_step(bt, qi_s, qd_s, wl.sm_scale, ci, ck, cv, wl.topk)
    ts, ab = oracle.index_scores(bt, qi_s, ci, with_abs=True)
    absmax = ab.reshape(ab.shape[:3] + (wl.max_pages, 128)).max(-1)
    ref_bs, got_bs = res["block_scores"][:, 0], g_bs[b, rows]
    fin = np.isfinite(ref_bs)
    assert np.array_equal(np.isfinite(got_bs), fin)
    assert (np.abs(got_bs[fin] - ref_bs[fin]) <= SCORE_TOL * absmax[:, 0][fin] + 1e-30).all()
    mism = 0
    for i in range(n):
        for g in range(4):
            ok, _ = selection_guard_ok(res["block_scores"][i, 0, g], res["sel"][i, 0, g], res["cnt"][i, 0, g],
                                       g_sel[b, rows[i], g], g_cnt[b, rows[i], g], p[i], wl.topk)
            mism += not ok
    assert mism == 0
    ref_own = oracle.attention(bt, qd_s, wl.sm_scale, ck, cv, g_sel[b, rows][:, None], g_cnt[b, rows][:, None])
    err = _out_err(g_out[b, rows][:, None], ref_own)
    print(f"  {n} rows: max per-vector relative error {err.max():.3e}", flush=True)
    assert err.max() <= OUT_TOL


def test_abi_errors_on_device(M):
    print("[case] abi errors", flush=True)
    wl = CASES["cfg2_small"]()
    dec, q_idx, q = gpu_setup(M, wl)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(M.MsaError) as e:
        M.msa_sparse_decode(dec.batch, q, M.MSA_FP8_E4M3, 1.0, wl.sm_scale, dec.k, dec.v, dec.sel, dec.cnt,
                            wl.topk, dec.out, small)
    assert e.value.status == M.MSA_ERR_WORKSPACE
    with pytest.raises(M.MsaError) as e:
        M.msa_block_maxpool_topk(dec.batch, dec.block_scores, 0, 0, dec.sel, dec.cnt)
    assert e.value.status == M.MSA_ERR_INVALID_ARG
    f32 = W.make_workload(1, seed=0)
    dec32, _, q32 = gpu_setup(M, f32)
    with pytest.raises(M.MsaError) as e:
        dec32.select_attend(q32, 1.0, f32.sm_scale)
    assert e.value.status == M.MSA_ERR_UNSUPPORTED
