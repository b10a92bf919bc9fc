"""Shared test helpers: oracle cache construction and comparison rules.

Nothing here imports the HIP library; GPU-side helpers live in the GPU test
files themselves.
"""
import numpy as np

import workload as W


def oracle_caches(o, wl):
    """Fill the oracle's own caches from the seeded FP32 rows (oracle quantiser)."""
    dt = {"f32": o.F32, "nvfp4": o.NVFP4, "fp8": o.FP8_E4M3}[wl.cache]
    vlayout = o.TOKEN_MAJOR if dt == o.F32 else o.DIM_MAJOR
    idx = o.OracleCache(dt, o.HALF_ROWS if dt == o.FP8_E4M3 else o.TOKEN_MAJOR, 1, wl.num_pages, wl.tensor_scale)
    k = o.OracleCache(dt, o.TOKEN_MAJOR, wl.G, wl.num_pages, wl.tensor_scale)
    v = o.OracleCache(dt, vlayout, wl.G, wl.num_pages, wl.tensor_scale)
    slots, xi, xk, xv = W.all_rows(wl)
    if slots.shape[0]:
        idx.write(slots, xi)
        k.write(slots, xk)
        v.write(slots, xv)
    return idx, k, v


def oracle_queries(o, wl):
    """Queries as the oracle sees them: FP8 bytes (its own quantiser) decoded, or FP32."""
    q_idx, q = W.queries(wl)
    if wl.cache == "f32":
        return q_idx, q, o.decode_queries(q_idx, o.F32), o.decode_queries(q, o.F32)
    bi = o.quantize_queries(q_idx, wl.q_scale)
    bq = o.quantize_queries(q, wl.q_scale)
    return bi, bq, o.decode_queries(bi, o.FP8_E4M3, wl.q_scale), o.decode_queries(bq, o.FP8_E4M3, wl.q_scale)


def oracle_batch(o, wl):
    return o.OracleBatch(wl.block_table, wl.lengths, wl.R)


def row_positions(wl):
    """p[b][r] = L_b - R + r."""
    return wl.lengths[:, None].astype(np.int64) - wl.R + np.arange(wl.R)[None, :]


def selection_guard_ok(ref_scores, ref_sel, ref_cnt, got_sel, got_cnt, p, topk, rel=1e-3):
    """Compare one (b, r, g) selection under the guard rule.

    Sets must be identical where the oracle's (topk-1)-th and topk-th candidate
    scores (the latest block set aside) differ by more than ``rel`` relative.
    Inside the band, the GPU set must hold the latest block, every block whose
    score is clearly above the band, the right count, and only blocks from the
    band otherwise.  Returns (ok, guarded).
    """
    n = 0 if p < 0 else p // 128 + 1
    ref = set(int(x) for x in ref_sel[:ref_cnt])
    got = set(int(x) for x in got_sel[:got_cnt])
    pad_ok = all(int(x) == -1 for x in got_sel[got_cnt:]) and list(got_sel[:got_cnt]) == sorted(got)
    if got_cnt != ref_cnt or not pad_ok:
        return False, False
    if n <= topk:
        return got == ref, False
    latest = n - 1
    cand = sorted(((float(ref_scores[j]), j) for j in range(latest)), key=lambda t: (-t[0], t[1]))
    a = cand[topk - 2][0]
    b = cand[topk - 1][0]
    denom = max(abs(a), abs(b))
    gap = abs(a - b) / denom if denom > 0 else 0.0
    if gap > rel:
        return got == ref, False
    lo = b - rel * denom
    hi = a + rel * denom
    if latest not in got:
        return False, True
    for s, j in cand:
        if s > hi and j not in got:
            return False, True
    for j in got:
        if j != latest and ref_scores[j] < lo:
            return False, True
    return True, True


def _e2m1_table():
    from conftest import read_golden

    t = np.zeros(16)
    for code, val in read_golden("e2m1_table.txt"):
        t[int(code, 16)] = float(val)
    return t


def _e4m3_table():
    import torch

    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def decode_pages_f64(raw, nvfp4: bool, dim_major: bool, heads: int, num_pages: int, tensor_scale: float,
                     fp8: bool = False, half_rows: bool = False):
    """Exact float64 values [pages][heads][128 tok][128 dim] of a page pool, decoded from
    its bytes by the documented slab layout (test-side, independent of the oracle).
    fp8: one E4M3 byte per element, [tok][dim] (token-major), [dim][tok] (dim_major) or
    [tok/16][dim/64][tok%16][dim%64] (half_rows), times the tensor scale."""
    raw = np.asarray(raw, dtype=np.uint8)
    if fp8:
        if half_rows:
            b = raw.reshape(num_pages, heads, 8, 2, 16, 64)  # [chunk][half][tok][dim]
            b = np.transpose(b, (0, 1, 2, 4, 3, 5)).reshape(num_pages, heads, 128, 128)
            return _e4m3_table()[b] * tensor_scale
        v = _e4m3_table()[raw.reshape(num_pages, heads, 128, 128)] * tensor_scale
        return np.swapaxes(v, -1, -2) if dim_major else v
    if not nvfp4:
        return raw.view(np.float32).reshape(num_pages, heads, 128, 128).astype(np.float64)
    slabs = raw.reshape(num_pages, heads, 9216)
    codes = slabs[..., :8192].reshape(num_pages, heads, 128, 64)
    scales = slabs[..., 8192:]
    nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(num_pages, heads, 128, 128)
    vals = _e2m1_table()[nib]
    e4 = _e4m3_table()
    if not dim_major:  # nib[..., t, d]; scales [t][8]
        s = e4[scales.reshape(num_pages, heads, 128, 8)]
        return vals * np.repeat(s, 16, axis=-1) * tensor_scale
    # dim-major: nib[..., d, t]; scales [8 groups][128 tokens]
    s = e4[scales.reshape(num_pages, heads, 8, 128)]  # [.., j, t]
    s_dt = np.repeat(s, 16, axis=-2)  # [.., d, t]
    return np.swapaxes(vals * s_dt, -1, -2) * tensor_scale
