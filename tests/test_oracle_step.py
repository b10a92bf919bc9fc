"""Pins of the oracle's MSA decode step (CPU only).

Each step is checked against something other than the oracle itself:
numpy matrix products over the raw FP32 rows or over pinned dequantised pages
(indexer), numpy reductions (max-pool), brute-force sorting (selection),
torch's scaled_dot_product_attention in float64 (attention; the dense special
case when every block is selected, and the masked case otherwise), plus the
invariants the pages state.
"""
import numpy as np
import pytest
import torch

import workload as W
from conftest import read_golden
from helpers import decode_pages_f64, oracle_batch, oracle_caches, oracle_queries, row_positions


def _gather_tokens(wl, dequant_pages, head, b, n_tok):
    """Rows of request b in position order from a [pages][heads][128][128] dequantised pool."""
    pages = wl.block_table[b, : -(-n_tok // 128)] if n_tok else np.zeros(0, np.int32)
    rows = dequant_pages[pages, head].reshape(-1, 128)
    return rows[:n_tok].astype(np.float64)


def _raw_rows_by_position(wl, b):
    """FP32 generator rows of request b in position order (prefix included)."""
    parts_i, parts_k, parts_v = [], [], []
    if wl.prefix_tokens:
        pi, pk, pv = W.prefix_rows(wl)
        parts_i.append(pi), parts_k.append(pk), parts_v.append(pv)
    ri, rk, rv = W.request_rows(wl, b)
    parts_i.append(ri), parts_k.append(rk), parts_v.append(rv)
    return (np.concatenate(parts_i).astype(np.float64), np.concatenate(parts_k).astype(np.float64),
            np.concatenate(parts_v).astype(np.float64))


@pytest.mark.parametrize("R,lens", [(1, [4096]), (4, [1000, 131, 4]), (2, [300, 1])])
def test_indexer_f32_matches_numpy(oracle, R, lens):
    wl = W.make_workload(1, seed=3, lengths=lens, R=R)
    ci, ck, cv = oracle_caches(oracle, wl)
    _, _, qi, _ = oracle_queries(oracle, wl)
    bt = oracle_batch(oracle, wl)
    ts = oracle.index_scores(bt, qi, ci)
    p = row_positions(wl)
    for b in range(wl.B):
        rows, _, _ = _raw_rows_by_position(wl, b)
        for r in range(R):
            n = max(p[b, r] + 1, 0)
            for g in range(wl.G):
                w = np.full(wl.max_pages * 128, -np.inf)
                w[:n] = rows[:n] @ qi[b, r, g]
                np.testing.assert_allclose(ts[b, r, g], w, rtol=1e-12, atol=1e-12)


def test_indexer_nvfp4_matches_numpy_over_dequantised_pages(oracle):
    wl = W.make_workload(3, seed=1, B=3, len_div=64, R=2)
    ci, ck, cv = oracle_caches(oracle, wl)
    _, _, qi, _ = oracle_queries(oracle, wl)
    bt = oracle_batch(oracle, wl)
    ts = oracle.index_scores(bt, qi, ci)
    deq = decode_pages_f64(ci.bytes, True, False, 1, wl.num_pages, wl.tensor_scale)
    assert np.array_equal(ci.dequant_pages(np.arange(wl.num_pages)), deq.astype(np.float32))
    p = row_positions(wl)
    for b in range(wl.B):
        rows = _gather_tokens(wl, deq, 0, b, int(wl.lengths[b]))
        for r in range(wl.R):
            n = p[b, r] + 1
            for g in range(wl.G):
                w = np.full(wl.max_pages * 128, -np.inf)
                w[:n] = rows[:n] @ qi[b, r, g]
                np.testing.assert_allclose(ts[b, r, g], w, rtol=1e-12, atol=1e-9)


def test_indexer_fp8_matches_numpy_over_dequantised_pages(oracle):
    wl = W.make_workload(3, seed=1, B=3, len_div=64, R=2, cache="fp8")
    ci, ck, cv = oracle_caches(oracle, wl)
    _, _, qi, _ = oracle_queries(oracle, wl)
    bt = oracle_batch(oracle, wl)
    ts = oracle.index_scores(bt, qi, ci)
    deq = decode_pages_f64(ci.bytes, False, False, 1, wl.num_pages, wl.tensor_scale, fp8=True, half_rows=True)
    assert np.array_equal(ci.dequant_pages(np.arange(wl.num_pages)), deq.astype(np.float32))
    p = row_positions(wl)
    for b in range(wl.B):
        rows = _gather_tokens(wl, deq, 0, b, int(wl.lengths[b]))
        for r in range(wl.R):
            n = p[b, r] + 1
            for g in range(wl.G):
                w = np.full(wl.max_pages * 128, -np.inf)
                w[:n] = rows[:n] @ qi[b, r, g]
                np.testing.assert_allclose(ts[b, r, g], w, rtol=1e-12, atol=1e-9)


def test_maxpool_matches_numpy(oracle):
    wl = W.make_workload(3, seed=2, B=2, len_div=64, R=3)
    ci, _, _ = oracle_caches(oracle, wl)
    _, _, qi, _ = oracle_queries(oracle, wl)
    bt = oracle_batch(oracle, wl)
    ts = oracle.index_scores(bt, qi, ci)
    bs = oracle.block_maxpool(bt, ts)
    want = ts.reshape(ts.shape[:3] + (wl.max_pages, 128)).max(-1)
    assert np.array_equal(bs, want)


def _brute_select(scores, n, topk):
    if n <= topk:
        return list(range(n))
    latest = n - 1

    def key(j):
        s = scores[j]
        return (1, 0.0, j) if np.isnan(s) else (0, -s, j)

    best = sorted(range(latest), key=key)[: topk - 1]
    return sorted(best + [latest])


@pytest.mark.parametrize("topk", [1, 4, 16, 64])
def test_select_matches_bruteforce_with_ties(oracle, topk):
    rng = np.random.default_rng(topk)
    B, R, G, P = 5, 2, 4, 90
    lens = np.array([1, 128, 129, 90 * 128, 3000])
    wl_table = np.zeros((B, P), np.int32)
    bt = oracle.OracleBatch(wl_table, lens, R)
    scores = rng.integers(-3, 4, size=(B, R, G, P)).astype(np.float64)  # many exact ties
    scores[0, 0, 0, :5] = [-0.0, 0.0, -0.0, 0.0, np.nan]
    scores[3, 1, 2, 10:20] = np.nan
    sel, cnt = oracle.select(bt, scores, topk)
    for b in range(B):
        for r in range(R):
            p = lens[b] - R + r
            n = 0 if p < 0 else p // 128 + 1
            for g in range(G):
                want = _brute_select(scores[b, r, g], n, topk)
                assert cnt[b, r, g] == len(want)
                assert list(sel[b, r, g, : len(want)]) == want
                assert (sel[b, r, g, len(want):] == -1).all()


def test_select_invariants_on_real_scores(oracle):
    facts = {r[0]: int(r[1]) for r in read_golden("page_facts.txt")}
    wl = W.make_workload(3, seed=4, B=4, len_div=32, R=4)
    ci, _, _ = oracle_caches(oracle, wl)
    _, _, qi, _ = oracle_queries(oracle, wl)
    bt = oracle_batch(oracle, wl)
    bs = oracle.block_maxpool(bt, oracle.index_scores(bt, qi, ci))
    sel, cnt = oracle.select(bt, bs, facts["topk_blocks"])
    p = row_positions(wl)
    for b in range(wl.B):
        for r in range(wl.R):
            n = p[b, r] // 128 + 1
            for g in range(wl.G):
                s = sel[b, r, g, : cnt[b, r, g]]
                assert cnt[b, r, g] == min(facts["topk_blocks"], n)
                assert n - 1 in s, "latest block always kept"
                keys = sum(min(128, p[b, r] + 1 - 128 * j) for j in s)
                assert keys <= facts["keys_per_query_cap"]


def test_dcp_merge_of_shard_topk_is_exact(oracle):
    """Context-parallel selection (each shard's local candidates, merged by
    score with global block ids) equals the single-device selection."""
    rng = np.random.default_rng(9)
    P, topk = 400, 16
    scores = rng.integers(-50, 50, size=(1, 1, 1, P)).astype(np.float64)
    bt = oracle.OracleBatch(np.zeros((1, P), np.int32), np.array([P * 128]), 1)
    sel, cnt = oracle.select(bt, scores, topk)
    latest = P - 1
    shards = np.array_split(np.arange(latest), 4)
    cands = []
    for sh in shards:
        local = sorted(sh, key=lambda j: (-scores[0, 0, 0, j], j))[: topk - 1]
        cands += list(local)
    merged = sorted(cands, key=lambda j: (-scores[0, 0, 0, j], j))[: topk - 1]
    assert sorted(merged + [latest]) == list(sel[0, 0, 0])


def _sdpa_reference(q, k, v, mask, scale):
    """torch scaled_dot_product_attention on CPU in float64. q [H][D], k/v [T][D], mask [H][T] bool."""
    qt = torch.from_numpy(q)[None, :, None, :]  # [1][H][1][D]
    kt = torch.from_numpy(k)[None, None].expand(1, q.shape[0], -1, -1).contiguous()
    vt = torch.from_numpy(v)[None, None].expand(1, q.shape[0], -1, -1).contiguous()
    m = torch.from_numpy(mask)[None, :, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return out[0, :, 0, :].numpy()


@pytest.mark.parametrize("cfg,R,lens,cache", [(1, 1, [2048], None), (1, 4, [1999, 5], None),
                                              (3, 1, [1500, 2048], None), (3, 2, [1500, 2048, 3], "fp8")])
def test_attention_dense_case_equals_sdpa(oracle, cfg, R, lens, cache):
    """With <= 16 blocks every block is selected: MSA is dense causal GQA attention."""
    wl = W.make_workload(cfg, seed=5, lengths=lens, R=R, cache=cache)
    ci, ck, cv = oracle_caches(oracle, wl)
    _, _, qi, q = oracle_queries(oracle, wl)
    bt = oracle_batch(oracle, wl)
    res = oracle.decode_step(bt, qi, q, wl.sm_scale, ci, ck, cv, wl.topk)
    p = row_positions(wl)
    if wl.cache != "f32":
        fp8 = wl.cache == "fp8"
        dk = decode_pages_f64(ck.bytes, not fp8, False, wl.G, wl.num_pages, wl.tensor_scale, fp8=fp8)
        dv = decode_pages_f64(cv.bytes, not fp8, True, wl.G, wl.num_pages, wl.tensor_scale, fp8=fp8)
        assert np.array_equal(cv.dequant_pages(np.arange(wl.num_pages)), dv.astype(np.float32))
    for b in range(wl.B):
        if wl.cache == "f32":
            _, kr, vr = _raw_rows_by_position(wl, b)
        for g in range(wl.G):
            if wl.cache == "f32":
                K, V = kr[:, g], vr[:, g]
            else:
                K = _gather_tokens(wl, dk, g, b, int(wl.lengths[b]))
                V = _gather_tokens(wl, dv, g, b, int(wl.lengths[b]))
            for r in range(R):
                if p[b, r] < 0:
                    assert (res["out"][b, r] == 0).all()
                    continue
                hs = slice(g * 8, g * 8 + 8)
                T = K.shape[0]
                mask = np.broadcast_to(np.arange(T) <= p[b, r], (8, T)).copy()
                want = _sdpa_reference(q[b, r, hs], K, V, mask, wl.sm_scale)
                np.testing.assert_allclose(res["out"][b, r, hs], want, rtol=1e-10, atol=1e-12)


def test_attention_sparse_case_equals_masked_sdpa(oracle):
    """Beyond 16 blocks: attention equals SDPA restricted to the selected blocks' visible tokens,
    with every head of a group using the group's set."""
    wl = W.make_workload(3, seed=6, B=2, len_div=32, R=2)
    ci, ck, cv = oracle_caches(oracle, wl)
    _, _, qi, q = oracle_queries(oracle, wl)
    bt = oracle_batch(oracle, wl)
    res = oracle.decode_step(bt, qi, q, wl.sm_scale, ci, ck, cv, wl.topk)
    dk = decode_pages_f64(ck.bytes, True, False, wl.G, wl.num_pages, wl.tensor_scale)
    dv = decode_pages_f64(cv.bytes, True, True, wl.G, wl.num_pages, wl.tensor_scale)
    p = row_positions(wl)
    for b in range(wl.B):
        for g in range(wl.G):
            K = _gather_tokens(wl, dk, g, b, int(wl.lengths[b]))
            V = _gather_tokens(wl, dv, g, b, int(wl.lengths[b]))
            T = K.shape[0]
            for r in range(wl.R):
                sel = res["sel"][b, r, g, : res["cnt"][b, r, g]]
                assert res["cnt"][b, r, g] == 16
                vis = np.zeros(T, bool)
                for j in sel:
                    vis[128 * j: 128 * j + 128] = True
                vis &= np.arange(T) <= p[b, r]
                hs = slice(g * 8, g * 8 + 8)
                want = _sdpa_reference(q[b, r, hs], K, V, np.broadcast_to(vis, (8, T)).copy(), wl.sm_scale)
                np.testing.assert_allclose(res["out"][b, r, hs], want, rtol=1e-10, atol=1e-12)


def test_physical_page_permutation_invariance(oracle):
    wl = W.make_workload(3, seed=7, B=2, len_div=48, R=1)
    ci, ck, cv = oracle_caches(oracle, wl)
    _, _, qi, q = oracle_queries(oracle, wl)
    res = oracle.decode_step(oracle_batch(oracle, wl), qi, q, wl.sm_scale, ci, ck, cv, wl.topk)
    perm = np.random.default_rng(0).permutation(wl.num_pages)
    wl2 = W.make_workload(3, seed=7, B=2, len_div=48, R=1)
    wl2.block_table = perm[wl.block_table].astype(np.int32)
    ci2, ck2, cv2 = oracle_caches(oracle, wl2)
    res2 = oracle.decode_step(oracle_batch(oracle, wl2), qi, q, wl.sm_scale, ci2, ck2, cv2, wl.topk)
    for k in ("block_scores", "sel", "cnt", "out"):
        assert np.array_equal(res[k], res2[k]), k


def test_empty_and_short_requests(oracle):
    wl = W.make_workload(3, seed=8, lengths=[0, 2, 130, 2049], R=4)
    ci, ck, cv = oracle_caches(oracle, wl)
    _, _, qi, q = oracle_queries(oracle, wl)
    res = oracle.decode_step(oracle_batch(oracle, wl), qi, q, wl.sm_scale, ci, ck, cv, wl.topk)
    assert (res["cnt"][0] == 0).all() and (res["sel"][0] == -1).all() and (res["out"][0] == 0).all()
    assert np.isneginf(res["block_scores"][0]).all()
    # L=2 with R=4: rows 0,1 sit at negative positions and see nothing
    assert (res["cnt"][1, :2] == 0).all() and (res["out"][1, :2] == 0).all()
    assert (res["cnt"][1, 2:] == 1).all() and np.all(np.isfinite(res["out"][1, 2:]))
    assert list(res["cnt"][2, :, 0]) == [1, 1, 2, 2]  # rows at 126..129
    # 2049 tokens, R=4: rows at 2045..2048 -> rows 0-2 have 16 blocks (all), row 3 has 17 (select)
    assert list(res["cnt"][3, :, 0]) == [16, 16, 16, 16]
    assert 16 in res["sel"][3, 3, 0] and 16 not in res["sel"][3, 0, 0]


def test_shared_prefix_equals_private_copies(oracle):
    """Requests reading shared prefix pages get the same results as with private copies."""
    wl = W.make_workload(5, seed=1, B=3, len_div=64)
    assert wl.prefix_pages > 16
    ci, ck, cv = oracle_caches(oracle, wl)
    _, _, qi, q = oracle_queries(oracle, wl)
    res = oracle.decode_step(oracle_batch(oracle, wl), qi, q, wl.sm_scale, ci, ck, cv, wl.topk)
    for b in range(wl.B):
        one = W.make_workload(5, seed=1, B=3, len_div=64)
        one.block_table = wl.block_table[b:b + 1]
        one.lengths = wl.lengths[b:b + 1]
        r1 = oracle.decode_step(oracle_batch(oracle, one), qi[b:b + 1], q[b:b + 1], wl.sm_scale, ci, ck, cv, wl.topk)
        for k in ("block_scores", "sel", "out"):
            assert np.array_equal(res[k][b], r1[k][0]), k


def test_index_scan_is_one_eighth_of_dense_kv_bytes():
    facts = {r[0]: int(r[1]) for r in read_golden("page_facts.txt")}
    assert facts["index_bytes_per_token_fp8"] * 8 == facts["dense_kv_bytes_per_token_fp8"]
    # NVFP4 caches: 72 B index per token vs 576 B of K+V (4 heads x 128 x 2 x 0.5625)
    nv_index = 128 * 0.5625
    nv_kv = facts["kv_heads"] * facts["head_dim"] * 2 * 0.5625
    assert nv_index * 8 == nv_kv
    assert facts["topk_blocks"] * facts["block_tokens"] == facts["keys_per_query_cap"]
