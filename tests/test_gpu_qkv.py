"""GPU parity of msa_qkv_project_insert -- the projection of a step's new rows fused
with their norm, rotary embedding and quantisation into the caches (vLLM M3.1 post,
"QKV GEMM + norm + RoPE + KV insert fusion") -- against the oracle on the same seeded
inputs, through the C ABI.

Bars:
  * values just before quantisation (the pre_quant output): |got - ref| <= bar =
    4 (H/32 + 8) 2^-24 max |ref| over the head's 128 values, H the hidden size.
    Derived: the products are exact in FP32 (BF16 x BF16); the matrix cores sum them
    in blocks of 32 into FP32 and the workgroup adds four partial sums, so the sum
    takes about H/32 + 4 roundings of 2^-24 relative to partial sums of the order of
    max |ref|; the norm and rotation add a few more; 4 is the margin.
  * bytes (FP8 queries, NVFP4 K/V/index pages): equal to the oracle's quantisation of
    its own values wherever that quantisation does not change when every value moves
    by the bar above, toward or away from zero; bytes that do change (a value within
    the bar of a rounding boundary) are counted and must stay under 2% of the written
    bytes.  Untouched bytes must stay untouched.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workload as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_attention_index_amd as M

    return M


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_gpu(M, q, with_pre=True):
    """Run the fused call; return (pre, q_out, q_idx_out, k bytes, v bytes, idx bytes) as numpy."""
    n = q.x.shape[0]
    x = _dev(q.x.view(np.int16))
    w = _dev(W.pack_qkv_weights(q.w).view(np.int16))
    kc = M.Cache.empty(M.MSA_NVFP4, M.MSA_TOKEN_MAJOR, 4, q.num_pages, q.tensor_scale)
    vc = M.Cache.empty(M.MSA_NVFP4, M.MSA_DIM_MAJOR, 4, q.num_pages, q.tensor_scale)
    ic = M.Cache.empty(M.MSA_NVFP4, M.MSA_TOKEN_MAJOR, 1, q.num_pages, q.tensor_scale)
    q_out = torch.full((n, 32, 128), 0xAB, dtype=torch.uint8, device="cuda")
    qi_out = torch.full((n, 4, 128), 0xAB, dtype=torch.uint8, device="cuda")
    pre = torch.full((n, 45, 128), float("nan"), dtype=torch.float32, device="cuda") if with_pre else None
    M.msa_qkv_project_insert(x, w, _dev(q.norm_weight), q.eps, _dev(q.rope), _dev(q.positions), _dev(q.slots),
                             q.q_scale, q_out, qi_out, kc, vc, ic, pre)
    torch.cuda.synchronize()
    pre_np = None if pre is None else pre.cpu().numpy()
    return (pre_np, q_out.cpu().numpy(), qi_out.cpu().numpy(), kc.pages.cpu().numpy(), vc.pages.cpu().numpy(),
            ic.pages.cpu().numpy())


def _bar(ref, hidden):
    return 4.0 * (hidden / 32 + 8) * 2.0 ** -24 * np.max(np.abs(ref), axis=-1, keepdims=True)


def _variants(ref, hidden):
    """The oracle's values and the two moved by the bar: (ref, away from zero, toward zero)."""
    bar = _bar(ref, hidden)
    s = np.sign(ref)
    return [ref, ref + bar * s, ref - bar * s]


def _stable_compare(got, outs, written_mask=None, what=""):
    """outs: the oracle's bytes for the three variants.  Where they agree the GPU must
    match; returns the fraction of written bytes where they do not."""
    b0, b1, b2 = outs
    stable = (b0 == b1) & (b0 == b2)
    bad = np.flatnonzero((got != b0) & stable)
    assert bad.size == 0, f"{what}: {bad.size} stable bytes differ, first at {bad[:5]}"
    written = written_mask if written_mask is not None else np.ones_like(b0, dtype=bool)
    frac = float((~stable & written).sum()) / max(1, int(written.sum()))
    print(f"  {what}: unstable {frac:.4%} of {int(written.sum())} bytes", flush=True)
    assert frac < 0.02
    return frac


def check_against_oracle(q, got, tokens=None):
    """got: run_gpu output.  tokens: the token indices the oracle evaluates (all by default);
    cache bytes are then compared over those tokens' slots only."""
    pre, q_out, qi_out, kb, vb, ib = got
    n = q.x.shape[0]
    tok = np.arange(n) if tokens is None else np.asarray(tokens)
    ref = O.qkv_project(q.x[tok], q.w, q.norm_weight, q.eps, q.rope, q.positions[tok]).astype(np.float64)
    ok = (q.positions[tok] >= 0) & (q.positions[tok] < q.rope.shape[0])
    in_pool = (q.slots[tok] >= 0) & (q.slots[tok] < q.num_pages * 128)
    # values before quantisation
    if pre is not None:
        p = pre[tok].astype(np.float64)
        assert np.isnan(p[~ok]).all(), "a token past the rotary table wrote values"
        bar = _bar(ref[ok], q.x.shape[1])
        err = np.abs(p[ok] - ref[ok])
        ratio = float((err / bar).max()) if err.size else 0.0
        print(f"  pre-quantisation error / bar max = {ratio:.4f}", flush=True)
        assert ratio <= 1.0
    var = _variants(np.where(ok[:, None, None], ref, 0.0).astype(np.float64), q.x.shape[1])
    # FP8 queries and index queries
    for lo, hi, out, name in ((0, 32, q_out, "queries"), (40, 44, qi_out, "index queries")):
        outs = [O.quantize_queries(v[ok, lo:hi].astype(np.float32), q.q_scale) for v in var]
        _stable_compare(out[tok][ok], outs, what=name)
        assert (out[tok][~ok] == 0xAB).all(), f"{name} of a token past the rotary table were written"
    # caches: only valid tokens write; everything else in the pools must stay zero
    wtok = ok & in_pool
    slots = q.slots[tok][wtok]
    for lo, hi, layout, heads, got_b, name in ((32, 36, O.TOKEN_MAJOR, 4, kb, "key pages"),
                                               (36, 40, O.DIM_MAJOR, 4, vb, "value pages"),
                                               (44, 45, O.TOKEN_MAJOR, 1, ib, "index-key pages")):
        outs = []
        for v in var:
            c = O.OracleCache(O.NVFP4, layout, heads, q.num_pages, q.tensor_scale)
            c.write(slots, v[wtok, lo:hi].astype(np.float32))
            outs.append(c.bytes)
        if tokens is not None:
            # sampled tokens: compare the bytes those tokens own (token-major rows and scales;
            # dim-major nibbles through the page decoder would mix in unsampled tokens)
            if layout == O.TOKEN_MAJOR:
                own = np.zeros(outs[0].shape, dtype=bool)
                slab = 9216
                for s in slots:
                    pg, off = divmod(int(s), 128)
                    for h in range(heads):
                        base = (pg * heads + h) * slab
                        own[base + off * 64: base + off * 64 + 64] = True
                        own[base + 8192 + off * 8: base + 8192 + off * 8 + 8] = True
                _stable_compare(got_b[own], [o[own] for o in outs], what=name)
            continue
        written = np.zeros(outs[0].shape, dtype=bool)
        for o in outs:
            written |= o != 0
        _stable_compare(got_b, outs, written, what=name)


# at most 64 rows: one workgroup per (head, 16 rows); more: per (head, 64 rows)
@pytest.mark.parametrize("n,hidden,bad_pos,bad_slot", [(1, 256, 0, 0), (17, 768, 1, 0), (37, 512, 2, 2),
                                                       (64, 256, 0, 3), (65, 256, 1, 1), (130, 512, 3, 0),
                                                       (200, 1024, 1, 1), (32, 3072, 0, 0)])
def test_qkv_project_insert_matches_oracle(M, n, hidden, bad_pos, bad_slot):
    q = W.make_qkv_inputs(100 + n, n, hidden, max_pos=5000, bad_positions=bad_pos, bad_slots=bad_slot)
    print(f"[case] qkv n={n} hidden={hidden} bad_positions={bad_pos} bad_slots={bad_slot}", flush=True)
    got = run_gpu(M, q)
    check_against_oracle(q, got)


def test_qkv_without_pre_output_writes_the_same_bytes(M):
    q = W.make_qkv_inputs(7, 70, 512, max_pos=3000, bad_positions=1, bad_slots=1)
    a = run_gpu(M, q, with_pre=True)
    b = run_gpu(M, q, with_pre=False)
    for x, y in zip(a[1:], b[1:]):
        assert np.array_equal(x, y)


def test_qkv_consecutive_slots_of_a_prompt_chunk(M):
    """A prompt chunk writes consecutive slots: both tokens of every value byte come from
    one call (the dim-major nibble merge)."""
    q = W.make_qkv_inputs(8, 300, 256, max_pos=5000)
    q.num_pages = 4
    q.slots = np.arange(5, 305, dtype=np.int64)
    got = run_gpu(M, q)
    check_against_oracle(q, got)


def test_qkv_prefill_chunk_sampled(M):
    """A 2,048-token chunk at a model width of 3,072: the oracle on 12 sampled tokens."""
    q = W.make_qkv_inputs(9, 2048, 3072, max_pos=70000)
    q.num_pages = 16
    q.slots = np.arange(2048, dtype=np.int64)
    got = run_gpu(M, q)
    rows = np.random.default_rng(1).choice(2048, 12, replace=False)
    check_against_oracle(q, got, tokens=rows)


@pytest.mark.parametrize("n,hidden", [(32, 1024), (300, 512)])
def test_qkv_graph_replay_matches_eager(M, n, hidden):
    """Captured in a HIP graph and replayed three times (eager work and synchronisations in
    between, caches cleared by a fill kernel before each replay): every replay writes the
    bytes of the eager call."""
    q = W.make_qkv_inputs(40 + n, n, hidden, max_pos=4000, bad_positions=1, bad_slots=1)
    q.num_pages = max(q.num_pages, 4)
    print(f"[case] qkv graph n={n} hidden={hidden}", flush=True)
    x = _dev(q.x.view(np.int16))
    w = _dev(W.pack_qkv_weights(q.w).view(np.int16))
    g, rope, pos, slots = _dev(q.norm_weight), _dev(q.rope), _dev(q.positions), _dev(q.slots)
    kc = M.Cache.empty(M.MSA_NVFP4, M.MSA_TOKEN_MAJOR, 4, q.num_pages, q.tensor_scale)
    vc = M.Cache.empty(M.MSA_NVFP4, M.MSA_DIM_MAJOR, 4, q.num_pages, q.tensor_scale)
    ic = M.Cache.empty(M.MSA_NVFP4, M.MSA_TOKEN_MAJOR, 1, q.num_pages, q.tensor_scale)
    q_out = torch.zeros((n, 32, 128), dtype=torch.uint8, device="cuda")
    qi_out = torch.zeros((n, 4, 128), dtype=torch.uint8, device="cuda")
    outs = (q_out, qi_out, kc.pages, vc.pages, ic.pages)

    def call(stream=None):
        M.msa_qkv_project_insert(x, w, g, q.eps, rope, pos, slots, q.q_scale, q_out, qi_out, kc, vc, ic,
                                 stream=stream)

    call()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for t in outs:
            t.zero_()
        call(stream)  # warm-up on the capture stream
        stream.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            call(stream)
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            assert torch.equal(a, b), f"replay {rep} differs"
        _ = (x.float() * 2).sum().item()  # eager work between replays
