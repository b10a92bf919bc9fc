"""msa_sparse_decode_noalloc (the library's fixed per-GPU scratch array instead of a caller
workspace) against msa_sparse_decode through the C ABI: bitwise the same outputs on two calls
in a row, the second with a smaller batch, in F32 caches (whose route keeps per-block partial
results in scratch memory) and NVFP4 caches (no scratch); and the outputs within the
attention bar (per head vector max|o - o_ref| / max|o_ref| <= 2e-3) of the oracle's."""
import numpy as np
import pytest
import torch

import workload as W
from helpers import oracle_batch, oracle_caches, oracle_queries

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import block_sparse_attention_index_amd as M

    return M


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _run(M, oracle, wl):
    from block_sparse_attention_index_amd.decoder import MsaDecoder, make_caches

    dtype = {"nvfp4": M.MSA_NVFP4, "f32": M.MSA_F32}[wl.cache]
    k, v, idx = make_caches(dtype, wl.num_pages, wl.tensor_scale)
    batch = M.Batch(_dev(wl.block_table), _dev(wl.lengths), wl.R)
    dec = MsaDecoder(batch, k, v, idx, wl.topk)
    slots, xi, xk, xv = W.all_rows(wl)
    dec.insert(_dev(xk), _dev(xv), _dev(xi), _dev(slots))
    qi32, q32 = W.queries(wl)
    if wl.cache == "f32":
        q_idx, q = _dev(qi32), _dev(q32)
    else:
        q_idx, q = M.msa_quantize_e4m3(_dev(qi32), wl.q_scale), M.msa_quantize_e4m3(_dev(q32), wl.q_scale)
    dec.index(q_idx, wl.q_scale)
    dec.select()
    dec.attend(q, wl.q_scale, wl.sm_scale)  # msa_sparse_decode, caller workspace
    ref = dec.out.clone()
    out = torch.full_like(dec.out, 7.0)
    M.msa_sparse_decode_noalloc(batch, q, dec.q_dtype, wl.q_scale, wl.sm_scale, k, v, dec.sel, dec.cnt, wl.topk, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    # the oracle on the GPU's selection
    _, ck, cv = oracle_caches(oracle, wl)
    _, _, _, qd = oracle_queries(oracle, wl)
    want = oracle.attention(oracle_batch(oracle, wl), qd, wl.sm_scale, ck, cv, dec.sel.cpu().numpy(),
                            dec.cnt.cpu().numpy())
    got = out.cpu().numpy().astype(np.float64)
    err = np.abs(got - want).max(-1) / np.maximum(np.abs(want).max(-1), 1e-30)
    assert err.max() <= 2e-3
    return batch


@pytest.mark.parametrize("cache", ["f32", "nvfp4"])
def test_noalloc_matches_workspace_call_twice(M, oracle, cache):
    """Two calls in a row, the second smaller: the scratch keeps the first call's contents and
    the second must not depend on them."""
    print(f"[case] noalloc {cache}", flush=True)
    if cache == "f32":
        big = W.make_workload(1, seed=40, lengths=[4096, 1500, 130], R=2)
        small = W.make_workload(1, seed=41, lengths=[700], R=1)
    else:
        big = W.make_workload(3, seed=42, B=6, len_div=24)
        small = W.make_workload(3, seed=43, B=2, len_div=48)
    _run(M, oracle, big)
    _run(M, oracle, small)


def test_noalloc_rejects_oversized_f32_batch(M):
    """An F32 batch whose partial results exceed the scratch array is refused before any launch."""
    print("[case] noalloc oversized", flush=True)
    wl = W.make_workload(1, seed=44, lengths=[4096] * 16, R=1)
    from block_sparse_attention_index_amd.decoder import MsaDecoder, make_caches

    k, v, idx = make_caches(M.MSA_F32, wl.num_pages, 1.0)
    batch = M.Batch(_dev(wl.block_table), _dev(wl.lengths), wl.R)
    assert M.msa_workspace_bytes(batch, wl.topk) > M.MSA_NOALLOC_SCRATCH_BYTES
    dec = MsaDecoder(batch, k, v, idx, wl.topk)
    q = torch.zeros((wl.B, wl.R, 32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(M.MsaError) as e:
        M.msa_sparse_decode_noalloc(batch, q, M.MSA_F32, 1.0, wl.sm_scale, k, v, dec.sel, dec.cnt, wl.topk, dec.out)
    assert e.value.status == M.MSA_ERR_WORKSPACE
