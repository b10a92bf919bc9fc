"""Python binding of the MI355X MSA decode library (``libmsa.so``, include/msa.h).

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI.  PyTorch supplies device memory and streams.  Importing
this package raises if the HIP library has not been built -- there is no
CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_HIP = 0, -1, -2, -3, -4
MSA_F32, MSA_FP8_E4M3, MSA_NVFP4 = 0, 1, 2
MSA_TOKEN_MAJOR, MSA_DIM_MAJOR, MSA_HALF_ROWS = 0, 1, 2
MSA_MAX_ROWS, MSA_MAX_PREFILL_ROWS = 8, 8192
MSA_NOALLOC_SCRATCH_BYTES = 4 << 20
PAGE_TOKENS = 128
HEAD_DIM = 128
HEADS_PER_GROUP = 8
NVFP4_SLAB_BYTES = 9216
F32_SLAB_BYTES = 65536
FP8_SLAB_BYTES = 16384


class MsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_text(status)} ({status})")
        self.status = status


class msa_cache(C.Structure):
    _fields_ = [("dtype", C.c_int32), ("layout", C.c_int32), ("num_heads", C.c_int32), ("num_pages", C.c_int32),
                ("tensor_scale", C.c_float), ("pages", C.c_void_p)]


class msa_batch(C.Structure):
    _fields_ = [("num_reqs", C.c_int32), ("rows_per_req", C.c_int32), ("max_pages_per_req", C.c_int32),
                ("shared_prefix_pages", C.c_int32), ("block_table", C.c_void_p), ("ctx_lens", C.c_void_p),
                ("page_owner", C.c_void_p)]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950)")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
    P = C.POINTER
    sigs = {
        "msa_kv_insert": (C.c_int, [vp, vp, vp, vp, i32, P(msa_cache), P(msa_cache), P(msa_cache), vp]),
        "msa_kv_insert_nvfp4": (C.c_int, [vp, vp, vp, vp, i32, P(msa_cache), P(msa_cache), P(msa_cache), vp]),
        "msa_quantize_e4m3": (C.c_int, [vp, i64, f32, vp, vp]),
        "msa_index_score": (C.c_int, [P(msa_batch), vp, i32, f32, P(msa_cache), vp, vp, vp]),
        "msa_page_owner": (C.c_int, [P(msa_batch), i32, vp, vp]),
        "msa_block_maxpool_topk": (C.c_int, [P(msa_batch), vp, i32, i32, vp, vp, vp]),
        "msa_workspace_bytes": (sz, [P(msa_batch), i32]),
        "msa_sparse_decode": (C.c_int, [P(msa_batch), vp, i32, f32, f32, P(msa_cache), P(msa_cache), vp, vp, i32,
                                        vp, vp, sz, vp]),
        "msa_sparse_decode_noalloc": (C.c_int, [P(msa_batch), vp, i32, f32, f32, P(msa_cache), P(msa_cache), vp, vp,
                                                i32, vp, vp]),
        "msa_select_decode": (C.c_int, [P(msa_batch), vp, i32, vp, i32, f32, f32, P(msa_cache), P(msa_cache), vp,
                                        vp, vp, vp, sz, vp]),
        "msa_insert_index_score": (C.c_int, [P(msa_batch), vp, vp, vp, vp, i32, f32, P(msa_cache), P(msa_cache),
                                             P(msa_cache), vp, vp, vp]),
        "msa_qkv_project_insert": (C.c_int, [vp, vp, i32, i32, vp, f32, vp, i32, vp, vp, f32, vp, vp, P(msa_cache),
                                             P(msa_cache), P(msa_cache), vp, vp]),
        "msa_status_str": (C.c_char_p, [C.c_int]),
        "msa_debug_dequant": (C.c_int, [P(msa_cache), vp, i32, i32, vp, vp]),
        "msa_debug_stream_read": (C.c_int, [vp, i64, i32, vp, vp]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    return L


lib = _load()


def status_text(status: int) -> str:
    return lib.msa_status_str(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != MSA_OK:
        raise MsaError(status, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        return int(t)
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MSA library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


class Cache:
    """A device page pool for one cache tensor (keys, values or index keys)."""

    def __init__(self, pages: torch.Tensor, dtype: int, layout: int, num_heads: int, num_pages: int,
                 tensor_scale: float = 1.0):
        self.pages, self.dtype, self.layout = pages, dtype, layout
        self.num_heads, self.num_pages, self.tensor_scale = num_heads, num_pages, float(tensor_scale)
        self.struct = msa_cache(dtype, layout, num_heads, num_pages, self.tensor_scale, pages.data_ptr())

    @staticmethod
    def slab_bytes(dtype: int) -> int:
        return {MSA_F32: F32_SLAB_BYTES, MSA_FP8_E4M3: FP8_SLAB_BYTES, MSA_NVFP4: NVFP4_SLAB_BYTES}[dtype]

    @classmethod
    def empty(cls, dtype: int, layout: int, num_heads: int, num_pages: int, tensor_scale: float = 1.0,
              device="cuda") -> "Cache":
        nbytes = num_pages * num_heads * cls.slab_bytes(dtype)
        pages = torch.zeros(nbytes, dtype=torch.uint8, device=device)
        return cls(pages, dtype, layout, num_heads, num_pages, tensor_scale)

    def ref(self):
        return C.byref(self.struct)


class Batch:
    """Block table and context lengths (device int32) of one decode step."""

    def __init__(self, block_table: torch.Tensor, ctx_lens: torch.Tensor, rows_per_req: int,
                 shared_prefix_pages: int = 0, page_owner: torch.Tensor | None = None):
        """page_owner: None, or a device int32 [index pool pages] owner map (msa_page_owner builds it)."""
        assert block_table.dtype == torch.int32 and ctx_lens.dtype == torch.int32
        assert page_owner is None or (page_owner.dtype == torch.int32 and page_owner.is_contiguous())
        self.block_table, self.ctx_lens, self.page_owner = block_table, ctx_lens, page_owner
        B, P = block_table.shape
        self.struct = msa_batch(B, rows_per_req, P, shared_prefix_pages, _ptr(block_table), _ptr(ctx_lens),
                                _ptr(page_owner))

    def ref(self):
        return C.byref(self.struct)

    @property
    def B(self):
        return self.struct.num_reqs

    @property
    def R(self):
        return self.struct.rows_per_req

    @property
    def max_pages(self):
        return self.struct.max_pages_per_req


def _cref(c):
    return None if c is None else c.ref()


def msa_kv_insert(k, v, idx_k, slot_mapping, k_cache, v_cache, idx_cache, stream=None) -> None:
    n = slot_mapping.shape[0]
    _check(lib.msa_kv_insert(_ptr(k), _ptr(v), _ptr(idx_k), _ptr(slot_mapping), n, _cref(k_cache), _cref(v_cache),
                             _cref(idx_cache), _stream(stream)), "msa_kv_insert")


def msa_kv_insert_nvfp4(k, v, idx_k, slot_mapping, k_cache, v_cache, idx_cache, stream=None) -> None:
    n = slot_mapping.shape[0]
    _check(lib.msa_kv_insert_nvfp4(_ptr(k), _ptr(v), _ptr(idx_k), _ptr(slot_mapping), n, _cref(k_cache),
                                   _cref(v_cache), _cref(idx_cache), _stream(stream)), "msa_kv_insert_nvfp4")


def msa_qkv_project_insert(x, w, norm_weight, eps: float, rope_cos_sin, positions, slot_mapping, q_scale: float,
                           q_out, q_idx_out, k_cache, v_cache, idx_cache, pre_quant=None, stream=None) -> None:
    """x [n][hidden] BF16 bit patterns (int16/uint16/bfloat16 tensor); w the BF16 weights in the
    library's 32-k blocked layout, [45][hidden/32][128][32]."""
    n, hidden = x.shape
    _check(lib.msa_qkv_project_insert(_ptr(x), _ptr(w), n, hidden, _ptr(norm_weight), float(eps), _ptr(rope_cos_sin),
                                      rope_cos_sin.shape[0], _ptr(positions), _ptr(slot_mapping), float(q_scale),
                                      _ptr(q_out), _ptr(q_idx_out), _cref(k_cache), _cref(v_cache), _cref(idx_cache),
                                      _ptr(pre_quant), _stream(stream)),
           "msa_qkv_project_insert")


def msa_quantize_e4m3(x: torch.Tensor, scale: float = 1.0, out: torch.Tensor | None = None, stream=None):
    if out is None:
        out = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(lib.msa_quantize_e4m3(_ptr(x), x.numel(), float(scale), _ptr(out), _stream(stream)), "msa_quantize_e4m3")
    return out


def msa_index_score(batch: Batch, q_idx, q_dtype: int, q_scale: float, idx_cache: Cache, block_scores,
                    token_scores=None, stream=None) -> None:
    _check(lib.msa_index_score(batch.ref(), _ptr(q_idx), q_dtype, float(q_scale), idx_cache.ref(),
                               _ptr(block_scores), _ptr(token_scores), _stream(stream)), "msa_index_score")


def msa_page_owner(batch: Batch, num_pages: int, page_owner=None, stream=None):
    """The block table's inverse over an index pool of num_pages pages (device int32 [num_pages])."""
    if page_owner is None:
        page_owner = torch.empty(num_pages, dtype=torch.int32, device=batch.block_table.device)
    _check(lib.msa_page_owner(batch.ref(), int(num_pages), _ptr(page_owner), _stream(stream)), "msa_page_owner")
    return page_owner


def msa_insert_index_score(batch: Batch, k_new, v_new, idx_new, q_idx, q_dtype: int, q_scale: float,
                           k_cache: Cache, v_cache: Cache, idx_cache: Cache, block_scores, token_scores=None,
                           stream=None) -> None:
    _check(lib.msa_insert_index_score(batch.ref(), _ptr(k_new), _ptr(v_new), _ptr(idx_new), _ptr(q_idx), q_dtype,
                                      float(q_scale), k_cache.ref(), v_cache.ref(), idx_cache.ref(),
                                      _ptr(block_scores), _ptr(token_scores), _stream(stream)),
           "msa_insert_index_score")


def msa_block_maxpool_topk(batch: Batch, scores, scores_are_token_level: int, topk: int, sel_blocks, sel_count,
                           stream=None) -> None:
    _check(lib.msa_block_maxpool_topk(batch.ref(), _ptr(scores), int(scores_are_token_level), int(topk),
                                      _ptr(sel_blocks), _ptr(sel_count), _stream(stream)), "msa_block_maxpool_topk")


def msa_workspace_bytes(batch: Batch, topk: int) -> int:
    return int(lib.msa_workspace_bytes(batch.ref(), int(topk)))


def msa_sparse_decode(batch: Batch, q, q_dtype: int, q_scale: float, sm_scale: float, k_cache: Cache,
                      v_cache: Cache, sel_blocks, sel_count, topk: int, out, workspace, stream=None) -> None:
    _check(lib.msa_sparse_decode(batch.ref(), _ptr(q), q_dtype, float(q_scale), float(sm_scale), k_cache.ref(),
                                 v_cache.ref(), _ptr(sel_blocks), _ptr(sel_count), int(topk), _ptr(out),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "msa_sparse_decode")


def msa_select_decode(batch: Batch, block_scores, topk: int, q, q_dtype: int, q_scale: float, sm_scale: float,
                      k_cache: Cache, v_cache: Cache, sel_blocks, sel_count, out, workspace=None, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.msa_select_decode(batch.ref(), _ptr(block_scores), int(topk), _ptr(q), q_dtype, float(q_scale),
                                 float(sm_scale), k_cache.ref(), v_cache.ref(), _ptr(sel_blocks), _ptr(sel_count),
                                 _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)), "msa_select_decode")


def msa_status_str(status: int) -> str:
    return status_text(status)


def msa_debug_dequant(cache: Cache, pages, mode: int, out, stream=None) -> None:
    _check(lib.msa_debug_dequant(cache.ref(), _ptr(pages), pages.shape[0], int(mode), _ptr(out), _stream(stream)),
           "msa_debug_dequant")


def msa_debug_stream_read(src: torch.Tensor, workgroups: int, sink: torch.Tensor, stream=None) -> None:
    """Read all of src (a contiguous device tensor) with the index scan's streaming loads: a measurement aid."""
    _check(lib.msa_debug_stream_read(_ptr(src), src.numel() * src.element_size(), int(workgroups), _ptr(sink),
                                     _stream(stream)), "msa_debug_stream_read")


def msa_sparse_decode_noalloc(batch: Batch, q, q_dtype: int, q_scale: float, sm_scale: float, k_cache: Cache,
                              v_cache: Cache, sel_blocks, sel_count, topk: int, out, stream=None) -> None:
    """msa_sparse_decode with the library's fixed per-GPU scratch array instead of a workspace."""
    _check(lib.msa_sparse_decode_noalloc(batch.ref(), _ptr(q), q_dtype, float(q_scale), float(sm_scale),
                                         k_cache.ref(), v_cache.ref(), _ptr(sel_blocks), _ptr(sel_count), int(topk),
                                         _ptr(out), _stream(stream)), "msa_sparse_decode_noalloc")
