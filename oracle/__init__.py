"""CPU oracle for the MSA decode step: numpy-facing wrapper over ``liboracle.so``.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the cpu_baseline leg of ``bench.py`` may import this package.  It does not
import, load or share anything with the HIP library
(``block_sparse_attention_index_amd``); the two are compared with each other,
never composed.

Every function here marshals arguments; the arithmetic is in
``msa_oracle.c`` (FP64 accumulation, plain loops, each step citing the page
passage it follows).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

from . import build as _build

F32, FP8_E4M3, NVFP4 = 0, 1, 2
TOKEN_MAJOR, DIM_MAJOR, HALF_ROWS = 0, 1, 2
PAGE = 128
DIM = 128
NVFP4_SLAB = 9216
F32_SLAB = PAGE * DIM * 4
FP8_SLAB = PAGE * DIM

_lib = None


def lib() -> C.CDLL:
    """Load liboracle.so, building it with gcc first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        u8, f32, f64, i32, i64, vp = C.c_uint8, C.c_float, C.c_double, C.c_int32, C.c_int64, C.c_void_p
        L.ref_e4m3_value.restype, L.ref_e4m3_value.argtypes = f64, [u8]
        L.ref_e2m1_value.restype, L.ref_e2m1_value.argtypes = f64, [u8]
        L.ref_e4m3_encode.restype, L.ref_e4m3_encode.argtypes = u8, [f32]
        L.ref_e2m1_encode.restype, L.ref_e2m1_encode.argtypes = u8, [f32]
        L.ref_nvfp4_quantize_group.restype = None
        L.ref_nvfp4_quantize_group.argtypes = [vp, f32, vp, vp]
        L.ref_nvfp4_value.restype, L.ref_nvfp4_value.argtypes = f64, [u8, u8, f32]
        L.ref_fp8_quantize.restype, L.ref_fp8_quantize.argtypes = u8, [f32, f32]
        L.ref_fp8_value.restype, L.ref_fp8_value.argtypes = f64, [u8, f32]
        L.ref_cache_write.restype, L.ref_cache_write.argtypes = C.c_int, [vp, i64, C.c_int, vp]
        L.ref_cache_write_many.restype, L.ref_cache_write_many.argtypes = i64, [vp, vp, i64, vp]
        L.ref_cache_value.restype, L.ref_cache_value.argtypes = f64, [vp, i64, C.c_int, C.c_int, C.c_int]
        L.ref_cache_dequant_pages.restype, L.ref_cache_dequant_pages.argtypes = None, [vp, vp, i32, vp]
        L.ref_decode_queries.restype, L.ref_decode_queries.argtypes = None, [vp, i32, f32, i64, vp]
        L.ref_quantize_queries.restype, L.ref_quantize_queries.argtypes = None, [vp, i64, f32, vp]
        L.ref_index_scores.restype, L.ref_index_scores.argtypes = None, [vp, C.c_int, vp, vp, vp, vp]
        L.ref_block_maxpool.restype, L.ref_block_maxpool.argtypes = None, [vp, C.c_int, vp, vp]
        L.ref_select.restype, L.ref_select.argtypes = None, [vp, C.c_int, vp, C.c_int, vp, vp]
        L.ref_bf16_value.restype, L.ref_bf16_value.argtypes = f64, [C.c_uint16]
        L.ref_qkv_project.restype = None
        L.ref_qkv_project.argtypes = [vp, vp, i32, i32, vp, f32, vp, i32, vp, vp]
        L.ref_attention.restype = None
        L.ref_attention.argtypes = [vp, C.c_int, C.c_int, vp, f64, vp, vp, vp, vp, C.c_int, vp]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> C.c_void_p:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return C.c_void_p(a.ctypes.data)


# --------------------------------------------------------------------------- codecs
def e4m3_value(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    L = lib()
    return np.array([L.ref_e4m3_value(int(c)) for c in codes.ravel()], dtype=np.float64).reshape(codes.shape)


def e2m1_value(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    L = lib()
    return np.array([L.ref_e2m1_value(int(c)) for c in codes.ravel()], dtype=np.float64).reshape(codes.shape)


def e4m3_encode(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    L = lib()
    return np.array([L.ref_e4m3_encode(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def e2m1_encode(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    L = lib()
    return np.array([L.ref_e2m1_encode(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def nvfp4_quantize(x, tensor_scale: float):
    """Quantise rows of 16 values: returns (codes [..., 8] uint8, scales [...] uint8)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    assert x.shape[-1] % 16 == 0
    groups = x.reshape(-1, 16)
    codes = np.zeros((groups.shape[0], 8), dtype=np.uint8)
    scales = np.zeros((groups.shape[0],), dtype=np.uint8)
    L = lib()
    ts = C.c_float(tensor_scale)
    for i in range(groups.shape[0]):
        g = np.ascontiguousarray(groups[i])
        c = np.zeros(8, dtype=np.uint8)
        s = np.zeros(1, dtype=np.uint8)
        L.ref_nvfp4_quantize_group(_ptr(g), ts, _ptr(c), _ptr(s))
        codes[i] = c
        scales[i] = s[0]
    lead = x.shape[:-1] + (x.shape[-1] // 16,)
    return codes.reshape(lead + (8,)), scales.reshape(lead)


def nvfp4_value(code: int, scale: int, tensor_scale: float) -> float:
    return lib().ref_nvfp4_value(code, scale, C.c_float(tensor_scale))


def fp8_quantize(x, tensor_scale: float) -> np.ndarray:
    """FP8 cache codes of FP32 values: E4M3(x / tensor_scale)."""
    x = np.asarray(x, dtype=np.float32)
    L = lib()
    ts = C.c_float(tensor_scale)
    return np.array([L.ref_fp8_quantize(float(v), ts) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def fp8_value(code: int, tensor_scale: float) -> float:
    return lib().ref_fp8_value(code, C.c_float(tensor_scale))


def quantize_queries(x, q_scale: float = 1.0) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.zeros(x.shape, dtype=np.uint8)
    lib().ref_quantize_queries(_ptr(x), x.size, C.c_float(q_scale), _ptr(out))
    return out


def decode_queries(q, dtype: int, q_scale: float = 1.0) -> np.ndarray:
    q = np.ascontiguousarray(q)
    out = np.zeros(q.shape, dtype=np.float64)
    lib().ref_decode_queries(_ptr(q), dtype, C.c_float(q_scale), q.size, _ptr(out))
    return out


QKV_HEADS = 45  # query heads 0..31, keys 32..35, values 36..39, index queries 40..43, index key 44


def bf16_value(bits: int) -> float:
    return lib().ref_bf16_value(int(bits))


def qkv_project(x_bits, w_bits, norm_weight, eps: float, rope, positions) -> np.ndarray:
    """The rows a step's projection produces after norm and rotary embedding (values as
    projected): [n][45][128] FP32.  x_bits [n][hidden], w_bits [45*128][hidden] BF16 bit
    patterns (uint16); norm_weight [4][128]; rope [rows][128] (cos, then sin); positions [n]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_bits, dtype=np.uint16)
    g = np.ascontiguousarray(norm_weight, dtype=np.float32)
    rp = np.ascontiguousarray(rope, dtype=np.float32)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    n, hidden = x.shape
    assert w.shape == (QKV_HEADS * DIM, hidden) and g.shape == (4, DIM) and rp.shape[1] == DIM
    out = np.zeros((n, QKV_HEADS, DIM), dtype=np.float32)
    lib().ref_qkv_project(_ptr(x), _ptr(w), n, hidden, _ptr(g), C.c_float(eps), _ptr(rp), rp.shape[0], _ptr(pos),
                          _ptr(out))
    return out


# --------------------------------------------------------------------------- caches
class _RefCache(C.Structure):
    _fields_ = [
        ("dtype", C.c_int32),
        ("layout", C.c_int32),
        ("num_heads", C.c_int32),
        ("num_pages", C.c_int32),
        ("tensor_scale", C.c_float),
        ("pages", C.c_void_p),
    ]


class OracleCache:
    """A paged cache held in host memory in the byte layout the format defines."""

    def __init__(self, dtype: int, layout: int, num_heads: int, num_pages: int, tensor_scale: float = 1.0):
        self.dtype, self.layout, self.num_heads, self.num_pages = dtype, layout, num_heads, num_pages
        self.tensor_scale = float(np.float32(tensor_scale))
        self.slab = {F32: F32_SLAB, FP8_E4M3: FP8_SLAB, NVFP4: NVFP4_SLAB}[dtype]
        self.bytes = np.zeros(num_pages * num_heads * self.slab, dtype=np.uint8)
        self._s = _RefCache(dtype, layout, num_heads, num_pages, self.tensor_scale, self.bytes.ctypes.data)

    def ref(self) -> C.c_void_p:
        return C.cast(C.pointer(self._s), C.c_void_p)

    def write(self, slots, x) -> None:
        """Quantise and store tokens: x [n][num_heads][128] (or [n][128] for one head)."""
        x = np.asarray(x, dtype=np.float32)
        if x.ndim == 2:
            x = x[:, None, :]
        x = np.ascontiguousarray(x)
        slots = np.asarray(slots, dtype=np.int64)
        assert x.shape == (slots.shape[0], self.num_heads, DIM)
        slots = np.ascontiguousarray(slots)
        bad = lib().ref_cache_write_many(self.ref(), _ptr(slots), slots.shape[0], _ptr(x))
        if bad:
            raise ValueError(f"{bad} slot(s) outside the page pool")

    def value(self, page: int, head: int, t: int, d: int) -> float:
        return lib().ref_cache_value(self.ref(), page, head, t, d)

    def dequant_pages(self, pages) -> np.ndarray:
        pages = np.ascontiguousarray(np.asarray(pages, dtype=np.int32))
        out = np.zeros((pages.shape[0], self.num_heads, PAGE, DIM), dtype=np.float32)
        lib().ref_cache_dequant_pages(self.ref(), _ptr(pages), pages.shape[0], _ptr(out))
        return out


# --------------------------------------------------------------------------- step
class _RefBatch(C.Structure):
    _fields_ = [
        ("B", C.c_int32),
        ("R", C.c_int32),
        ("max_pages", C.c_int32),
        ("block_table", C.c_void_p),
        ("ctx_lens", C.c_void_p),
    ]


@dataclass
class OracleBatch:
    block_table: np.ndarray  # [B][max_pages] int32
    ctx_lens: np.ndarray  # [B] int32
    R: int

    def __post_init__(self):
        self.block_table = np.ascontiguousarray(self.block_table, dtype=np.int32)
        self.ctx_lens = np.ascontiguousarray(self.ctx_lens, dtype=np.int32)
        B, P = self.block_table.shape
        self._s = _RefBatch(B, self.R, P, self.block_table.ctypes.data, self.ctx_lens.ctypes.data)

    @property
    def B(self):
        return self.block_table.shape[0]

    @property
    def max_pages(self):
        return self.block_table.shape[1]

    def ref(self) -> C.c_void_p:
        return C.cast(C.pointer(self._s), C.c_void_p)


def index_scores(batch: OracleBatch, q_idx: np.ndarray, idx_cache: OracleCache, with_abs: bool = False):
    """Step 1. q_idx: decoded [B][R][G][128] float64. Returns token scores [B][R][G][max_pages*128]."""
    B, R, G, _ = q_idx.shape
    q_idx = np.ascontiguousarray(q_idx, dtype=np.float64)
    T = batch.max_pages * PAGE
    ts = np.zeros((B, R, G, T), dtype=np.float64)
    ab = np.zeros((B, R, G, T), dtype=np.float64) if with_abs else None
    lib().ref_index_scores(batch.ref(), G, _ptr(q_idx), idx_cache.ref(), _ptr(ts),
                           _ptr(ab) if with_abs else None)
    return (ts, ab) if with_abs else ts


def block_maxpool(batch: OracleBatch, token_scores: np.ndarray) -> np.ndarray:
    """Step 2. token scores [B][R][G][T] -> block scores [B][R][G][max_pages]."""
    B, R, G, _ = token_scores.shape
    token_scores = np.ascontiguousarray(token_scores, dtype=np.float64)
    out = np.zeros((B, R, G, batch.max_pages), dtype=np.float64)
    lib().ref_block_maxpool(batch.ref(), G, _ptr(token_scores), _ptr(out))
    return out


def select(batch: OracleBatch, block_scores: np.ndarray, topk: int = 16):
    """Step 3. Returns (sel [B][R][G][topk] int32 ascending, -1 padded; count [B][R][G] int32)."""
    B, R, G, _ = block_scores.shape
    block_scores = np.ascontiguousarray(block_scores, dtype=np.float64)
    sel = np.zeros((B, R, G, topk), dtype=np.int32)
    cnt = np.zeros((B, R, G), dtype=np.int32)
    lib().ref_select(batch.ref(), G, _ptr(block_scores), topk, _ptr(sel), _ptr(cnt))
    return sel, cnt


def attention(batch: OracleBatch, q: np.ndarray, sm_scale: float, k_cache: OracleCache, v_cache: OracleCache,
              sel: np.ndarray, cnt: np.ndarray) -> np.ndarray:
    """Step 4. q: decoded [B][R][H][128] float64. Returns out [B][R][H][128] float64."""
    B, R, H, _ = q.shape
    G = sel.shape[2]
    topk = sel.shape[3]
    q = np.ascontiguousarray(q, dtype=np.float64)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    cnt = np.ascontiguousarray(cnt, dtype=np.int32)
    out = np.zeros((B, R, H, DIM), dtype=np.float64)
    lib().ref_attention(batch.ref(), H, G, _ptr(q), float(sm_scale), k_cache.ref(), v_cache.ref(),
                        _ptr(sel), _ptr(cnt), topk, _ptr(out))
    return out


def decode_step(batch: OracleBatch, q_idx: np.ndarray, q: np.ndarray, sm_scale: float, idx_cache: OracleCache,
                k_cache: OracleCache, v_cache: OracleCache, topk: int = 16) -> dict:
    """Steps 1-4 in order; returns every intermediate."""
    ts = index_scores(batch, q_idx, idx_cache)
    bs = block_maxpool(batch, ts)
    sel, cnt = select(batch, bs, topk)
    out = attention(batch, q, sm_scale, k_cache, v_cache, sel, cnt)
    return {"token_scores": ts, "block_scores": bs, "sel": sel, "cnt": cnt, "out": out}
