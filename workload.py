"""Seeded synthetic inputs for the MSA decode step.

This module is shared by the tests, ``bench.py`` and ``smoke()``.  It feeds both
the HIP path and the CPU oracle, so it holds none of the method's arithmetic:
it draws FP32 key/value/index-key rows, FP32 queries, context lengths and page
tables, and nothing else.  Quantisation to NVFP4 / FP8 happens on each side
separately (the HIP insert and query kernels; the oracle's own quantiser).

Shapes follow the workloads the pages describe (one sparse layer of the
MiniMax-M3 family, [vLLM M3.1 post, "How MiniMax Sparse Attention works" and
"NVFP4 indexer DCP on CDNA4"]): 4 KV heads of dim 128, 8 query heads per GQA
group, one shared index-key head of dim 128, 128-token pages = selection
blocks, top-16.  The pages' own workloads (agentic traces, "45 requests of
30K-210K tokens") are not available; these seeded N(0,1) caches stand in for
them and take only their shapes.

Draw order is fixed: lengths -> physical page permutation -> per-request
token rows (one stream per request, idx then K then V) -> queries (q_idx then q).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE = 128
DIM = 128
G = 4  # KV heads = GQA groups
HPG = 8  # query heads per group
H = G * HPG
TOPK = 16
# NVFP4 per-tensor FP32 scale for N(0,1) rows: amax bound 8 over (E2M1 max 6 x E4M3 max 448).
NVFP4_TENSOR_SCALE = float(np.float32(8.0 / (6.0 * 448.0)))
# FP8 (E4M3 per element) per-tensor FP32 scale for N(0,1) rows: amax bound 8 over E4M3 max 448.
FP8_TENSOR_SCALE = float(np.float32(8.0 / 448.0))
SM_SCALE = float(np.float32(1.0 / np.sqrt(DIM)))

CONFIGS = {
    1: dict(name="tiny_f32_4k", B=1, R=1, lens=("fixed", 4096), cache="f32", table="contiguous"),
    2: dict(name="nvfp4_b8_32k", B=8, R=1, lens=("fixed", 32768), cache="nvfp4", table="shuffled"),
    3: dict(name="long_ctx_b32_64k_192k", B=32, R=1, lens=("uniform", 65536, 196608), cache="nvfp4",
            table="shuffled"),
    4: dict(name="spec_r4_b16_30k_210k", B=16, R=4, lens=("uniform", 30720, 215040), cache="nvfp4",
            table="shuffled"),
    5: dict(name="shared_prefix_b64_256k", B=64, R=1, lens=("uniform", 1024, 8192), prefix=262144,
            cache="nvfp4", table="shuffled"),
    # prefill: the last 2,048 tokens of 64K-token prompts scored, selected and attended as one chunk
    6: dict(name="prefill_b4_2k_chunk_64k", B=4, R=2048, lens=("fixed", 65536), cache="nvfp4", table="shuffled"),
    # a measurement aid, not a workload of the pages: every block selected (64 blocks, top-64), so the
    # attention reads the whole K/V and its traffic can be set against the index scan's (8:1 by bytes)
    7: dict(name="forced_dense_b32_8k_top64", B=32, R=1, lens=("fixed", 8192), cache="nvfp4", table="shuffled",
            topk=64),
}


@dataclass
class Workload:
    name: str
    seed: int
    B: int
    R: int
    cache: str  # "f32" | "nvfp4" | "fp8"
    lengths: np.ndarray  # [B] int32, tokens in cache incl. the R new rows
    block_table: np.ndarray  # [B][max_pages] int32 physical page ids (unused tail = 0)
    num_pages: int
    prefix_tokens: int = 0  # leading tokens shared by every request (same pages)
    topk: int = TOPK
    G: int = G
    H: int = H
    D: int = DIM
    tensor_scale: float = 1.0
    q_scale: float = 1.0
    sm_scale: float = SM_SCALE
    extra: dict = field(default_factory=dict)

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def prefix_pages(self) -> int:
        return self.prefix_tokens // PAGE

    def own_positions(self, b: int) -> np.ndarray:
        """Positions whose rows belong to request b alone (the prefix is written once)."""
        return np.arange(self.prefix_tokens, int(self.lengths[b]), dtype=np.int64)

    def slots(self, b: int, positions: np.ndarray) -> np.ndarray:
        """Slot (physical page * 128 + offset) of request b's token positions."""
        positions = np.asarray(positions, dtype=np.int64)
        return self.block_table[b, positions // PAGE].astype(np.int64) * PAGE + positions % PAGE

    def new_row_positions(self, b: int) -> np.ndarray:
        L = int(self.lengths[b])
        return np.arange(max(L - self.R, 0), L, dtype=np.int64)


def make_workload(config: int, seed: int = 0, B: int | None = None, len_div: int = 1,
                  lengths: list[int] | None = None, R: int | None = None, cache: str | None = None,
                  topk: int = TOPK, table_width: int | None = None, spare_pages: int = 0) -> Workload:
    """Build the shapes of a configuration.  ``B``/``len_div`` shrink it for
    parity tests; ``lengths`` overrides the drawn lengths (edge cases);
    ``cache`` = "fp8" stores the same shapes in FP8 caches instead of NVFP4;
    ``topk`` sets the selected blocks per row; ``table_width`` pads the block
    table with unused columns (page 0) up to that many entries per request;
    ``spare_pages`` adds that many pages no request uses to the pool (scattered
    among the used ones when the table is permuted)."""
    cfg = CONFIGS[config]
    rng = np.random.default_rng([seed, 0])
    B = cfg["B"] if B is None else B
    R = cfg["R"] if R is None else R
    kind = cfg["lens"]
    if lengths is not None:
        lens = np.asarray(lengths, dtype=np.int64)
        B = lens.shape[0]
    elif kind[0] == "fixed":
        lens = np.full(B, kind[1], dtype=np.int64)
    else:
        lens = rng.integers(kind[1], kind[2], size=B, endpoint=True).astype(np.int64)
    prefix = cfg.get("prefix", 0)
    if len_div > 1:
        lens = np.maximum(lens // len_div, 1 if lengths is None else 0)
        prefix = (prefix // len_div) // PAGE * PAGE
    if lengths is None:
        lens = lens + prefix
    prefix_pages = prefix // PAGE
    own_pages = [max(0, -(-int(L) // PAGE) - prefix_pages) for L in lens]
    max_pages = max(1, max(prefix_pages + n for n in own_pages))
    num_pages = prefix_pages + sum(own_pages)
    num_pages = max(num_pages, 1) + spare_pages
    if cfg["table"] == "contiguous":
        perm = np.arange(num_pages, dtype=np.int64)
    else:
        perm = rng.permutation(num_pages)
    if table_width is not None:
        assert table_width >= max_pages
        max_pages = table_width
    table = np.zeros((B, max_pages), dtype=np.int32)
    nxt = prefix_pages
    for b in range(B):
        table[b, :prefix_pages] = perm[:prefix_pages]
        n = own_pages[b]
        table[b, prefix_pages:prefix_pages + n] = perm[nxt:nxt + n]
        nxt += n
    topk = cfg.get("topk", topk)
    kind = cfg["cache"] if cache is None else cache
    assert kind in ("f32", "nvfp4", "fp8")
    ts = {"nvfp4": NVFP4_TENSOR_SCALE, "fp8": FP8_TENSOR_SCALE, "f32": 1.0}[kind]
    name = cfg["name"] if kind == cfg["cache"] else f'{cfg["name"]}_{kind}'
    return Workload(name=name, seed=seed, B=B, R=R, cache=kind, lengths=lens.astype(np.int32),
                    block_table=table, num_pages=int(num_pages), prefix_tokens=int(prefix), topk=topk,
                    tensor_scale=ts)


def request_rows(wl: Workload, b: int):
    """FP32 N(0,1) rows for request b's own positions: (idx [n][128], k [n][G][128], v [n][G][128])."""
    n = wl.own_positions(b).shape[0]
    rng = np.random.default_rng([wl.seed, 1, b])
    idx = rng.standard_normal((n, wl.D), dtype=np.float32)
    k = rng.standard_normal((n, wl.G, wl.D), dtype=np.float32)
    v = rng.standard_normal((n, wl.G, wl.D), dtype=np.float32)
    return idx, k, v


def prefix_rows(wl: Workload):
    """FP32 N(0,1) rows of the shared prefix (written once, into the shared pages)."""
    n = wl.prefix_tokens
    rng = np.random.default_rng([wl.seed, 2])
    idx = rng.standard_normal((n, wl.D), dtype=np.float32)
    k = rng.standard_normal((n, wl.G, wl.D), dtype=np.float32)
    v = rng.standard_normal((n, wl.G, wl.D), dtype=np.float32)
    return idx, k, v


def queries(wl: Workload):
    """FP32 N(0,1) queries: (q_idx [B][R][G][128], q [B][R][H][128])."""
    rng = np.random.default_rng([wl.seed, 3])
    q_idx = rng.standard_normal((wl.B, wl.R, wl.G, wl.D), dtype=np.float32)
    q = rng.standard_normal((wl.B, wl.R, wl.H, wl.D), dtype=np.float32)
    return q_idx, q


def all_rows(wl: Workload):
    """Every cached row once, with its slot: (slots [n], idx [n][128], k [n][G][128], v [n][G][128])."""
    parts = []
    if wl.prefix_tokens:
        pos = np.arange(wl.prefix_tokens, dtype=np.int64)
        parts.append((wl.slots(0, pos),) + prefix_rows(wl))
    for b in range(wl.B):
        pos = wl.own_positions(b)
        if pos.shape[0]:
            parts.append((wl.slots(b, pos),) + request_rows(wl, b))
    if not parts:
        z = np.zeros((0,), np.int64)
        return z, np.zeros((0, wl.D), np.float32), np.zeros((0, wl.G, wl.D), np.float32), \
            np.zeros((0, wl.G, wl.D), np.float32)
    return tuple(np.concatenate([p[i] for p in parts]) for i in range(4))


def torch_rows(wl: Workload, b: int, device, prefix: bool = False):
    """Device-side draw of the same shapes (for the benchmark's large caches).
    Seeded, N(0,1), but a different stream from the numpy one."""
    import torch

    n = wl.prefix_tokens if prefix else wl.own_positions(b).shape[0]
    gen = torch.Generator(device=device)
    gen.manual_seed((wl.seed * 1_000_003 + (0 if prefix else b + 1)) & 0x7FFFFFFF)
    idx = torch.randn((n, wl.D), generator=gen, device=device, dtype=torch.float32)
    k = torch.randn((n, wl.G, wl.D), generator=gen, device=device, dtype=torch.float32)
    v = torch.randn((n, wl.G, wl.D), generator=gen, device=device, dtype=torch.float32)
    return idx, k, v


# --------------------------------------------------------------------------- projection inputs
QKV_HEADS = 45  # query heads 0..31, key heads 32..35, value heads 36..39, index queries 40..43, index key 44
ROPE_THETA = 10000.0  # rotary base of the synthetic cos/sin table (the pages give none)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """FP32 values -> BF16 bit patterns, round to nearest even: how the synthetic hidden
    states and weights are drawn as BF16 numbers."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


@dataclass
class QkvInputs:
    x: np.ndarray            # [n][hidden] BF16 bits (uint16): hidden states of the step's new rows
    w: np.ndarray            # [45*128][hidden] BF16 bits: projection weights, row c -> column c
    norm_weight: np.ndarray  # [4][128] FP32: queries, keys, index queries, index key
    rope: np.ndarray         # [rows][128] FP32: cos of the 64 frequencies, then sin
    positions: np.ndarray    # [n] int32
    slots: np.ndarray        # [n] int64
    num_pages: int
    eps: float = 1e-6
    q_scale: float = 1.0
    tensor_scale: float = 4.5 / (6 * 448)  # |normalised values| and |projected values| stay below ~4.5


def pack_qkv_weights(w: np.ndarray) -> np.ndarray:
    """[45*128][hidden] -> the library's 32-k blocked layout [45][hidden/32][128][32] (a
    permutation of the BF16 words, done once per model)."""
    rows, hidden = w.shape
    return np.ascontiguousarray(w.reshape(QKV_HEADS, DIM, hidden // 32, 32).transpose(0, 2, 1, 3))


def rope_table(rows: int) -> np.ndarray:
    """cos/sin of position x theta^(-2i/128), i < 64, computed in float64, stored FP32."""
    inv = ROPE_THETA ** (-np.arange(64, dtype=np.float64) * 2.0 / DIM)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def make_qkv_inputs(seed: int, n: int, hidden: int, max_pos: int = 4096, num_pages: int | None = None,
                    bad_positions: int = 0, bad_slots: int = 0) -> QkvInputs:
    """Seeded inputs of the fused projection: x ~ N(0,1), w ~ N(0, 1/hidden) (projected values
    ~ N(0,1)), norm weights 1 + 0.1 N(0,1), positions uniform in [0, max_pos), distinct slots
    drawn from the page pool; the first `bad_positions` tokens get a position past the table
    and the next `bad_slots` tokens a slot outside the pool."""
    rng = np.random.default_rng([seed, 7])
    x = bf16_bits(rng.standard_normal((n, hidden), dtype=np.float32))
    w = bf16_bits(rng.standard_normal((QKV_HEADS * DIM, hidden), dtype=np.float32) / np.float32(np.sqrt(hidden)))
    g = (1.0 + 0.1 * rng.standard_normal((4, DIM))).astype(np.float32)
    pos = rng.integers(0, max_pos, size=n).astype(np.int32)
    if num_pages is None:
        num_pages = max(1, -(-2 * n // PAGE))
    slots = rng.permutation(num_pages * PAGE)[:n].astype(np.int64)
    pos[:bad_positions] = max_pos + np.arange(bad_positions, dtype=np.int32)
    slots[bad_positions:bad_positions + bad_slots] = np.where(np.arange(bad_slots) % 2 == 0, -1,
                                                              num_pages * PAGE + np.arange(bad_slots))
    return QkvInputs(x=x, w=w, norm_weight=g, rope=rope_table(max_pos), positions=pos, slots=slots,
                     num_pages=num_pages)
