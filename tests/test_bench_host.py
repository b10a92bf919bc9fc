"""Host-side checks of bench.py (no GPU): its refusal of several GPUs and its
algorithmic byte count on hand-made batches."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def _wl(lengths, table, cache="nvfp4", R=1, prefix_pages=0):
    table = np.asarray(table, np.int32)
    return SimpleNamespace(B=len(lengths), R=R, lengths=np.asarray(lengths, np.int32), block_table=table,
                           cache=cache, prefix_pages=prefix_pages, max_pages=table.shape[1])


def test_algorithmic_bytes_by_hand():
    """Two requests, one row each: 130 and 256 tokens on pages [0, 1] and [2, 3].
    Every group of request 0 selects blocks 0 and 1 (130 visible tokens), every
    group of request 1 selects block 1 only (its 128 tokens)."""
    wl = _wl([130, 256], [[0, 1], [2, 3]])
    sel = np.full((2, 1, 4, 16), -1, np.int32)
    cnt = np.zeros((2, 1, 4), np.int32)
    sel[0, 0, :, :2] = [0, 1]
    cnt[0, 0, :] = 2
    sel[1, 0, :, 0] = 1
    cnt[1, 0, :] = 1
    got = bench.algorithmic_bytes(wl, sel, cnt)
    index = (130 + 256) * 72
    kv_tokens = 4 * 130 + 4 * 128
    table = 2 * 2 * 4 + 2 * 4  # block table + context lengths
    queries = 2 * 4 * 128 + 2 * 32 * 128  # FP8 index queries and queries
    out = 2 * 32 * 128 * 4
    insert = 2 * (9 * 128 * 4 + 9 * 72)  # FP32 rows in, NVFP4 rows out
    assert got["kv_tokens"] == kv_tokens
    assert got["kv"] == kv_tokens * 144
    assert got["index"] == index + 2 * 4 * 128 + table
    assert got["total"] == index + kv_tokens * 144 + queries + out + table + insert


def test_algorithmic_bytes_count_a_shared_page_once():
    """Both requests name physical page 5 as their block 0 (a shared prefix of one
    page): its index bytes and its K/V bytes count once, with the widest visibility."""
    wl = _wl([200, 140], [[5, 1], [5, 2]], prefix_pages=1)
    sel = np.full((2, 1, 4, 16), -1, np.int32)
    cnt = np.full((2, 1, 4), 2, np.int32)
    sel[:, 0, :, :2] = [0, 1]
    got = bench.algorithmic_bytes(wl, sel, cnt)
    # index: page 5 (128 tokens, once), page 1 (72 tokens), page 2 (12 tokens)
    assert got["index"] - (2 * 4 * 128 + (1 + 2 * 1) * 4 + 2 * 4) == (128 + 72 + 12) * 72
    # K/V per group: page 5 once (128), page 1 (72), page 2 (12)
    assert got["kv_tokens"] == 4 * (128 + 72 + 12)


def test_algorithmic_bytes_fp8_rows():
    wl = _wl([256], [[0, 1]], cache="fp8")
    sel = np.full((1, 1, 4, 16), -1, np.int32)
    sel[0, 0, :, :2] = [0, 1]
    cnt = np.full((1, 1, 4), 2, np.int32)
    got = bench.algorithmic_bytes(wl, sel, cnt)
    assert got["kv"] == 4 * 256 * 2 * 128
    assert got["index"] == 256 * 128 + 4 * 128 + 2 * 4 + 4
