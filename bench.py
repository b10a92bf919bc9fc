"""MSA decode benchmark on one MI355X: layer-steps/s and achieved HBM bandwidth.

Workload: one sparse layer at 128K mean context -- 32 requests, one query row
each, contexts uniform in 64K..192K tokens, NVFP4 K/V and index caches,
FP8 queries, 4 KV heads x 128, 32 query heads, top-16 of 128-token blocks,
random physical page order.  Inputs are seeded, synthetic N(0,1) rows drawn
on the device.

A step is one pass of the whole path over the batch: insert of the B*R new
tokens (NVFP4 quantisation into the pages), indexer score + block max-pool,
top-16 selection with the latest block kept, sparse attention (each
workgroup's waves merge their softmax states on chip).
Inputs sit in HBM before timing starts; the caches rotate over replicas so
that consecutive steps cannot serve the index scan from the 256 MB Infinity
Cache.

Prints one JSON line (rank 0, one GPU).
"""
from __future__ import annotations

import argparse
import hashlib
import json
from types import SimpleNamespace
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_F16_MFMA_TFLOPS = 2500.0  # MI355X dense FP16 matrix peak
METRIC = "MSA decode layer-steps/s + achieved HBM GB/s (% of peak), 128K ctx NVFP4 KV"
CONFIG_ID = 3  # the 128K-context batch the metric is quoted on


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(wl, sel, cnt):
    """Minimum bytes one step moves (per the method): the index of every
    context (72 B/token in NVFP4, 128 B in FP8), K+V of the selected tokens of
    each (request, group) (NVFP4 144 B/token: 64+8 B of K, 64+8 B of V; FP8
    256 B), queries, outputs, block table, and the insert of the new rows
    (FP32 in, quantised out).  A physical page is counted once however many
    requests (a shared prefix) or rows select it."""
    B, R = wl.B, wl.R
    row_b = 128 if wl.cache == "fp8" else 72  # one 128-dim row of one head
    L = wl.lengths.astype(np.int64)
    idx_tok = {}  # physical page -> tokens of it some request's context covers
    for b in range(B):
        npb = -(-int(L[b]) // 128)
        for j in range(npb):
            ph = int(wl.block_table[b, j])
            idx_tok[ph] = max(idx_tok.get(ph, 0), min(128, int(L[b]) - 128 * j))
    idx = sum(idx_tok.values()) * row_b
    kv_lim = {}  # (group, physical page) -> last token any selecting row sees
    p = L[:, None] - R + np.arange(R)[None, :]
    for b in range(B):
        for g in range(4):
            for r in range(R):
                for j in sel[b, r, g, : cnt[b, r, g]]:
                    j = int(j)
                    key = (g, int(wl.block_table[b, j]))
                    kv_lim[key] = max(kv_lim.get(key, -1), min(127, int(p[b, r]) - 128 * j))
    kv_tokens = sum(v + 1 for v in kv_lim.values())
    kv = kv_tokens * 2 * row_b
    q_bytes = B * R * 4 * 128 + B * R * 32 * 128  # FP8 index queries + queries
    out_bytes = B * R * 32 * 128 * 4
    P = wl.prefix_pages
    table = (P + B * (wl.max_pages - P)) * 4 + B * 4
    insert = B * R * (9 * 128 * 4 + 9 * row_b)  # FP32 rows in, quantised rows out
    return {"index": idx + B * R * 4 * 128 + table, "insert_index": idx + B * R * 4 * 128 + table + insert, "kv": kv,
            "total": idx + kv + q_bytes + out_bytes + table + insert, "kv_tokens": kv_tokens}


def cpu_baseline(wl, sample_reqs, min_seconds=10.0, last_rows=None):
    """The oracle (plain FP64 C, OpenMP over (request, row, group)) timed on a
    bounded sample of the same workload: all four steps for `sample_reqs`
    requests (with last_rows, only the last rows of each request's chunk: a
    shorter chunk at the same context), repeated until min_seconds of work;
    scaled to whole-batch steps/s by rows x context tokens (work is linear in
    both)."""
    import oracle as O
    import workload as W

    rows = np.asarray(sample_reqs)
    dt = O.FP8_E4M3 if wl.cache == "fp8" else O.NVFP4
    ci = O.OracleCache(dt, O.TOKEN_MAJOR, 1, wl.num_pages, wl.tensor_scale)
    ck = O.OracleCache(dt, O.TOKEN_MAJOR, 4, wl.num_pages, wl.tensor_scale)
    cv = O.OracleCache(dt, O.DIM_MAJOR, 4, wl.num_pages, wl.tensor_scale)
    if wl.prefix_tokens:
        xi, xk, xv = W.prefix_rows(wl)
        s = wl.slots(0, np.arange(wl.prefix_tokens, dtype=np.int64))
        ci.write(s, xi), ck.write(s, xk), cv.write(s, xv)
        del xi, xk, xv
    for b in rows:
        pos = wl.own_positions(int(b))
        xi, xk, xv = W.request_rows(wl, int(b))
        s = wl.slots(int(b), pos)
        ci.write(s, xi), ck.write(s, xk), cv.write(s, xv)
    qi32, q32 = W.queries(wl)
    R = wl.R if last_rows is None else min(last_rows, wl.R)
    qi32, q32 = np.ascontiguousarray(qi32[rows][:, wl.R - R:]), np.ascontiguousarray(q32[rows][:, wl.R - R:])
    qi = O.decode_queries(O.quantize_queries(qi32, wl.q_scale), O.FP8_E4M3, wl.q_scale)
    q = O.decode_queries(O.quantize_queries(q32, wl.q_scale), O.FP8_E4M3, wl.q_scale)
    bt = O.OracleBatch(wl.block_table[rows], wl.lengths[rows], R)
    reps, t0 = 0, time.perf_counter()
    while True:
        O.decode_step(bt, qi, q, wl.sm_scale, ci, ck, cv, wl.topk)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    per_sample = el / reps
    frac = (R * float(wl.lengths[rows].astype(np.int64).sum())) / (wl.R * float(wl.lengths.astype(np.int64).sum()))
    full_step = per_sample / frac
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    part = "" if R == wl.R else f", the last {R} of each chunk's {wl.R} rows"
    return {"value": 1.0 / full_step, "unit": "layer-steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(rows)} of {wl.B} requests ({int(wl.lengths[rows].sum())} of "
                      f"{int(wl.lengths.sum())} context tokens{part}), full step x{reps} in {el:.1f} s, "
                      f"scaled by rows x context tokens"}


QKV_HEADS = 45  # 32 query heads, 4 key, 4 value, 4 index queries, 1 index key
PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense BF16 matrix peak


def qkv_algorithmic(n, hidden):
    """(bytes, flops) of one fused projection + norm + RoPE + insert launch: weights and
    hidden states once, the rotary rows of n positions, FP8 queries and index queries out,
    72 B per token per NVFP4 head written (4 key, 4 value, 1 index-key head)."""
    nbytes = (QKV_HEADS * 128 * hidden * 2 + n * hidden * 2 + n * 128 * 4 + n * 36 * 128 + n * 9 * 72
              + 4 * 128 * 4 + n * 12)
    return nbytes, 2.0 * n * QKV_HEADS * 128 * hidden


def bench_qkv(args):
    """The fused projection of n new rows at model width `hidden` (the pages give no width;
    3,072 by default): HIP events around a graph of back-to-back launches."""
    import torch

    import block_sparse_attention_index_amd as M
    import workload as W

    n, hidden = args.qkv, args.hidden
    q = W.make_qkv_inputs(args.seed, n, hidden, max_pos=200_000, num_pages=max(1, -(-n // 128)) + 1)
    if n >= 512:  # a prompt chunk: consecutive slots
        q.slots = np.arange(n, dtype=np.int64) + 64
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x, w = dev(q.x.view(np.int16)), dev(W.pack_qkv_weights(q.w).view(np.int16))
    g, rope, pos, slots = dev(q.norm_weight), dev(q.rope), dev(q.positions), dev(q.slots)
    kc = M.Cache.empty(M.MSA_NVFP4, M.MSA_TOKEN_MAJOR, 4, q.num_pages, q.tensor_scale)
    vc = M.Cache.empty(M.MSA_NVFP4, M.MSA_DIM_MAJOR, 4, q.num_pages, q.tensor_scale)
    ic = M.Cache.empty(M.MSA_NVFP4, M.MSA_TOKEN_MAJOR, 1, q.num_pages, q.tensor_scale)
    q_out = torch.empty((n, 32, 128), dtype=torch.uint8, device="cuda")
    qi_out = torch.empty((n, 4, 128), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    hbm = n <= 256  # the weights dominate: a stream; else the products do
    # a few new rows: rotate over weight copies larger together than the 256 MB Infinity
    # Cache, as the layers of a model would, so that no launch finds its weights cached
    ws = [w] + [w.clone() for _ in range((8 if hbm else 1) - 1)]

    def launch(i):
        M.msa_qkv_project_insert(x, ws[i % len(ws)], g, q.eps, rope, pos, slots, q.q_scale, q_out, qi_out, kc, vc,
                                 ic, stream=stream)

    per_graph = 24
    reps = max(1, args.steps // per_graph)
    with torch.cuda.stream(stream):
        for i in range(max(1, args.warmup)):
            launch(i)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(per_graph):
                launch(i)
        graph.replay()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a_.record(stream)
        for _ in range(reps):
            graph.replay()
        b_.record(stream)
    torch.cuda.synchronize()
    us = a_.elapsed_time(b_) * 1e3 / (reps * per_graph)
    nbytes, flops = qkv_algorithmic(n, hidden)
    if hbm:
        roof = {"bound": "hbm", "kernel": "qkv_insert_kernel", "achieved": nbytes / us / 1e3, "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "bytes_per_launch": nbytes}
    else:
        roof = {"bound": "mfma", "kernel": "qkv_insert_kernel (v_mfma_f32_16x16x32_bf16)",
                "achieved": flops / us / 1e6, "peak": PEAK_BF16_MFMA_TFLOPS, "unit": "TFLOP/s",
                "flops_per_launch": flops}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["avg_launch_us"] = us
    roof["traffic"] = None
    log(f"qkv n={n} hidden={hidden}: {us:.1f} us per launch")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as O

        k = min(n, 16)
        reps_c, t0 = 0, time.perf_counter()
        while True:
            O.qkv_project(q.x[:k], q.w, q.norm_weight, q.eps, q.rope, q.positions[:k])
            reps_c += 1
            el = time.perf_counter() - t0
            if el >= 5.0:
                break
        cpu = {"value": k * reps_c / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"projection + norm + rotary of {k} of {n} tokens x{reps_c} in {el:.1f} s "
                         f"(quantisation not included)"}
    line = {"metric": "fused QKV projection + norm + RoPE + NVFP4 insert, tokens/s", "value": n / us * 1e6,
            "unit": "tokens/s", "n_gpus": 1, "steps": reps * per_graph, "warmup": args.warmup,
            "ms_per_step": us / 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "bf16 x bf16 (f32 accumulate) -> fp8 q, nvfp4 kv", "data": "synthetic N(0,1), seeded",
            "config": {"workload": f"qkv_project_insert_n{n}_hidden{hidden}", "tokens": n, "hidden": hidden,
                       "heads": "32 q + 4 k + 4 v + 4 index q + 1 index k, dim 128", "parallelism": "single-gpu",
                       "hip_graph": True, "launches_per_graph": per_graph, "weight_copies": len(ws)},
            "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(line), flush=True)


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "index_nvfp4_long_ctx_b32_64k_192k_hbm_traffic.md")
INDEX_KERNEL_SOURCES = ["include/msa.h", "block_sparse_attention_index_amd/csrc/msa_device.h",
                        "block_sparse_attention_index_amd/csrc/msa_scan.h",
                        "block_sparse_attention_index_amd/csrc/msa_index.hip"]


def recorded_traffic(key="insert-index-kernel-traffic-bytes-per-launch"):
    """HBM bytes per launch of the step's index kernel (with the insert fused in,
    or, by key, the plain scan; "owned-" keys: the physical-order scan) as the
    committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary records them
    (copy-kernel calibrated), or None when the summary is absent or the
    kernel's sources changed since it was taken."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None
    fields = dict(line.strip().split(": ", 1) for line in text.splitlines()
                  if "kernel-" in line and ": " in line and line.strip().split(":")[0].endswith(("sha256", "launch")))
    h = hashlib.sha256()
    for f in INDEX_KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("index-kernel-source-sha256") != h.hexdigest():
        return None
    return int(fields[key]) if key in fields else None


def setup(seed=0, n_replicas=2, config=CONFIG_ID, kv="nvfp4", scan="owner"):
    """Device state of the benchmark workload: filled caches (``n_replicas`` copies),
    decoders, the step's new rows and quantised queries.  scan="owner": the batch
    carries the owner map (decode batches without a shared prefix), which the
    index scan then reads in physical page order; "table": it walks the table rows."""
    import torch

    import block_sparse_attention_index_amd as M
    import workload as W
    from block_sparse_attention_index_amd.decoder import MsaDecoder, make_caches

    dev = torch.device("cuda:0")
    wl = W.make_workload(config, seed=seed, cache=kv)
    kv_dtype = M.MSA_FP8_E4M3 if kv == "fp8" else M.MSA_NVFP4
    log(f"workload {wl.name}: B={wl.B} R={wl.R} tokens={int(wl.lengths.sum())} pages={wl.num_pages}")

    # ---- caches (replica 0 filled by the insert kernel from device-drawn rows)
    k0, v0, i0 = make_caches(kv_dtype, wl.num_pages, wl.tensor_scale, dev)
    table = torch.from_numpy(wl.block_table).to(dev)
    lens = torch.from_numpy(wl.lengths).to(dev)
    batch = M.Batch(table, lens, wl.R, wl.prefix_pages)
    table_batch, owner_us = batch, None
    if scan == "owner" and not wl.prefix_pages and wl.R <= M.MSA_MAX_ROWS:
        # the block table's inverse, kept with the table (the step itself records the pages of
        # its new rows); built here once, its build time reported beside the step
        own = M.msa_page_owner(batch, wl.num_pages)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            M.msa_page_owner(batch, wl.num_pages, own)
        e1.record()
        torch.cuda.synchronize()
        owner_us = e0.elapsed_time(e1) * 1e3 / 10
        batch = M.Batch(table, lens, wl.R, wl.prefix_pages, page_owner=own)
    if wl.prefix_tokens:  # the shared prefix is written once, into the pages every request's table names
        xi, xk, xv = W.torch_rows(wl, 0, dev, prefix=True)
        slots = torch.from_numpy(wl.slots(0, np.arange(wl.prefix_tokens, dtype=np.int64))).to(dev)
        M.msa_kv_insert(xk, xv, xi, slots, k0, v0, i0)
        del xi, xk, xv
    for b in range(wl.B):
        pos = wl.own_positions(b)
        xi, xk, xv = W.torch_rows(wl, b, dev)
        slots = torch.from_numpy(wl.slots(b, pos)).to(dev)
        M.msa_kv_insert(xk, xv, xi, slots, k0, v0, i0)
        del xi, xk, xv
    torch.cuda.synchronize()
    replicas = [(k0, v0, i0)]
    for _ in range(n_replicas - 1):
        k, v, i = make_caches(kv_dtype, wl.num_pages, wl.tensor_scale, dev)
        k.pages.copy_(k0.pages), v.pages.copy_(v0.pages), i.pages.copy_(i0.pages)
        replicas.append((k, v, i))
    decs = [MsaDecoder(batch, k, v, i, wl.topk, dev) for (k, v, i) in replicas]
    for d in decs[1:]:  # share the output buffers: every replica computes the same step
        d.block_scores, d.sel, d.cnt, d.out, d.workspace = (decs[0].block_scores, decs[0].sel, decs[0].cnt,
                                                            decs[0].out, decs[0].workspace)

    # ---- step inputs: new rows of the R latest positions, FP8 queries
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 12345)
    n_new = wl.B * wl.R
    new_k = torch.randn((n_new, 4, 128), generator=gen, device=dev)
    new_v = torch.randn((n_new, 4, 128), generator=gen, device=dev)
    new_i = torch.randn((n_new, 128), generator=gen, device=dev)
    new_slots = torch.from_numpy(np.concatenate([wl.slots(b, wl.new_row_positions(b)) for b in range(wl.B)])).to(dev)
    qi32, q32 = W.queries(wl)
    q_idx = M.msa_quantize_e4m3(torch.from_numpy(qi32).to(dev), wl.q_scale)
    q = M.msa_quantize_e4m3(torch.from_numpy(q32).to(dev), wl.q_scale)
    new = (new_k, new_v, new_i, new_slots)
    torch.cuda.synchronize()

    return SimpleNamespace(torch=torch, M=M, W=W, wl=wl, decs=decs, q_idx=q_idx, q=q, new=new, batch=batch,
                           table_batch=table_batch, owner_us=owner_us)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--config", type=int, default=CONFIG_ID, choices=[2, 3, 4, 5, 6, 7],
                    help="workload: 3 = 32 requests at 64K-192K tokens (the default, the metric's own); "
                         "2 = 8 x 32K; 4 = 16 requests x 4 speculative rows; 5 = 64 requests sharing a "
                         "256K-token prefix; 6 = prefill, 4 prompts of 64K tokens whose last 2,048 form the chunk; "
                         "7 = 32 x 8K with top-64 (every block selected: the forced-dense traffic check)")
    ap.add_argument("--kv", choices=["nvfp4", "fp8"], default="nvfp4",
                    help="cache format of keys, values and index keys (default NVFP4, the metric's own)")
    ap.add_argument("--scan", choices=["owner", "table"], default="owner",
                    help="index scan order: physical page order from the block table's inverse (owner map; "
                         "NVFP4 decode without a shared prefix) or each request's table row")
    ap.add_argument("--replicas", type=int, default=2)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of HIP graph replays")
    ap.add_argument("--layers-per-graph", type=int, default=10,
                    help="layer-steps captured in one HIP graph, as one forward pass over that many sparse layers "
                         "captures them (replicas alternate as the layers' own caches); the largest divisor of "
                         "--steps not above this value is used")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=4, help="requests in the oracle's timed sample")
    ap.add_argument("--qkv", type=int, default=0, metavar="N",
                    help="instead of the step: the fused projection + norm + RoPE + insert of N new rows "
                         "(32 = the default workload's decode step, 8192 = the prefill chunk)")
    ap.add_argument("--hidden", type=int, default=3072, help="model width for --qkv (the pages give none)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the context-parallel indexer is a design, not code).", file=sys.stderr)
        sys.exit(2)

    if args.qkv:
        bench_qkv(args)
        return

    st = setup(args.seed, args.replicas, args.config, args.kv, args.scan)
    owned = st.batch.page_owner is not None
    headline = args.config == CONFIG_ID and args.kv == "nvfp4"
    torch, M, W, wl, decs, q_idx, q, new = st.torch, st.M, st.W, st.wl, st.decs, st.q_idx, st.q, st.new

    stream = torch.cuda.Stream()
    use_graph = not args.no_graph

    def run_step(i, s):
        decs[i % len(decs)].step(q_idx, q, wl.q_scale, wl.sm_scale, new_tokens=new, stream=s)

    # layer-steps per graph: the largest divisor of K not above the request, a multiple of the
    # replica count (so the replicas keep alternating across replays) unless it is 1
    per_graph = 1
    for d_ in range(min(args.layers_per_graph, args.steps), 0, -1):
        if args.steps % d_ == 0 and (d_ % len(decs) == 0 or d_ == 1):
            per_graph = d_
            break
    graph = None
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            run_step(i, stream)
        if use_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                for i in range(per_graph):
                    run_step(i, stream)
            graph.replay()  # untimed
    torch.cuda.synchronize()

    # ---- timed region: K whole steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    # an event after every replay (every step without graphs) gives the spread of step times
    marks = []
    with torch.cuda.stream(stream):
        t_start.record(stream)
        if use_graph:
            for _ in range(args.steps // per_graph):
                graph.replay()
                marks.append(torch.cuda.Event(enable_timing=True))
                marks[-1].record(stream)
        else:
            for i in range(args.steps):
                run_step(i, stream)
                marks.append(torch.cuda.Event(enable_timing=True))
                marks[-1].record(stream)
        t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    per = per_graph if use_graph else 1
    spans = [t_start.elapsed_time(marks[0])] + [a_.elapsed_time(b_) for a_, b_ in zip(marks[:-1], marks[1:])]
    step_us = np.array(spans) * 1e3 / per
    step_spread = {"p10": float(np.percentile(step_us, 10)), "median": float(np.median(step_us)),
                   "p90": float(np.percentile(step_us, 90)), "samples": len(spans), "steps_per_sample": per}
    log(f"timed {args.steps} steps ({per_graph} per graph): {ms_step * 1e3:.1f} us/step (events), "
        f"wall {wall / args.steps * 1e6:.1f} us/step")

    # ---- per-kernel durations: for each kernel, a HIP graph of `reps` back-to-back
    # launches (alternating cache replicas) replayed between two HIP events on
    # the launch stream; per-launch time = elapsed / (replays * reps)
    reps, replays = 20, max(1, args.steps // 20)
    calls = {
        "insert": lambda d: d.insert(*new, stream=stream),
        "index": lambda d: d.index(q_idx, wl.q_scale, None, stream),
        "insert_index": lambda d: d.insert_index(new[0], new[1], new[2], q_idx, wl.q_scale, None, stream),
        "topk": lambda d: d.select(stream),
        "decode": lambda d: d.attend(q, wl.q_scale, wl.sm_scale, stream),
        "select_decode": lambda d: d.select_attend(q, wl.q_scale, wl.sm_scale, stream),
    }
    prefill = wl.R > M.MSA_MAX_ROWS  # a prefill chunk: no fused insert; the indexer is the dense kernel
    if prefill:
        del calls["insert_index"]
    P = wl.prefix_pages
    if owned:  # the table-order scan on the same caches, for comparison
        from block_sparse_attention_index_amd.decoder import MsaDecoder

        tdec = {id(d): MsaDecoder(st.table_batch, d.k, d.v, d.idx, wl.topk) for d in decs}
        calls["index_table_order"] = lambda d: tdec[id(d)].index(q_idx, wl.q_scale, None, stream)
        calls["insert_index_table_order"] = lambda d: tdec[id(d)].insert_index(new[0], new[1], new[2], q_idx,
                                                                              wl.q_scale, None, stream)
    if P:
        # the prefix kernel alone: a batch whose table ends with the shared pages leaves the
        # per-request scan nothing to do
        from block_sparse_attention_index_amd.decoder import MsaDecoder

        pbatch = M.Batch(st.batch.block_table[:, :P].contiguous(), st.batch.ctx_lens, wl.R, P)
        pdec = {id(d): MsaDecoder(pbatch, d.k, d.v, d.idx, wl.topk) for d in decs}
        calls["prefix"] = lambda d: pdec[id(d)].index(q_idx, wl.q_scale, None, stream)
    us = {}
    for name, call in calls.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for i in range(reps):
                    call(decs[i % len(decs)])
            g.replay()
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            for _ in range(replays):
                g.replay()
            b_.record(stream)
        torch.cuda.synchronize()
        us[name] = a_.elapsed_time(b_) * 1e3 / (replays * reps)
    if owned:
        us["page_owner_build"] = st.owner_us
    log("per-kernel us (graph of back-to-back launches): " + ", ".join(f"{k} {v:.1f}" for k, v in us.items()))

    # ---- the practical HBM read ceiling in this process: a plain streaming read of as many
    # bytes as the index scan reads, with the scan's load form, alternating two buffers
    # (together larger than the 256 MB Infinity Cache), timed like the kernels above
    stream_ref = None
    if not prefill:
        nbytes_idx = algorithmic_bytes(wl, decs[0].sel.cpu().numpy(), decs[0].cnt.cpu().numpy())["index"]
        n16 = nbytes_idx // 16 * 16
        bufs = [torch.empty(n16, dtype=torch.uint8, device="cuda") for _ in range(2)]
        for b_ in bufs:
            b_.fill_(1)
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        # 65,535 workgroups were the best grid of a sweep over 310 MB (7.05 TB/s; 6.6 TB/s at 1,024);
        # a smaller read keeps at least 4 KB per workgroup (one 16-byte load per thread)
        wgs = int(min(65535, max(1024, n16 // 4096)))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for i in range(reps):
                    M.msa_debug_stream_read(bufs[i % 2], wgs, sink, stream)
            g.replay()
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            for _ in range(replays):
                g.replay()
            b_.record(stream)
        torch.cuda.synchronize()
        st_us = a_.elapsed_time(b_) * 1e3 / (replays * reps)
        stream_ref = {"kernel": f"stream_read_kernel (16-byte non-temporal loads, {wgs:,} workgroups)",
                      "bytes_per_launch": int(n16), "avg_launch_us": st_us, "achieved_GBps": n16 / st_us / 1e3}
        del bufs
        log(f"streaming read of {n16 / 1e6:.1f} MB: {st_us:.1f} us = {n16 / st_us / 1e3:.0f} GB/s")

    sel = decs[0].sel.cpu().numpy()
    cnt = decs[0].cnt.cpu().numpy()
    nbytes = algorithmic_bytes(wl, sel, cnt)
    steps_per_s = 1e3 / ms_step
    idx_key = "index" if prefill else "insert_index"
    idx_gbps = nbytes[idx_key] / (us[idx_key] * 1e-6) / 1e9
    # prefill: every page of a request against its R*4 index queries (full pages, masked or not)
    pages_scored = int(sum(-(-int(L) // 128) for L in wl.lengths))
    prefill_flops = 2 * 128 * 128 * pages_scored * wl.R * 4
    prefix_flops = 2 * 128 * 128 * P * wl.B * wl.R * 4  # dims x tokens x index queries
    step_gbps = nbytes["total"] / (ms_step * 1e-3) / 1e9
    if stream_ref is not None:
        stream_ref["index_scan_frac"] = (nbytes["index"] / (us["index"] * 1e-6) / 1e9) / stream_ref["achieved_GBps"]

    cpu = None
    if not args.no_cpu_baseline:
        rng = np.random.default_rng(args.seed)
        prefill_rows = 64 if wl.R > M.MSA_MAX_ROWS else None  # a prompt chunk: one request, its last rows
        n_sample = 1 if prefill_rows else min(args.cpu_sample, wl.B)
        sample = sorted(rng.choice(wl.B, size=n_sample, replace=False).tolist())
        log(f"cpu baseline: oracle on requests {sample}" + (f", last {prefill_rows} rows" if prefill_rows else ""))
        cpu = cpu_baseline(wl, sample, last_rows=prefill_rows)
        log(f"cpu baseline: {cpu['value']:.3f} steps/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC,
        "value": steps_per_s,
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8 kv x fp8 q (fp8xfp8 + f16 mfma, f32 accumulate)" if wl.cache == "fp8"
                  else "nvfp4 kv x fp8 q (fp8xfp4 + f16 mfma, f32 accumulate)"),
        "data": "synthetic N(0,1) rows, seeded, device-generated",
        "config": {"workload": wl.name, "global_batch": wl.B, "rows_per_req": wl.R,
                   "ctx_tokens_mean": float(wl.lengths.mean()), "ctx_tokens_min": int(wl.lengths.min()),
                   "ctx_tokens_max": int(wl.lengths.max()), "kv_cache": wl.cache, "index_cache": wl.cache,
                   "topk_blocks": wl.topk, "block_tokens": 128, "parallelism": "single-gpu",
                   "cache_replicas": len(decs), "hip_graph": use_graph,
                   "index_scan": "physical page order (owner map)" if owned else "block-table order",
                   "layer_steps_per_graph": per_graph if use_graph else None},
        "roofline": ({"bound": "mfma", "kernel": "prefill_index_kernel (dense indexer on v_mfma_f32_16x16x32_f16)",
                      "flops_per_launch": prefill_flops, "avg_launch_us": us["index"],
                      "achieved": prefill_flops / (us["index"] * 1e-6) / 1e12, "peak": PEAK_F16_MFMA_TFLOPS,
                      "unit": "TFLOP/s", "frac": prefill_flops / (us["index"] * 1e-6) / 1e12 / PEAK_F16_MFMA_TFLOPS,
                      "traffic": None, "index_GBps": idx_gbps} if prefill else
                     {"bound": "hbm", "scope": "dominant kernel, per launch (the whole step: step_hbm)",
                      "kernel": (f"index_{wl.cache}_owned_kernel" if owned else f"index_{wl.cache}_kernel")
                      + " with the insert fused in (steps 0-2)",
                      "achieved": idx_gbps,
                      "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": idx_gbps / PEAK_HBM_GBPS,
                      "traffic": recorded_traffic(("owned-" if owned else "") +
                                                  "insert-index-kernel-traffic-bytes-per-launch") if headline else None,
                      "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x 2 + WRITE_SIZE x 1, copy-calibrated)",
                      "bytes_per_launch": nbytes["insert_index"], "avg_launch_us": us["insert_index"],
                      "plain_scan": {"bytes_per_launch": nbytes["index"], "avg_launch_us": us["index"],
                                     "achieved": nbytes["index"] / (us["index"] * 1e-6) / 1e9,
                                     "traffic": recorded_traffic(("owned-" if owned else "") +
                                                                 "index-kernel-traffic-bytes-per-launch")
                                     if headline else None}}),
        "prefix_mfma": None if not P else {
            "kernel": "prefix_index_kernel (shared-prefix scores on v_mfma_f32_16x16x32_f16)",
            "bound": "mfma", "flops_per_launch": prefix_flops, "avg_launch_us": us["prefix"],
            "achieved": prefix_flops / (us["prefix"] * 1e-6) / 1e12, "peak": PEAK_F16_MFMA_TFLOPS,
            "unit": "TFLOP/s", "frac": prefix_flops / (us["prefix"] * 1e-6) / 1e12 / PEAK_F16_MFMA_TFLOPS},
        "step_hbm": {"scope": "whole step (insert, index, selection, attention) per layer-step",
                     "algorithmic_bytes": nbytes["total"], "achieved_GBps": step_gbps,
                     "frac_of_peak": step_gbps / PEAK_HBM_GBPS, "kv_tokens_read": nbytes["kv_tokens"]},
        "step_us": step_spread,
        "stream_read": stream_ref,
        "kernel_us": us,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
