#!/usr/bin/env python3
"""CSA + HCA decode benchmark on one MI355X (gfx950).

One step = one pass of the whole decode hot path over one batch: indexer
scoring, exact top-k, CSA sparse attention over the top-k pooled rows plus the
sliding window, and HCA dense attention, for every sequence's query at
position T-1.  By default the step is the single-launch csa_hca_decode call;
--path separate times csa_index_topk + csa_sparse_attn + hca_attn instead.
Pooled caches are built once with csa_compress before timing (its throughput
is reported apart).  --copy-calibration runs only a 1 GiB device copy, the
scale reference for the HBM byte counters.

Default workload: 4 sequences x 1,048,576 tokens, 64 query heads on one bf16
KV head, d = 128, m = 4 (262,144 pooled entries), top-k 1024, window 128,
m' = 128 (8192 entries), indexer 4 heads x 64 in MXFP4.  Inputs are seeded
synthetic data already resident in HBM; R input sets are rotated so that
consecutive steps do not hit the 256 MB Infinity Cache.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

T0 = time.time()
METRIC = "CSA+HCA decode queries/s & HBM GB/s at 1M ctx; prefill indexer TFLOP/s"
HBM_PEAK_GBS = 8000.0
FP4_PEAK_TFLOPS = 10100.0


def log(msg: str):
    print(f"[bench {time.time() - T0:7.1f}s] {msg}", file=sys.stderr, flush=True)


def decode_bytes_per_query(n_vis, k, W, L, n_hvis, H, d, es):
    """Algorithmic HBM bytes of one decode query: indexer keys + scales, the
    gathered pooled rows, the window rows, the HCA rows, q and out for both
    branches, the indices, and the indexer query codes, scales and weights."""
    k_eff = min(k, n_vis)
    return (34 * n_vis + k_eff * 2 * d * es + min(W, L) * 2 * d * es + n_hvis * 2 * d * es
            + 4 * H * d * es + 4 * k + (4 * 34 + 4 * 4))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_b4_t1m")
    ap.add_argument("--rotate", type=int, default=20, help="input sets cycled through the timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-shared", action="store_true", help="skip the shared-prefix decode section")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a captured HIP graph")
    ap.add_argument("--path", choices=["fused", "separate"], default="fused",
                    help="fused: one csa_hca_decode launch per step; separate: csa_index_topk + csa_sparse_attn + hca_attn")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time the prefill indexer (4096 queries over a 65,536-token cache) and print its record")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device-to-device copy of known size (the HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (a decode batch would "
              "shard by sequence, with no exchange between GPUs). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import long_context_compressed_05_amd as csa
    from long_context_compressed_05_amd.step import Layer, Params, to_device

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    if args.copy_calibration:
        copy_calibration(torch)
        return
    csa.lib()
    dev = "cuda"
    torch.cuda.init()
    if args.prefill_only:
        print(json.dumps({"prefill_indexer": bench_prefill_indexer(torch, csa, synth, to_device, log)}), flush=True)
        return

    wl = synth.WORKLOADS[args.workload]()
    log(f"workload {wl.name}: B={wl.B} max_len={max(wl.lengths)} n_q={wl.n_q}; generating inputs")
    host = synth.make_inputs(wl)
    es = 2 if wl.dtype == "bf16" else 4
    p = Params(H=wl.H, d=wl.d, m=wl.m, k=wl.k, W=wl.W, m_hca=wl.m_hca, W_hca=wl.W_hca)
    layer = Layer.from_host(p, host, dev)
    log("inputs resident on the GPU; building pooled caches")

    # ---- compress (cache build), timed apart ----------------------------------
    n_pool, n_hpool = int(host["pool_off"][-1]), int(host["hpool_off"][-1])
    layer.pooled = torch.empty((n_pool, 2, wl.d), dtype=layer.kv.dtype, device=dev)
    layer.hpooled = torch.empty((n_hpool, 2, wl.d), dtype=layer.kv.dtype, device=dev)
    compress = {}
    for name, m, off, out in (("csa", wl.m, layer.pool_off, layer.pooled), ("hca", wl.m_hca, layer.hpool_off, layer.hpooled)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        csa.csa_compress(layer.kv, layer.z, layer.tok_off, off, layer.batch.max_len, m, out)  # warm
        torch.cuda.synchronize()
        e0.record()
        csa.csa_compress(layer.kv, layer.z, layer.tok_off, off, layer.batch.max_len, m, out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        rows = sum((L // m) * m for L in wl.lengths)
        nbytes = 2 * rows * 2 * wl.d * es + (rows // m) * 2 * wl.d * es
        compress[name] = {"m": m, "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1)}
    log(f"compress: {compress}")

    # ---- rotation sets ---------------------------------------------------------
    R = max(1, args.rotate)
    sets = []
    P_tot = int(host["pool_off"][-1])
    for r in range(R):
        if r == 0:
            hs = {k: host[k] for k in ("q", "qc", "qs", "w", "kc", "ks")}
        else:
            s = wl.seed + 7919 * r
            hs = {
                "q": synth.normal(s, synth.S_Q, wl.n_q * wl.H * wl.d, wl.dtype).reshape(wl.n_q, wl.H, wl.d),
                "qc": synth.codes4(s, synth.S_QCODE, wl.n_q * 128, wl.codeset).reshape(wl.n_q, 4, 32),
                "qs": synth.exp_bytes(s, synth.S_QSCALE, wl.n_q * 8, *wl.scale_exp).reshape(wl.n_q, 4, 2),
                "w": synth.pow2(s, synth.S_W, wl.n_q * 4, *wl.w_exp).reshape(wl.n_q, 4),
                "kc": synth.codes4(s, synth.S_KCODE, P_tot * 32, wl.codeset).reshape(P_tot, 32),
                "ks": synth.exp_bytes(s, synth.S_KSCALE, P_tot * 2, *wl.scale_exp).reshape(P_tot, 2),
            }
        d = to_device(hs, dev)
        d["hpooled"] = layer.hpooled if r == 0 else layer.hpooled.clone()
        d["idx"] = torch.empty((wl.n_q, wl.k), dtype=torch.int32, device=dev)
        d["co"] = torch.empty((wl.n_q, wl.H, wl.d), dtype=layer.kv.dtype, device=dev)
        d["cl"] = torch.empty((wl.n_q, wl.H), dtype=torch.float32, device=dev)
        d["ho"] = torch.empty_like(d["co"])
        d["hl"] = torch.empty_like(d["cl"])
        sets.append(d)
    log(f"{R} rotation sets resident")

    batch = layer.batch
    scale = 1.0 / math.sqrt(wl.d)

    def step_fused(r):
        d = sets[r % R]
        layer.decode_fused(d["q"], d["qc"], d["qs"], d["w"], idx=d["idx"], csa_out=d["co"], csa_lse=d["cl"],
                           hca_out=d["ho"], hca_lse=d["hl"], kc=d["kc"], ks=d["ks"], hpooled=d["hpooled"])

    def step_separate(r):
        d = sets[r % R]
        csa.csa_index_topk(batch, layer.pool_off, layer.max_pool, wl.m, wl.k, d["qc"], d["qs"], d["w"], d["kc"],
                           d["ks"], idx=d["idx"], ws=layer.ws_idx)
        csa.csa_sparse_attn(batch, layer.pool_off, d["q"], layer.pooled, layer.kv, d["idx"], wl.W, scale,
                            out=d["co"], lse=d["cl"], ws=layer.ws_csa)
        csa.hca_attn(batch, layer.hpool_off, layer.max_hpool, wl.m_hca, d["q"], d["hpooled"], layer.kv, wl.W_hca,
                     scale, out=d["ho"], lse=d["hl"], ws=layer.ws_hca)

    step = step_fused if args.path == "fused" else step_separate
    # the kernel whose duration is the roofline figure: the fused step kernel, or the indexer scoring kernel
    prof_id = csa.CSA_K_FUSED if args.path == "fused" else csa.CSA_K_IDX_SCORE
    prof_name = "k_decode_fused" if args.path == "fused" else "k_idx_score"

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done; timing {args.steps} steps")

    K = args.steps
    # dominant kernel: HIP events around every launch of the indexer scoring kernel
    # (eager steps, same inputs and rotation)
    ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        csa.csa_profile_events(prof_id, ev[i][0], ev[i][1])
        step(i)
    torch.cuda.synchronize()
    csa.csa_profile_events(prof_id)
    if args.path == "fused":
        layer.check_fused()
    score_ms = float(np.mean([a.elapsed_ms(b) for a, b in ev]))

    graph = None
    if not args.eager:
        try:
            graph = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap):
                with torch.cuda.graph(graph, stream=cap):
                    for r in range(R):
                        step(r)
            torch.cuda.current_stream().wait_stream(cap)
            for _ in range(max(1, args.warmup // R)):
                graph.replay()
            torch.cuda.synchronize()
        except Exception as e:
            log(f"graph capture unavailable ({e!r}); timing eager launches")
            graph = None
    reps = max(1, K // R) if graph is not None else K
    t_start, t_stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    if graph is not None:
        for _ in range(reps):
            graph.replay()
    else:
        for i in range(K):
            step(i)
    t_stop.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_stop)
    K = reps * R if graph is not None else K
    ms_step = total_ms / K
    if args.path == "fused":
        layer.check_fused()
    log(f"timed ({'graph' if graph is not None else 'eager'}, {args.path}): {ms_step * 1e3:.2f} us/step; "
        f"profiled kernel {score_ms * 1e3:.2f} us/launch")

    # algorithmic bytes
    m_, mh = wl.m, wl.m_hca
    q_pos = host["q_pos"]
    q_seq = np.repeat(np.arange(wl.B), np.diff(host["q_off"]))
    P_b = np.diff(host["pool_off"])
    Ph_b = np.diff(host["hpool_off"])
    step_bytes = 0
    score_bytes = 0
    for i in range(wl.n_q):
        b = q_seq[i]
        t = int(q_pos[i])
        n_vis = min((t + 1) // m_, int(P_b[b]))
        n_hvis = min((t + 1) // mh, int(Ph_b[b]))
        step_bytes += decode_bytes_per_query(n_vis, wl.k, wl.W, t + 1, n_hvis, wl.H, wl.d, es)
        score_bytes += 34 * n_vis + 4 * 34 + 4 * 4
    qps = wl.n_q / (ms_step * 1e-3)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    kernel_bytes = step_bytes if args.path == "fused" else score_bytes
    achieved = kernel_bytes / (score_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(qps, 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {**wl.describe(), "indexer": "mxfp4 4x64", "rotate_sets": R, "path": args.path,
                   "timing": "hip graph of the rotated steps, replayed" if graph is not None else "eager launches"},
        "hbm_gbps": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "step_bytes": int(step_bytes),
        "roofline": {"bound": "hbm", "kernel": prof_name,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": counted_traffic(prof_name, wl.name),
                     "bytes_per_launch": int(kernel_bytes), "avg_launch_us": round(score_ms * 1e3, 3)},
        "compress": compress,
    }

    # ---- streaming cache upkeep (appends at the end of the 1M-token caches) -----
    try:
        result["cache_append"] = bench_cache_append(torch, csa, layer, wl, host, log)
    except Exception as e:  # reported, never silently replaced
        result["cache_append"] = {"error": repr(e)}

    # ---- MXFP4 quantiser and the recall of the FP4 indexer's top-k -------------
    try:
        result["mxfp4_indexer"] = bench_mxfp4_recall(torch, csa, log)
    except Exception as e:  # reported, never silently replaced
        result["mxfp4_indexer"] = {"error": repr(e)}

    # ---- shared-prefix decode: 4 questions over one ~1M-token document ----------
    if args.workload == "decode_b4_t1m" and args.path == "fused" and not args.no_shared:
        try:
            result["shared_prefix"] = bench_shared_prefix(torch, csa, synth, to_device, log, score_ms)
        except Exception as e:  # reported, never silently replaced
            result["shared_prefix"] = {"error": repr(e)}
        try:
            result["paged"] = bench_paged(torch, csa, layer, wl, host, sets, log, score_ms)
        except Exception as e:  # reported, never silently replaced
            result["paged"] = {"error": repr(e)}

    # ---- prefill indexer (4096-token chunk on a 64K cache) ----------------------
    if not args.no_prefill:
        try:
            result["prefill_indexer"] = bench_prefill_indexer(torch, csa, synth, to_device, log)
        except Exception as e:  # reported, never silently replaced
            result["prefill_indexer"] = {"error": repr(e)}

    # ---- CPU oracle baseline --------------------------------------------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, host, log)

    print(json.dumps(result), flush=True)


COPY_BYTES = 1 << 30
# the device sources each kernel is built from: a stored counter reading is
# used only while these are unchanged
KERNEL_SOURCES = {
    "k_decode_fused": ["k_fused.hip", "attn_core.hpp", "common.hpp", "kernels.hpp", "select_core.hpp"],
    "k_idx_score": ["k_index.hip", "common.hpp", "kernels.hpp", "select_core.hpp"],
}


def copy_calibration(torch):
    """A plain device copy of COPY_BYTES: under rocprofv3 --pmc its FETCH_SIZE
    and WRITE_SIZE readings give the counters' scale (reads = writes = COPY_BYTES)."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}), flush=True)


def kernel_source_digest(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_compressed_05_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, f)) as fh:
            # whole-line comments and blank lines do not change the kernel
            for line in fh:
                t = line.strip()
                if t and not t.startswith("//"):
                    h.update(line.rstrip().encode())
                    h.update(b"\n")
    return h.hexdigest()


def counted_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by the
    copy-kernel calibration), or None when there is none or the kernel's
    sources changed since the counters were taken."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic-json: "):
                rec = json.loads(line[len("traffic-json: "):])
                if rec.get("source_sha256") != kernel_source_digest(kernel):
                    return None
                return int(rec["traffic_bytes_per_launch"])
    return None


def bench_cache_append(torch, csa, layer, wl, host, log, reps: int = 50):
    """csa_cache_append at the end of the resident 1M-token caches: (a) one
    decode step, one new token for each of the 4 sequences, each completing a
    CSA and an HCA block; (b) a 4096-token chunk on one sequence.  The appended
    rows are the caches' own last rows, so every call rewrites identical data;
    lengths and tail rings are reset between calls, outside the timed region
    (HIP events around the call's two kernels, on their stream)."""
    dev = "cuda"
    B, L = wl.B, np.array(wl.lengths, dtype=np.int64)
    tok_off = host["tok_off"]
    ring = wl.m_hca
    es = 2 if wl.dtype == "bf16" else 4
    row = 2 * wl.d * es
    cases = {"decode_step": np.ones(B, dtype=np.int64),
             "prefill_chunk": np.array([4096] + [0] * (B - 1), dtype=np.int64)}
    out = {}
    for name, n in cases.items():
        L0 = L - n
        rows = np.concatenate([np.arange(tok_off[b] + L0[b], tok_off[b] + L[b]) for b in range(B)]).astype(np.int64)
        r = torch.from_numpy(rows).to(dev)
        x_new, z_new = layer.kv[r].contiguous(), layer.z[r].contiguous()
        new_off = torch.from_numpy(np.concatenate([[0], np.cumsum(n)]).astype(np.int64)).to(dev)
        tail_rows = np.array([[tok_off[b] + (p if p >= 0 else 0) for p in
                               [L0[b] - ring + ((s - (L0[b] - ring)) % ring) for s in range(ring)]]
                              for b in range(B)], dtype=np.int64)
        tail0 = layer.z[torch.from_numpy(tail_rows.reshape(-1)).to(dev)].reshape(B, ring, 2, wl.d).contiguous()
        len0 = torch.from_numpy(L0).to(dev)
        length, z_tail = len0.clone(), tail0.clone()
        args = (x_new, z_new, new_off, int(n.max()), layer.tok_off, length, layer.kv, z_tail, layer.pool_off, wl.m,
                layer.pooled, layer.hpool_off, wl.m_hca, layer.hpooled)
        csa.csa_cache_append(*args)
        torch.cuda.synchronize()
        ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(reps)]
        for i in range(reps):
            length.copy_(len0)
            z_tail.copy_(tail0)
            csa.csa_profile_events(csa.CSA_K_APPEND, ev[i][0], ev[i][1])
            csa.csa_cache_append(*args)
            csa.csa_profile_events(csa.CSA_K_APPEND)
        torch.cuda.synchronize()
        us = float(np.mean([a.elapsed_ms(b) for a, b in ev])) * 1e3
        blocks = int(((L // wl.m) - (L0 // wl.m)).sum() + ((L // wl.m_hca) - (L0 // wl.m_hca)).sum())
        # new rows in (values and logits), raw rows out, ring rows out, pooled rows out
        nbytes = int(n.sum()) * 3 * row + int(np.minimum(n, ring).sum()) * row + blocks * row
        out[name] = {"tokens": int(n.sum()), "blocks_pooled": blocks, "us": round(us, 2),
                     "bytes": nbytes, "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
    log(f"cache append: {out}")
    return out


def bench_shared_prefix(torch, csa, synth, to_device, log, contiguous_kernel_ms, steps: int = 100, n_rot: int = 8):
    """csa_hca_decode_shared on 4 questions over one document: sequence 0 holds
    a 1,048,576-token cache, sequences 1..3 store only their own 8192, 4096 and
    1024 tokens after a shared prefix of T = 1,032,192 tokens (so every row
    attends to about a million tokens, like decode_b4_t1m).  Eager launches,
    HIP events around each, n_rot input sets (queries, indexer keys, HCA cache)
    rotated as in the main decode timing."""
    from long_context_compressed_05_amd.step import Layer, Params
    T, own = 1032192, [8192, 4096, 1024]
    lengths = [1 << 20] + own
    wl = synth.Workload("decode_shared_1m", lengths, [L - 1 for L in lengths], k=1024, seed=1006)
    host = synth.make_inputs(wl)
    q_pos = np.array([(1 << 20) - 1] + [T + s - 1 for s in own], dtype=np.int64)
    host["q_pos"] = q_pos
    p = Params(H=wl.H, d=wl.d, m=wl.m, k=wl.k, W=wl.W, m_hca=wl.m_hca, W_hca=wl.W_hca)
    layer = Layer.from_host(p, host, "cuda")
    layer.build_caches()
    B = len(lengths)
    logical_pool = [((1 << 20) // wl.m)] + [(T + s) // wl.m for s in own]
    logical_hpool = [((1 << 20) // wl.m_hca)] + [(T + s) // wl.m_hca for s in own]
    max_pool, max_hpool = max(logical_pool), max(logical_hpool)
    pre_seq = torch.tensor([-1, 0, 0, 0], dtype=torch.int32, device="cuda")
    pre_tok = torch.tensor([0, T, T, T], dtype=torch.int64, device="cuda")
    P_tot = int(host["pool_off"][-1])
    sets = []
    for r in range(n_rot):
        s = wl.seed + 7919 * (r + 1)
        hs = {"q": synth.normal(s, synth.S_Q, B * wl.H * wl.d, wl.dtype).reshape(B, wl.H, wl.d),
              "qc": synth.codes4(s, synth.S_QCODE, B * 128, wl.codeset).reshape(B, 4, 32),
              "qs": synth.exp_bytes(s, synth.S_QSCALE, B * 8, *wl.scale_exp).reshape(B, 4, 2),
              "w": synth.pow2(s, synth.S_W, B * 4, *wl.w_exp).reshape(B, 4),
              "kc": synth.codes4(s, synth.S_KCODE, P_tot * 32, wl.codeset).reshape(P_tot, 32),
              "ks": synth.exp_bytes(s, synth.S_KSCALE, P_tot * 2, *wl.scale_exp).reshape(P_tot, 2)}
        d = to_device(hs)
        d["hp"] = layer.hpooled.clone()
        sets.append(d)
    ws = csa.Workspace()

    def step(i):
        d = sets[i % n_rot]
        return csa.csa_hca_decode_shared(layer.batch, pre_seq, pre_tok, layer.pool_off, max_pool, layer.hpool_off,
                                         max_hpool, wl.m, wl.m_hca, wl.k, wl.W, wl.W_hca, 1.0 / math.sqrt(wl.d),
                                         d["qc"], d["qs"], d["w"], d["kc"], d["ks"], d["q"], layer.pooled, d["hp"],
                                         layer.kv, ws=ws)
    for i in range(2 * n_rot):
        step(i)
    torch.cuda.synchronize()
    ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(steps)]
    for i in range(steps):
        csa.csa_profile_events(csa.CSA_K_FUSED, ev[i][0], ev[i][1])
        step(i)
    torch.cuda.synchronize()
    csa.csa_profile_events(csa.CSA_K_FUSED)
    csa.csa_hca_decode_check(layer.batch, ws)
    us = float(np.mean([a.elapsed_ms(b) for a, b in ev])) * 1e3
    es = 2
    step_bytes = sum(decode_bytes_per_query(logical_pool[b], wl.k, wl.W, int(q_pos[b]) + 1, logical_hpool[b], wl.H,
                                            wl.d, es) for b in range(B))
    row = 2 * wl.d * es
    stored = int(host["tok_off"][-1]) * row + P_tot * (row + 34) + int(host["hpool_off"][-1]) * row
    logical = (sum(int(x) + 1 for x in q_pos)) * row + sum(logical_pool) * (row + 34) + sum(logical_hpool) * row
    out = {"workload": wl.name, "prefix_tokens": T, "own_tokens": own, "us_per_step": round(us, 2),
           "queries_per_s": round(B / (us * 1e-6), 1), "logical_step_bytes": int(step_bytes),
           "logical_GB/s": round(step_bytes / (us * 1e-6) / 1e9, 1),
           "contiguous_b4_t1m_kernel_us": round(contiguous_kernel_ms * 1e3, 2),
           "cache_bytes_stored": stored, "cache_bytes_if_contiguous": logical}
    log(f"shared prefix: {out}")
    return out


def bench_paged(torch, csa, layer, wl, host, sets, log, contiguous_kernel_ms, steps: int = 100,
                page_rows: int = 256, hca_page_rows: int = 64):
    """csa_hca_decode_paged on the 4 x 1M workload with its pooled caches and
    indexer keys scattered into shuffled pages (page_rows CSA rows,
    hca_page_rows HCA rows a page): event-timed launches over the same
    rotated queries and keys as the contiguous step."""
    dev = "cuda"
    rng = np.random.default_rng(2024)
    P_b, Ph_b = np.diff(host["pool_off"]), np.diff(host["hpool_off"])

    def layout(rows, pr):
        need = (rows + pr - 1) // pr
        perm = rng.permutation(int(need.sum()))
        tab = np.zeros((len(rows), int(need.max())), dtype=np.int32)
        src = []  # physical row of each contiguous row
        k = 0
        for b in range(len(rows)):
            tab[b, :need[b]] = perm[k:k + need[b]]
            k += need[b]
            j = np.arange(rows[b])
            src.append(tab[b, j // pr].astype(np.int64) * pr + j % pr)
        return tab, int(need.sum()), torch.from_numpy(np.concatenate(src)).to(dev)

    tab, npg, rows_p = layout(P_b, page_rows)
    htab, nhpg, rows_h = layout(Ph_b, hca_page_rows)

    def scatter(t, n_rows, rows):
        out = torch.zeros((n_rows, *t.shape[1:]), dtype=t.dtype, device=dev)
        out[rows] = t
        return out
    pooled = scatter(layer.pooled, npg * page_rows, rows_p)
    psets = [{"kc": scatter(d["kc"], npg * page_rows, rows_p), "ks": scatter(d["ks"], npg * page_rows, rows_p),
              "hp": scatter(d["hpooled"], nhpg * hca_page_rows, rows_h)} for d in sets]
    t_tab, t_htab = torch.from_numpy(tab).to(dev), torch.from_numpy(htab).to(dev)
    t_P, t_Ph = torch.from_numpy(P_b.astype(np.int64)).to(dev), torch.from_numpy(Ph_b.astype(np.int64)).to(dev)
    ws = csa.Workspace()
    R = len(sets)

    def step(i):
        d, pd = sets[i % R], psets[i % R]
        return csa.csa_hca_decode_paged(layer.batch, page_rows, t_tab, t_P, hca_page_rows, t_htab, t_Ph,
                                        layer.max_pool, layer.max_hpool, wl.m, wl.m_hca, wl.k, wl.W, wl.W_hca,
                                        1.0 / math.sqrt(wl.d), d["qc"], d["qs"], d["w"], pd["kc"], pd["ks"], d["q"],
                                        pooled, pd["hp"], layer.kv, ws=ws)
    for i in range(2 * R):
        step(i)
    torch.cuda.synchronize()
    ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(steps)]
    for i in range(steps):
        csa.csa_profile_events(csa.CSA_K_FUSED, ev[i][0], ev[i][1])
        step(i)
    torch.cuda.synchronize()
    csa.csa_profile_events(csa.CSA_K_FUSED)
    csa.csa_hca_decode_check(layer.batch, ws)
    us = float(np.mean([a.elapsed_ms(b) for a, b in ev])) * 1e3
    out = {"workload": wl.name, "page_rows": page_rows, "hca_page_rows": hca_page_rows, "pages": npg,
           "hca_pages": nhpg, "us_per_step": round(us, 2), "queries_per_s": round(wl.n_q / (us * 1e-6), 1),
           "contiguous_kernel_us": round(contiguous_kernel_ms * 1e3, 2)}
    log(f"paged: {out}")
    return out


def bench_mxfp4_recall(torch, csa, log, n_seq: int = 4, n_keys: int = 262144, k: int = 1024, reps: int = 20):
    """fp32 indexer queries (4 heads x 64) and keys (64), quantised on the GPU
    with csa_mxfp4_quantize and selected with csa_index_topk, against the exact
    top-k of the unquantised scores (fp64 on the host): recall = the share of
    the exact top-k the FP4 path returns.  Two synthetic data models: i.i.d.
    normal, and keys of which 2k per query carry a planted component along the
    query's heads.  Also the quantiser's throughput on the 1M-context key set."""
    dev = "cuda"
    rng = np.random.default_rng(20260424)
    w = np.array([0.5, 1.0, 2.0, 1.0], np.float32)
    out = {"n_keys": n_keys, "k": k, "queries": n_seq}
    for model in ("iid_normal", "planted"):
        q = rng.standard_normal((n_seq, 4, 64)).astype(np.float32)
        kf = rng.standard_normal((n_seq * n_keys, 64)).astype(np.float32)
        if model == "planted":
            for b in range(n_seq):
                sel = rng.choice(n_keys, size=2 * k, replace=False) + b * n_keys
                u = q[b].sum(axis=0)
                kf[sel] += (0.5 * u / np.linalg.norm(u) * np.sqrt(64)).astype(np.float32)
        exact = []
        for b in range(n_seq):
            d = kf[b * n_keys:(b + 1) * n_keys].astype(np.float64) @ q[b].astype(np.float64).T  # [n][4]
            S = (np.maximum(d, 0.0) * w.astype(np.float64)).sum(axis=1)
            exact.append(set(np.argpartition(-S, k - 1)[:k].tolist()))
        qd, kd = torch.from_numpy(q).to(dev), torch.from_numpy(kf).to(dev)
        wd = torch.from_numpy(np.tile(w, (n_seq, 1))).to(dev)
        qc, qs = csa.csa_mxfp4_quantize(qd)
        kc, ks = csa.csa_mxfp4_quantize(kd)
        pool_off = torch.from_numpy(np.arange(n_seq + 1, dtype=np.int64) * n_keys).to(dev)
        lengths = np.full(n_seq, 4 * n_keys, dtype=np.int64)
        batch = csa.Batch.from_host(np.concatenate([[0], np.cumsum(lengths)]), np.arange(n_seq + 1), lengths - 1)
        idx = csa.csa_index_topk(batch, pool_off, n_keys, 4, k, qc, qs, wd, kc, ks)
        got = idx.cpu().numpy()
        rec = [len(exact[b] & set(got[b].tolist())) / k for b in range(n_seq)]
        out[model] = {"recall_mean": round(float(np.mean(rec)), 4), "recall_min": round(float(np.min(rec)), 4)}
        if model == "iid_normal":  # quantiser throughput on the key set
            ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(reps)]
            for i in range(reps):
                csa.csa_profile_events(csa.CSA_K_QUANT, ev[i][0], ev[i][1])
                csa.csa_mxfp4_quantize(kd, kc, ks)
                csa.csa_profile_events(csa.CSA_K_QUANT)
            torch.cuda.synchronize()
            us = float(np.mean([a.elapsed_ms(b) for a, b in ev])) * 1e3
            nbytes = kf.nbytes + kc.numel() + ks.numel()
            out["quantize_keys"] = {"rows": int(kf.shape[0]), "dtype": "f32", "us": round(us, 2),
                                    "bytes": int(nbytes), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del qd, kd, kc, ks
    log(f"mxfp4 indexer: {out}")
    return out


def bench_prefill_indexer(torch, csa, synth, to_device, log, reps: int = 10):
    """The prefill indexer on a 4096-query chunk over a 65,536-token cache
    (17,408 pooled keys, top-512): the scoring kernel computes every visible
    score exactly once (the algorithmic FLOPs are counted over visible scores
    only); the threshold and selection kernels are timed beside it."""
    wl = synth.prefill_4k_on_64k()
    host = synth.make_inputs(wl, raw=False)
    d = to_device({k: host[k] for k in ("qc", "qs", "w", "kc", "ks", "pool_off")})
    batch = csa.Batch.from_host(host["tok_off"], host["q_off"], host["q_pos"])
    max_pool = int(np.diff(host["pool_off"]).max())
    ws = csa.Workspace()
    idx = torch.empty((wl.n_q, wl.k), dtype=torch.int32, device="cuda")
    call = lambda: csa.csa_index_topk(batch, d["pool_off"], max_pool, wl.m, wl.k, d["qc"], d["qs"], d["w"],
                                      d["kc"], d["ks"], idx=idx, ws=ws)
    call()
    torch.cuda.synchronize()
    kernels = {"score": csa.CSA_K_IDX_SCORE, "threshold": csa.CSA_K_PF_THRESH, "select": csa.CSA_K_PF_SELECT}
    ev = {name: [(csa.HipEvent(), csa.HipEvent()) for _ in range(reps)] for name in kernels}
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(reps):
        for name, kid in kernels.items():
            csa.csa_profile_events(kid, ev[name][i][0], ev[name][i][1])
        call()
    t1.record()
    torch.cuda.synchronize()
    for kid in kernels.values():
        csa.csa_profile_events(kid)
    us = {name: float(np.mean([a.elapsed_ms(b) for a, b in ev[name]])) * 1e3 for name in kernels}
    call_ms = t0.elapsed_time(t1) / reps
    n_vis = np.minimum((host["q_pos"] + 1) // wl.m, int(host["pool_off"][-1]))
    flops = 2.0 * 4 * 64 * float(n_vis.sum())
    tf = flops / (us["score"] * 1e-6) / 1e12
    log(f"prefill indexer: scoring {us['score']:.1f} us ({tf:.1f} TFLOP/s), threshold {us['threshold']:.1f} us, "
        f"select {us['select']:.1f} us, whole index_topk {call_ms * 1e3:.1f} us")
    return {"workload": wl.name, "scoring_kernel": "k_pf_score", "scoring_kernel_us": round(us["score"], 2),
            "threshold_kernel_us": round(us["threshold"], 2), "select_kernel_us": round(us["select"], 2),
            "algorithmic_flop": flops, "tflops": round(tf, 2), "peak_tflops": FP4_PEAK_TFLOPS,
            "frac": round(tf / FP4_PEAK_TFLOPS, 5), "index_topk_us": round(call_ms * 1e3, 2),
            "queries_per_s": round(wl.n_q / (call_ms * 1e-3), 1),
            "overhead_flop": {"threshold_sample": flops / 16, "select_rescore": "about 2 k keys per query"}}


def cpu_baseline(wl, host, log, min_seconds: float = 12.0):
    """The oracle, as it stands, on the decode queries of the same workload
    (one thread per query).  The oracle's fp64 HCA caches are built first and
    not timed, as the GPU's pooled caches are not."""
    import oracle
    n = wl.n_q
    seqs = np.repeat(np.arange(wl.B), np.diff(host["q_off"]))
    scale = 1.0 / math.sqrt(wl.d)

    def seq_rows(b):
        t0, t1 = int(host["tok_off"][b]), int(host["tok_off"][b + 1])
        return host["kv"][t0:t1], host["z"][t0:t1]

    log(f"cpu baseline: building oracle HCA caches for {n} queries")
    with ThreadPoolExecutor(max_workers=n) as ex:
        hp = list(ex.map(lambda r: oracle.pool(*seq_rows(seqs[r]), wl.m_hca), range(n)))

    def one(r):
        b = seqs[r]
        kv, z = seq_rows(b)
        p0, p1 = int(host["pool_off"][b]), int(host["pool_off"][b + 1])
        t = int(host["q_pos"][r])
        oracle.csa_query(kv, z, host["q"][r], t, wl.m, wl.W, wl.k, scale, host["qc"][r], host["qs"][r],
                         host["w"][r], host["kc"][p0:p1], host["ks"][p0:p1])
        oracle.hca_query(kv, z, host["q"][r], t, wl.m_hca, wl.W_hca, scale, hpooled=hp[r])

    log(f"cpu baseline: timing the oracle on {n} queries with {n} threads, repeated for at least {min_seconds} s")
    t = time.time()
    passes = 0
    with ThreadPoolExecutor(max_workers=n) as ex:
        while passes == 0 or time.time() - t < min_seconds:
            list(ex.map(one, range(n)))
            passes += 1
    dt = time.time() - t
    log(f"cpu baseline: {passes} passes in {dt:.2f} s")
    return {"value": round(passes * n / dt, 4), "unit": "queries/s", "cores": n, "kind": "oracle",
            "sample": f"{passes} passes over all {n} decode queries of {wl.name} (CSA: exact MXFP4 scores of every "
                      f"visible pooled entry, full-sort top-{wl.k}, fp64 pooling of the selected blocks, attention; "
                      f"HCA: attention over the oracle's prebuilt fp64 cache), one thread per query",
            "seconds": round(dt, 3), "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
