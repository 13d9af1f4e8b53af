#!/usr/bin/env python3
"""CSA + HCA decode and prefill benchmark on one MI355X (gfx950).

One step = one pass of the whole decode hot path over one batch: indexer
scoring, exact top-k, CSA sparse attention over the top-k pooled rows plus the
sliding window, and HCA dense attention, for every sequence's query at
position T-1.  By default the step is the single-launch csa_hca_decode call;
--path separate times csa_index_topk + csa_sparse_attn + hca_attn instead.
Pooled caches are built once with csa_compress before timing (its throughput
is reported apart).  --copy-calibration runs only a 1 GiB device copy, the
scale reference for the HBM byte counters.

Headline workload: 4 sequences x 1,048,576 tokens, 64 query heads on one bf16
KV head, d = 128, m = 4 (262,144 pooled entries), top-k 1024, window 128,
m' = 128 (8192 entries), indexer 4 heads x 64 in MXFP4.  Inputs are seeded
synthetic data already resident in HBM; R input sets are rotated so that
consecutive steps do not hit the 256 MB Infinity Cache.  Also reported: the
other decode configurations (4096-token fp32, 16 x 64K, 32 ragged sequences),
HCA with a window, the prefill step of a 4096-token chunk on a 64K cache, the
measured peaks of the part (HBM read, FP4 and bf16 MFMA), cache upkeep,
shared-prefix and paged decode, and the CPU oracle beside them.

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


def pct(xs):
    """median, p10 and p90 of a list of durations (microseconds)."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 3), "p10": round(float(np.percentile(a, 10)), 3),
            "p90": round(float(np.percentile(a, 90)), 3), "mean": round(float(a.mean()), 3), "n": int(a.size)}


def step_bytes_of(wl, host):
    """Algorithmic bytes of one decode step over every query of the batch."""
    es = 2 if wl.dtype == "bf16" else 4
    q_pos = host["q_pos"]
    q_seq = np.repeat(np.arange(wl.B), np.diff(host["q_off"]))
    P_b, Ph_b = np.diff(host["pool_off"]), np.diff(host["hpool_off"])
    tot = 0
    for i in range(wl.n_q):
        b, t = q_seq[i], int(q_pos[i])
        n_vis = min((t + 1) // wl.m, int(P_b[b]))
        n_hvis = min((t + 1) // wl.m_hca, int(Ph_b[b]))
        tot += decode_bytes_per_query(n_vis, wl.k, wl.W, t + 1, n_hvis, wl.H, wl.d, es)
    return int(tot)


class DecodeBench:
    """One decode workload resident on the GPU: raw KV, pooled caches (built
    with csa_compress, timed apart) and R rotated input sets (queries, indexer
    codes, scales and weights, indexer keys, HCA cache) so that consecutive
    steps do not find their data in the 256 MB Infinity Cache."""

    def __init__(self, torch, csa, synth, to_device, wl, R, path):
        from long_context_compressed_05_amd.step import Layer, Params
        self.torch, self.csa, self.wl, self.R = torch, csa, wl, max(1, R)
        self.path = path
        dev = "cuda"
        self.host = host = synth.make_inputs(wl)
        self.es = 2 if wl.dtype == "bf16" else 4
        p = Params(H=wl.H, d=wl.d, m=wl.m, k=wl.k, W=wl.W, m_hca=wl.m_hca, W_hca=wl.W_hca)
        self.layer = layer = Layer.from_host(p, host, dev)
        n_pool, n_hpool = int(host["pool_off"][-1]), int(host["hpool_off"][-1])
        layer.pooled = torch.empty((n_pool, 2, wl.d), dtype=layer.kv.dtype, device=dev)
        layer.hpooled = torch.empty((n_hpool, 2, wl.d), dtype=layer.kv.dtype, device=dev)
        self.compress = {}
        for name, m, off, out, kid in (("csa", wl.m, layer.pool_off, layer.pooled, csa.CSA_K_COMPRESS),
                                       ("hca", wl.m_hca, layer.hpool_off, layer.hpooled, csa.CSA_K_COMPRESS)):
            csa.csa_compress(layer.kv, layer.z, layer.tok_off, off, layer.batch.max_len, m, out)  # warm
            e0, e1 = csa.HipEvent(), csa.HipEvent()
            csa.csa_profile_events(kid, e0, e1)
            csa.csa_compress(layer.kv, layer.z, layer.tok_off, off, layer.batch.max_len, m, out)
            csa.csa_profile_events(kid)
            ms = e0.elapsed_ms(e1)
            rows = sum((L // m) * m for L in wl.lengths)
            nbytes = 2 * rows * 2 * wl.d * self.es + (rows // m) * 2 * wl.d * self.es
            self.compress[name] = {"m": m, "us": round(ms * 1e3, 2), "GB/s": round(nbytes / ms / 1e6, 1)}
        self.sets = []
        P_tot = n_pool
        for r in range(self.R):
            if r == 0:
                hs = {k: host[k] for k in ("q", "qc", "qs", "w", "kc", "ks")}
            else:
                s_ = wl.seed + 7919 * r
                hs = {"q": synth.normal(s_, synth.S_Q, wl.n_q * wl.H * wl.d, wl.dtype).reshape(wl.n_q, wl.H, wl.d),
                      "qc": synth.codes4(s_, synth.S_QCODE, wl.n_q * 128, wl.codeset).reshape(wl.n_q, 4, 32),
                      "qs": synth.exp_bytes(s_, synth.S_QSCALE, wl.n_q * 8, *wl.scale_exp).reshape(wl.n_q, 4, 2),
                      "w": synth.pow2(s_, synth.S_W, wl.n_q * 4, *wl.w_exp).reshape(wl.n_q, 4),
                      "kc": synth.codes4(s_, synth.S_KCODE, P_tot * 32, wl.codeset).reshape(P_tot, 32),
                      "ks": synth.exp_bytes(s_, synth.S_KSCALE, P_tot * 2, *wl.scale_exp).reshape(P_tot, 2)}
            d = to_device(hs, dev)
            d["hpooled"] = layer.hpooled if r == 0 else layer.hpooled.clone()
            d["idx"] = torch.empty((wl.n_q, wl.k), dtype=torch.int32, device=dev)
            d["co"] = torch.empty((wl.n_q, wl.H, wl.d), dtype=layer.kv.dtype, device=dev)
            d["cl"] = torch.empty((wl.n_q, wl.H), dtype=torch.float32, device=dev)
            d["ho"] = torch.empty_like(d["co"])
            d["hl"] = torch.empty_like(d["cl"])
            self.sets.append(d)
        self.step_bytes = step_bytes_of(wl, host)
        self.scale = 1.0 / math.sqrt(wl.d)

    def step(self, r):
        d, layer, wl, csa = self.sets[r % self.R], self.layer, self.wl, self.csa
        if self.path == "fused":
            layer.decode_fused(d["q"], d["qc"], d["qs"], d["w"], idx=d["idx"], csa_out=d["co"], csa_lse=d["cl"],
                               hca_out=d["ho"], hca_lse=d["hl"], kc=d["kc"], ks=d["ks"], hpooled=d["hpooled"])
        else:
            b = layer.batch
            csa.csa_index_topk(b, layer.pool_off, layer.max_pool, wl.m, wl.k, d["qc"], d["qs"], d["w"], d["kc"],
                               d["ks"], idx=d["idx"], ws=layer.ws_idx)
            csa.csa_sparse_attn(b, layer.pool_off, d["q"], layer.pooled, layer.kv, d["idx"], wl.W, self.scale,
                                out=d["co"], lse=d["cl"], ws=layer.ws_csa)
            csa.hca_attn(b, layer.hpool_off, layer.max_hpool, wl.m_hca, d["q"], d["hpooled"], layer.kv, wl.W_hca,
                         self.scale, out=d["ho"], lse=d["hl"], ws=layer.ws_hca)

    def run(self, steps, warmup, graph=True):
        """Warm-up, then (1) `steps` eager steps with per-launch events (the
        fused kernel's events ride on its dispatch: kernel execution only; the
        separate calls' step is bracketed by stream events), (2) a HIP graph of
        the R rotated steps replayed until at least `steps` steps ran, timed as
        a whole.  Returns the per-step figures."""
        torch, csa = self.torch, self.csa
        for i in range(warmup):
            self.step(i)
        torch.cuda.synchronize()
        per = []
        if self.path == "fused":
            ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(steps)]
            for i in range(steps):
                csa.csa_profile_events(csa.CSA_K_FUSED, ev[i][0], ev[i][1])
                self.step(i)
            csa.csa_profile_events(csa.CSA_K_FUSED)
            torch.cuda.synchronize()
            self.layer.check_fused()
            per = [a.elapsed_ms(b) * 1e3 for a, b in ev]
        else:
            for i in range(steps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                self.step(i)
                e1.record()
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) * 1e3)
        g = None
        if graph:
            try:
                g = torch.cuda.CUDAGraph()
                cap = torch.cuda.Stream()
                cap.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(cap):
                    with torch.cuda.graph(g, stream=cap):
                        for r in range(self.R):
                            self.step(r)
                torch.cuda.current_stream().wait_stream(cap)
                g.replay()
                torch.cuda.synchronize()
            except Exception as e:
                log(f"graph capture unavailable ({e!r}); timing eager launches")
                g = None
        reps = max(1, (steps + self.R - 1) // self.R) if g is not None else steps
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        if g is not None:
            for _ in range(reps):
                g.replay()
        else:
            for i in range(steps):
                self.step(i)
        t1.record()
        torch.cuda.synchronize()
        n_steps = reps * self.R if g is not None else steps
        ms_step = t0.elapsed_time(t1) / n_steps
        if self.path == "fused":
            self.layer.check_fused()
        wl = self.wl
        kern = pct(per)
        out = {"workload": wl.name, "path": self.path, "rotate_sets": self.R, "steps_timed": n_steps,
               "us_per_step": round(ms_step * 1e3, 3),
               "timing": "hip graph of the rotated steps, replayed" if g is not None else "eager launches",
               "queries_per_s": round(wl.n_q / (ms_step * 1e-3), 1), "step_bytes": self.step_bytes,
               "GB/s": round(self.step_bytes / (ms_step * 1e-3) / 1e9, 1),
               "frac_of_8TB/s": round(self.step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               ("kernel_us" if self.path == "fused" else "eager_step_us"): kern}
        if self.path == "fused":
            achieved = self.step_bytes / (kern["median"] * 1e-6) / 1e9
            out["kernel_GB/s"] = round(achieved, 1)
            out["kernel_frac_of_8TB/s"] = round(achieved / HBM_PEAK_GBS, 4)
        return out, ms_step, per


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_b4_t1m")
    ap.add_argument("--rotate", type=int, default=20, help="input sets cycled through the timed steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the headline decode step only (no other configs, sections, peaks or CPU baseline)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a captured HIP graph")
    ap.add_argument("--path", choices=["fused", "separate"], default="fused",
                    help="fused: one csa_hca_decode launch per step; separate: csa_index_topk + csa_sparse_attn + hca_attn")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time the prefill step (4096 queries over a 65,536-token cache) and print its record")
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
    from long_context_compressed_05_amd.step import to_device

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    if args.copy_calibration:
        copy_calibration(torch)
        return
    csa.lib()
    torch.cuda.init()
    if args.prefill_only:
        print(json.dumps({"prefill": bench_prefill_chunk(torch, csa, synth, to_device, log)}), flush=True)
        return

    wl = synth.WORKLOADS[args.workload]()
    log(f"workload {wl.name}: B={wl.B} max_len={max(wl.lengths)} n_q={wl.n_q}; generating inputs")
    db = DecodeBench(torch, csa, synth, to_device, wl, args.rotate, args.path)
    log(f"inputs and {db.R} rotation sets resident; compress: {db.compress}")
    head, ms_step, per = db.run(args.steps, args.warmup, graph=not args.eager)
    log(f"headline: {head}")
    prof_name = "k_decode_fused" if args.path == "fused" else None
    result = {
        "metric": METRIC,
        "value": round(wl.n_q / (ms_step * 1e-3), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": head["steps_timed"],
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {**wl.describe(), "indexer": "mxfp4 4x64", "rotate_sets": db.R, "path": args.path,
                   "timing": head["timing"]},
        "hbm_gbps": head["GB/s"],
        "hbm_frac": head["frac_of_8TB/s"],
        "step_bytes": db.step_bytes,
        "decode": head,
        "compress": db.compress,
    }
    if prof_name:
        kern = head["kernel_us"]
        achieved = db.step_bytes / (kern["median"] * 1e-6) / 1e9
        result["roofline"] = {"bound": "hbm", "kernel": prof_name, "achieved": round(achieved, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                              "traffic": counted_traffic(prof_name, wl.name), "bytes_per_launch": db.step_bytes,
                              "launch_us": kern,
                              "duration": "median kernel execution per launch (events attached to each dispatch)"}
    if args.no_extras:
        print(json.dumps(result), flush=True)
        return

    # ---- measured peaks of this part ---------------------------------------------
    try:
        result["peaks"] = bench_peaks(torch, csa, db.step_bytes, log)
        if "roofline" in result and "hbm_read_GB/s" in result["peaks"]:
            mp = result["peaks"]["hbm_read_GB/s"]
            result["roofline"]["measured_peak"] = mp
            result["roofline"]["frac_of_measured_peak"] = round(result["roofline"]["achieved"] / mp, 4)
            sp = result["peaks"].get("hbm_read_1GiB_GB/s")
            if sp:  # the sustained rate of a long read, which a step of this size cannot reach
                result["roofline"]["sustained_read_peak"] = sp
                result["roofline"]["frac_of_sustained_read"] = round(result["roofline"]["achieved"] / sp, 4)
    except Exception as e:  # reported, never silently replaced
        result["peaks"] = {"error": repr(e)}

    # ---- the other decode configurations, each in its own launch configuration ---
    result["configs"] = {}
    cfgs = [("decode_t4096_fp32", "separate", 4), ("decode_b16_t64k", "fused", 60), ("decode_ragged_b32", "fused", 12)]
    for name, path, R in cfgs:
        try:
            cdb = DecodeBench(torch, csa, synth, to_device, synth.WORKLOADS[name](), R, path)
            result["configs"][name], _, _ = cdb.run(max(args.steps, 20), args.warmup)
            del cdb
            torch.cuda.empty_cache()
        except Exception as e:  # reported, never silently replaced
            result["configs"][name] = {"error": repr(e)}
        log(f"config {name}: {result['configs'][name]}")
    # reading D5's alternative: HCA with the same 128-token window as CSA
    try:
        wl_w = synth.WORKLOADS[args.workload]()
        wl_w.W_hca = wl_w.W
        wdb = DecodeBench(torch, csa, synth, to_device, wl_w, args.rotate, args.path)
        rec, _, _ = wdb.run(max(args.steps, 20), args.warmup)
        rec["W_hca"] = wl_w.W_hca
        result["configs"][args.workload + "_hca_window"] = rec
        del wdb
        torch.cuda.empty_cache()
    except Exception as e:  # reported, never silently replaced
        result["configs"][args.workload + "_hca_window"] = {"error": repr(e)}

    # ---- streaming cache upkeep (appends at the end of the 1M-token caches) -----
    try:
        result["cache_append"] = bench_cache_append(torch, csa, db.layer, wl, db.host, log)
    except Exception as e:  # reported, never silently replaced
        result["cache_append"] = {"error": repr(e)}

    # ---- MXFP4 quantiser and the recall of the FP4 indexer's top-k -------------
    try:
        result["mxfp4_indexer"] = bench_mxfp4_recall(torch, csa, log)
    except Exception as e:  # reported, never silently replaced
        result["mxfp4_indexer"] = {"error": repr(e)}

    # ---- shared-prefix and paged decode over ~1M-token caches --------------------
    if args.workload == "decode_b4_t1m" and args.path == "fused":
        kernel_ms = head["kernel_us"]["median"] * 1e-3
        try:
            result["shared_prefix"] = bench_shared_prefix(torch, csa, synth, to_device, log, kernel_ms)
        except Exception as e:  # reported, never silently replaced
            result["shared_prefix"] = {"error": repr(e)}
        try:
            result["paged"] = bench_paged(torch, csa, db.layer, wl, db.host, db.sets, log, kernel_ms)
        except Exception as e:  # reported, never silently replaced
            result["paged"] = {"error": repr(e)}

    # ---- the prefill step (4096-token chunk on a 64K cache) ----------------------
    if not args.no_prefill:
        try:
            result["prefill"] = bench_prefill_chunk(torch, csa, synth, to_device, log)
            if "peaks" in result and "bf16_mfma_TFLOP/s" in result["peaks"]:
                for part in ("csa_attn", "hca_attn"):
                    rec = result["prefill"][part]
                    rec["frac_of_measured_peak"] = round(rec["tflops"] / result["peaks"]["bf16_mfma_TFLOP/s"], 4)
            if "peaks" in result and "fp4_mfma_TFLOP/s" in result["peaks"]:
                rec = result["prefill"]["indexer"]
                rec["scoring_frac_of_measured_peak"] = round(rec["scoring_tflops"] /
                                                             result["peaks"]["fp4_mfma_TFLOP/s"], 4)
        except Exception as e:  # reported, never silently replaced
            result["prefill"] = {"error": repr(e)}

    # ---- CPU oracle baseline --------------------------------------------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, db.host, log)

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


def release_lines(lines, name="<source>"):
    """The lines of a kernel source that can change its release build: not
    blank, not whole-line comments, not inside #ifdef CSA_DEBUG blocks (code
    compiled only into the debug library)."""
    skip = 0  # depth inside a CSA_DEBUG block
    for line in lines:
        t = line.strip()
        if skip:
            if t.startswith("#if"):
                skip += 1
            elif t.startswith("#endif"):
                skip -= 1
            elif t.startswith("#el") and skip == 1:
                raise ValueError(f"{name}: #else or #elif in a CSA_DEBUG block")
            continue
        if t == "#ifdef CSA_DEBUG":
            skip = 1
            continue
        if t and not t.startswith("//"):
            yield line.rstrip()
    if skip:
        raise ValueError(f"{name}: unterminated CSA_DEBUG block")


def kernel_source_digest(kernel: str) -> str:
    """sha256 over the release lines of the sources `kernel` is built from."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "long_context_compressed_05_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, f)) as fh:
            for line in release_lines(fh, f):
                h.update(line.encode())
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
    """csa_cache_append at the end of the resident 1M-token caches.  Decode
    steps (one new token for each of the 4 sequences, one launch) in the three
    cases a step meets: the token completes no block, a CSA block (1 step in
    m), or a CSA and an HCA block (1 step in m'); their mean over a cycle of
    m' steps is the amortised cost per step.  Then a 4096-token chunk on one
    sequence (two launches).  Each completed CSA block's 64-element indexer
    vector is encoded into the MXFP4 key cache in the same call.  The appended
    rows are the caches' own rows, so every call rewrites identical data;
    lengths and tail rings are reset between calls, outside the timed region
    (events attached to the call's kernels; medians)."""
    dev = "cuda"
    B, L = wl.B, np.array(wl.lengths, dtype=np.int64)
    tok_off = host["tok_off"]
    ring = wl.m_hca
    es = 2 if wl.dtype == "bf16" else 4
    row = 2 * wl.d * es
    # (tokens per sequence, how far before the cache end the append ends)
    cases = {"decode_none": (np.ones(B, dtype=np.int64), 2), "decode_csa": (np.ones(B, dtype=np.int64), wl.m),
             "decode_csa_hca": (np.ones(B, dtype=np.int64), 0),
             "prefill_chunk": (np.array([4096] + [0] * (B - 1), dtype=np.int64), 0)}
    out = {}
    for name, (n, back) in cases.items():
        L1 = L - back
        L0 = L1 - n
        rows = np.concatenate([np.arange(tok_off[b] + L0[b], tok_off[b] + L1[b]) for b in range(B)]).astype(np.int64)
        r = torch.from_numpy(rows).to(dev)
        x_new, z_new = layer.kv[r].contiguous(), layer.z[r].contiguous()
        new_off = torch.from_numpy(np.concatenate([[0], np.cumsum(n)]).astype(np.int64)).to(dev)
        tail_rows = np.array([[tok_off[b] + (p if p >= 0 else 0) for p in
                               [L0[b] - ring + ((s - (L0[b] - ring)) % ring) for s in range(ring)]]
                              for b in range(B)], dtype=np.int64)
        tail0 = layer.z[torch.from_numpy(tail_rows.reshape(-1)).to(dev)].reshape(B, ring, 2, wl.d).contiguous()
        len0 = torch.from_numpy(L0).to(dev)
        length, z_tail = len0.clone(), tail0.clone()
        nblk = (L1 // wl.m) - (L0 // wl.m)
        hblk = (L1 // wl.m_hca) - (L0 // wl.m_hca)
        kvec = torch.randn((max(1, int(nblk.sum())), 64), device=dev).to(layer.kv.dtype)
        kvec_off = torch.from_numpy(np.concatenate([[0], np.cumsum(nblk)]).astype(np.int64)).to(dev)
        kc_scr = torch.zeros((int(host["pool_off"][-1]), 32), dtype=torch.uint8, device=dev)
        ks_scr = torch.zeros((int(host["pool_off"][-1]), 2), dtype=torch.uint8, device=dev)
        args = (x_new, z_new, new_off, int(n.max()), layer.tok_off, length, layer.kv, z_tail, layer.pool_off, wl.m,
                layer.pooled, layer.hpool_off, wl.m_hca, layer.hpooled, kvec_off, kvec, kc_scr, ks_scr)
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
        t_us = np.array([a.elapsed_ms(b) for a, b in ev]) * 1e3
        blocks = int(nblk.sum() + hblk.sum())
        # new rows in (values and logits), raw rows out, ring rows out, pooled rows out, key vectors in, keys out
        nbytes = (int(n.sum()) * 3 * row + int(np.minimum(n, ring).sum()) * row + blocks * row
                  + int(nblk.sum()) * (64 * es + 34))
        us = float(np.median(t_us))
        out[name] = {"tokens": int(n.sum()), "csa_blocks": int(nblk.sum()), "hca_blocks": int(hblk.sum()),
                     "keys_encoded": int(nblk.sum()), "launches": 1 if int(n.max()) <= 64 else 2,
                     "us_median": round(us, 2), "us_p10": round(float(np.percentile(t_us, 10)), 2),
                     "us_p90": round(float(np.percentile(t_us, 90)), 2),
                     "bytes_written_or_read_new": nbytes}
    c = wl.m_hca // wl.m  # CSA completions per HCA cycle
    amort = ((wl.m_hca - c) * out["decode_none"]["us_median"] + (c - 1) * out["decode_csa"]["us_median"]
             + out["decode_csa_hca"]["us_median"]) / wl.m_hca
    out["decode_amortised_us_per_step"] = round(amort, 2)
    out["note"] = ("a decode step's append reads the completed HCA block's 128 rows (values and logits); "
                   "its floor is one launch (peaks.empty_kernel_us)")
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
    """The MXFP4 indexer against a bf16 one and against exact scores.  fp32
    indexer queries (4 heads x 64) and keys (64) are quantised on the GPU with
    csa_mxfp4_quantize and selected with csa_index_topk; the same values
    rounded to bf16 are selected with csa_index_topk_bf16.  Recall = the share
    of a reference top-k a path returns: each path against the exact top-k of
    the unquantised fp64 scores (host), and FP4 against bf16.  Two synthetic
    data models: i.i.d. normal, and keys of which 2k per query carry a planted
    component along the query's heads.  Times (median of `reps`, kernel-only
    from the tracing hook for the scoring kernel, events around the call for
    the whole selection) give the FP4 path's speed-up.  Also the quantiser's
    throughput on the key set."""
    dev = "cuda"
    rng = np.random.default_rng(20260424)
    w = np.array([0.5, 1.0, 2.0, 1.0], np.float32)
    out = {"n_keys_per_query": n_keys, "k": k, "queries": n_seq}

    def timed(call):
        ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(reps)]
        tot = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        call()
        for i in range(reps):
            csa.csa_profile_events(csa.CSA_K_IDX_SCORE, ev[i][0], ev[i][1])
            tot[i][0].record()
            call()
            tot[i][1].record()
            csa.csa_profile_events(csa.CSA_K_IDX_SCORE)
        torch.cuda.synchronize()
        score = float(np.median([a.elapsed_ms(b) for a, b in ev])) * 1e3
        whole = float(np.median([a.elapsed_time(b) for a, b in tot])) * 1e3
        return score, whole

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
        qb, kb = qd.to(torch.bfloat16), kd.to(torch.bfloat16)
        wd = torch.from_numpy(np.tile(w, (n_seq, 1))).to(dev)
        qc, qs = csa.csa_mxfp4_quantize(qd)
        kc, ks = csa.csa_mxfp4_quantize(kd)
        pool_off = torch.from_numpy(np.arange(n_seq + 1, dtype=np.int64) * n_keys).to(dev)
        lengths = np.full(n_seq, 4 * n_keys, dtype=np.int64)
        batch = csa.Batch.from_host(np.concatenate([[0], np.cumsum(lengths)]), np.arange(n_seq + 1), lengths - 1)
        ws = csa.Workspace()
        idx = torch.empty((n_seq, k), dtype=torch.int32, device=dev)
        idx_b = torch.empty_like(idx)
        fp4 = lambda: csa.csa_index_topk(batch, pool_off, n_keys, 4, k, qc, qs, wd, kc, ks, idx=idx, ws=ws)
        bf16 = lambda: csa.csa_index_topk_bf16(batch, pool_off, n_keys, 4, k, qb, wd, kb, idx=idx_b, ws=ws)
        fp4()
        bf16()
        got, got_b = idx.cpu().numpy(), idx_b.cpu().numpy()
        sets_b = [set(got_b[b].tolist()) for b in range(n_seq)]
        rec = [len(exact[b] & set(got[b].tolist())) / k for b in range(n_seq)]
        rec_b = [len(exact[b] & sets_b[b]) / k for b in range(n_seq)]
        rec_fb = [len(sets_b[b] & set(got[b].tolist())) / k for b in range(n_seq)]
        r = lambda v: {"mean": round(float(np.mean(v)), 4), "min": round(float(np.min(v)), 4)}
        out[model] = {"fp4_vs_exact": r(rec), "bf16_vs_exact": r(rec_b), "fp4_vs_bf16": r(rec_fb)}
        if model == "iid_normal":
            s4, w4 = timed(fp4)
            s16, w16 = timed(bf16)
            kb4 = kc.numel() + ks.numel()
            kb16 = kb.numel() * 2
            out["time_us"] = {
                "fp4_score": round(s4, 2), "bf16_score": round(s16, 2),
                "fp4_call": round(w4, 2), "bf16_call": round(w16, 2),
                "score_speedup": round(s16 / s4, 2), "call_speedup": round(w16 / w4, 2),
                "key_bytes": {"fp4": int(kb4), "bf16": int(kb16)},
                "score_GB/s": {"fp4": round(kb4 / (s4 * 1e-6) / 1e9, 1), "bf16": round(kb16 / (s16 * 1e-6) / 1e9, 1)}}
            ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(reps)]
            for i in range(reps):  # quantiser throughput on the key set
                csa.csa_profile_events(csa.CSA_K_QUANT, ev[i][0], ev[i][1])
                csa.csa_mxfp4_quantize(kd, kc, ks)
                csa.csa_profile_events(csa.CSA_K_QUANT)
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_ms(b) for a, b in ev])) * 1e3
            nbytes = kf.nbytes + kc.numel() + ks.numel()
            out["quantize_keys"] = {"rows": int(kf.shape[0]), "dtype": "f32", "us_median": round(us, 2),
                                    "bytes": int(nbytes), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del qd, kd, qb, kb, kc, ks
    log(f"indexer fp4 vs bf16: {out}")
    return out


BF16_PEAK_TFLOPS = 2500.0


def bench_prefill_chunk(torch, csa, synth, to_device, log, reps: int = 10, oracle_queries: int = 8):
    """The whole prefill step of a 4096-token chunk on a 65,536-token cache:
    csa_cache_append of the chunk (1024 CSA and 32 HCA blocks pooled), then
    csa_index_topk (threshold, scoring and selection kernels), csa_sparse_attn
    and hca_attn for all 4096 queries.  Kernel times come from the tracing
    hook's events (kernel execution only); the step time from events around
    the four calls (eager, launch gaps included).  The attention FLOPs count
    the valid keys of each query only: 4*H*d per key (QK and PV)."""
    wl = synth.prefill_4k_on_64k()
    host = synth.make_inputs(wl)
    dev = "cuda"
    T0, L = wl.q_start[0], wl.lengths[0]
    n = L - T0
    d = to_device({k: host[k] for k in ("kv", "z", "q", "qc", "qs", "w", "kc", "ks")})
    kv_raw = torch.zeros_like(d["kv"])
    kv_raw[:T0] = d["kv"][:T0]
    P_cap, Ph_cap = L // wl.m, L // wl.m_hca
    pooled = torch.zeros((P_cap, 2, wl.d), dtype=d["kv"].dtype, device=dev)
    hpooled = torch.zeros((Ph_cap, 2, wl.d), dtype=d["kv"].dtype, device=dev)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.int64)).to(dev)
    tok0, pool_off, hpool_off, tok_off = t([0, T0]), t([0, P_cap]), t([0, Ph_cap]), t([0, L])
    csa.csa_compress(d["kv"], d["z"], tok0, pool_off, T0, wl.m, pooled)
    csa.csa_compress(d["kv"], d["z"], tok0, hpool_off, T0, wl.m_hca, hpooled)
    ring = wl.m_hca
    slots = np.array([T0 - ring + ((s_ - (T0 - ring)) % ring) for s_ in range(ring)])
    tail0 = d["z"][t(slots)].reshape(1, ring, 2, wl.d).contiguous()
    z_tail, len0 = tail0.clone(), t([T0])
    length = len0.clone()
    x_new, z_new, new_off = d["kv"][T0:].contiguous(), d["z"][T0:].contiguous(), t([0, n])
    batch = csa.Batch.from_host(host["tok_off"], host["q_off"], host["q_pos"])
    scale = 1.0 / math.sqrt(wl.d)
    idx = torch.empty((wl.n_q, wl.k), dtype=torch.int32, device=dev)
    co, ho = torch.empty_like(d["q"]), torch.empty_like(d["q"])
    cl = torch.empty((wl.n_q, wl.H), dtype=torch.float32, device=dev)
    hl = torch.empty_like(cl)
    ws_i, ws_c, ws_h = csa.Workspace(), csa.Workspace(), csa.Workspace()
    names = ("append", "threshold", "score", "select", "csa_attn", "csa_combine", "hca_attn", "hca_combine")
    ev = {nm: [(csa.HipEvent(), csa.HipEvent()) for _ in range(reps)] for nm in names}
    used = {nm: False for nm in names}

    def hook(kid, nm, i):
        csa.csa_profile_events(kid, ev[nm][i][0], ev[nm][i][1])

    def step(i=None):
        if i is not None:
            hook(csa.CSA_K_APPEND, "append", i)
        csa.csa_cache_append(x_new, z_new, new_off, n, tok_off, length, kv_raw, z_tail, pool_off, wl.m, pooled,
                             hpool_off, wl.m_hca, hpooled)
        if i is not None:
            hook(csa.CSA_K_PF_THRESH, "threshold", i)
            hook(csa.CSA_K_IDX_SCORE, "score", i)
            hook(csa.CSA_K_PF_SELECT, "select", i)
        csa.csa_index_topk(batch, pool_off, P_cap, wl.m, wl.k, d["qc"], d["qs"], d["w"], d["kc"], d["ks"], idx=idx,
                           ws=ws_i)
        if i is not None:
            hook(csa.CSA_K_ATTN, "csa_attn", i)
            hook(csa.CSA_K_ATTN_COMBINE, "csa_combine", i)
        csa.csa_sparse_attn(batch, pool_off, d["q"], pooled, kv_raw, idx, wl.W, scale, out=co, lse=cl, ws=ws_c)
        if i is not None:
            hook(csa.CSA_K_ATTN, "hca_attn", i)
            hook(csa.CSA_K_ATTN_COMBINE, "hca_combine", i)
        csa.hca_attn(batch, hpool_off, Ph_cap, wl.m_hca, d["q"], hpooled, kv_raw, wl.W_hca, scale, out=ho, lse=hl,
                     ws=ws_h)
        if i is not None:
            for kid in (csa.CSA_K_APPEND, csa.CSA_K_PF_THRESH, csa.CSA_K_IDX_SCORE, csa.CSA_K_PF_SELECT,
                        csa.CSA_K_ATTN, csa.CSA_K_ATTN_COMBINE):
                csa.csa_profile_events(kid)

    def reset():
        length.copy_(len0)
        z_tail.copy_(tail0)

    reset()
    step()
    torch.cuda.synchronize()
    # which combine kernels run at this shape (splits > 1)
    used["csa_combine"] = csa.csa_sparse_attn_workspace(csa.CSA_BF16, batch, wl.H, wl.d, wl.W, wl.k) > 0
    used["hca_combine"] = csa.hca_attn_workspace(csa.CSA_BF16, batch, Ph_cap, wl.H, wl.d, wl.W_hca) > 0
    for nm in names:
        if nm not in ("csa_combine", "hca_combine"):
            used[nm] = True
    step_ms = []
    for i in range(reps):
        reset()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step(i)
        e1.record()
        torch.cuda.synchronize()
        step_ms.append(e0.elapsed_time(e1))
    us = {nm: float(np.median([a.elapsed_ms(b) for a, b in ev[nm]])) * 1e3 for nm in names if used[nm]}
    step_us = float(np.median(step_ms)) * 1e3
    # the same step captured once in a HIP graph and replayed (no launch gaps
    # between its kernels); every replay's outputs must equal the eager step's
    def graph_of(fn):
        try:
            reset()
            step()
            torch.cuda.synchronize()
            ref = [t_.clone() for t_ in (idx, co, cl, ho, hl)]
            g = torch.cuda.CUDAGraph()
            cap = torch.cuda.Stream()
            reset()
            cap.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cap):
                with torch.cuda.graph(g, stream=cap):
                    fn()
            torch.cuda.current_stream().wait_stream(cap)
            torch.cuda.synchronize()
            g_ms = []
            for i in range(reps):
                reset()
                for t_ in (idx, co, cl, ho, hl):
                    t_.fill_(0)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                g_ms.append(e0.elapsed_time(e1))
                if not all(torch.equal(a_, b_) for a_, b_ in zip((idx, co, cl, ho, hl), ref)):
                    raise RuntimeError(f"graph replay {i} differs from the eager step")
            g_us = float(np.median(g_ms)) * 1e3
            return {"step_us": round(g_us, 2), "prefill_tokens_per_s": round(n / (g_us * 1e-6), 1),
                    "replays": reps, "check": "every replay's top-k, outputs and LSEs equal the eager step's"}
        except Exception as e:  # reported, never silently replaced
            return {"error": repr(e)}
    graph = graph_of(step)
    # algorithmic FLOPs
    q_pos = host["q_pos"]
    k_eff = np.minimum(wl.k, np.minimum((q_pos + 1) // wl.m, P_cap))
    win = np.minimum(wl.W, q_pos + 1)
    n_hvis = np.minimum((q_pos + 1) // wl.m_hca, Ph_cap)
    per_key = 4.0 * wl.H * wl.d
    csa_flop = per_key * float((k_eff + win).sum())
    hca_flop = per_key * float(n_hvis.sum())
    idx_flop = 2.0 * 4 * 64 * float(np.minimum((q_pos + 1) // wl.m, P_cap).sum())
    csa_us = us["csa_attn"] + us.get("csa_combine", 0.0)
    hca_us = us["hca_attn"] + us.get("hca_combine", 0.0)
    index_us = us["threshold"] + us["score"] + us["select"]
    kern_us = us["append"] + index_us + csa_us + hca_us

    def tf(flop, t_us):
        return round(flop / (t_us * 1e-6) / 1e12, 1)
    out = {
        "workload": wl.name, "chunk_tokens": n, "cache_tokens": T0, "H": wl.H, "top_k": wl.k, "W": wl.W,
        "step_us": round(step_us, 2), "kernels_us": {k_: round(v, 2) for k_, v in us.items()},
        "kernel_sum_us": round(kern_us, 2),
        "prefill_tokens_per_s": round(n / (step_us * 1e-6), 1),
        "prefill_tokens_per_s_kernels": round(n / (kern_us * 1e-6), 1),
        "csa_attn": {"algorithmic_flop": csa_flop, "us": round(csa_us, 2), "tflops": tf(csa_flop, csa_us),
                     "peak_tflops": BF16_PEAK_TFLOPS, "frac": round(csa_flop / (csa_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                     "gathered_bytes": int((k_eff + win).sum()) * 2 * wl.d * 2,
                     "gather_GB/s": round(float((k_eff + win).sum()) * 2 * wl.d * 2 / (csa_us * 1e-6) / 1e9, 1)},
        "hca_attn": {"algorithmic_flop": hca_flop, "us": round(hca_us, 2), "tflops": tf(hca_flop, hca_us),
                     "peak_tflops": BF16_PEAK_TFLOPS, "frac": round(hca_flop / (hca_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "indexer": {"algorithmic_flop": idx_flop, "scoring_kernel_us": round(us["score"], 2),
                    "scoring_tflops": tf(idx_flop, us["score"]), "peak_tflops": FP4_PEAK_TFLOPS,
                    "scoring_frac": round(idx_flop / (us["score"] * 1e-6) / 1e12 / FP4_PEAK_TFLOPS, 4),
                    "index_topk_us": round(index_us, 2),
                    "index_topk_queries_per_s": round(wl.n_q / (index_us * 1e-6), 1)},
        "timing": "median of %d eager steps; kernel times from events attached to each dispatch" % reps,
        "graph": graph,
    }
    # the oracle beside it, on a few of the same queries (fp64 pooled caches prebuilt, not timed)
    try:
        import oracle
        kv, z = host["kv"], host["z"]
        pooled64, hpooled64 = oracle.pool(kv, z, wl.m), oracle.pool(kv, z, wl.m_hca)
        rows = np.linspace(0, wl.n_q - 1, oracle_queries).astype(int)

        def one(r):
            tq = int(q_pos[r])
            oracle.csa_query(kv, z, host["q"][r], tq, wl.m, wl.W, wl.k, scale, host["qc"][r], host["qs"][r],
                             host["w"][r], host["kc"], host["ks"], pooled=pooled64)
            oracle.hca_query(kv, z, host["q"][r], tq, wl.m_hca, wl.W_hca, scale, hpooled=hpooled64)
        t0_ = time.time()
        for r in rows:
            one(r)
        dt1 = time.time() - t0_
        nthr = host_threads()
        t0_ = time.time()
        with ThreadPoolExecutor(max_workers=nthr) as ex:
            list(ex.map(one, [rows[i % len(rows)] for i in range(max(nthr, len(rows)))]))
        dtn = time.time() - t0_
        nq_n = max(nthr, len(rows))
        out["oracle"] = {"queries": int(len(rows)), "single_thread_queries_per_s": round(len(rows) / dt1, 2),
                         "threads": nthr, "all_threads_queries_per_s": round(nq_n / dtn, 2),
                         "sample": "CSA (exact scores of every visible entry, full sort, attention over the selected "
                                   "fp64 pooled rows and the window) and HCA attention for evenly spaced queries of "
                                   "the chunk; the fp64 pooled caches are built first and not timed"}
    except Exception as e:  # reported, never silently replaced
        out["oracle"] = {"error": repr(e)}
    log(f"prefill chunk: {out}")
    return out


def bench_peaks(torch, csa, step_bytes, log, R: int = 20):
    """Measured peaks of this part (the peaks/ reference kernels, events on
    each dispatch): (1) HBM read of the decode step's byte count, R buffers
    read in turn so that no launch finds its data in the Infinity Cache, best
    median over grid sizes and loads in flight, and the sustained rate of a
    1 GiB read; (2) dense FP4 MFMA (32x32x64, block-scaled) and bf16 MFMA
    (16x16x32 and 32x32x16) rates, best over grid sizes."""
    import peaks
    L = peaks.lib()
    dev = "cuda"
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = (int(step_bytes) + 15) // 16 * 16
    bufs = [torch.full((nbytes,), r, dtype=torch.uint8, device=dev) for r in range(R)]
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=dev)
    out = {"read_bytes": nbytes, "read_buffers": R}
    sweep = {}
    best = None
    modes = {"strided": L.peak_read, "chunked": L.peak_read_chunked}
    for mode, fn in modes.items():
        for grid in (256, 512, 1024, 2048, 4096):
            for unroll in (8, 16):
                ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(3 * R)]
                for i, (e0, e1) in enumerate(ev):
                    rc = fn(bufs[i % R].data_ptr(), nbytes, grid, unroll, sink.data_ptr(), e0.handle, e1.handle, stream)
                    assert rc == 0, "peak_read launch failed"
                torch.cuda.synchronize()
                us = float(np.median([a.elapsed_ms(b) * 1e3 for a, b in ev[R:]]))
                sweep[f"{mode}_grid{grid}_u{unroll}"] = round(us, 2)
                if best is None or us < best[0]:
                    best = (us, grid, unroll, mode)
    out["read_us"] = {"best": round(best[0], 2), "grid": best[1], "unroll": best[2], "mode": best[3], "sweep": sweep}
    out["hbm_read_GB/s"] = round(nbytes / (best[0] * 1e-6) / 1e9, 1)
    del bufs
    big = torch.full((1 << 30,), 7, dtype=torch.uint8, device=dev)
    big_rates = {}
    for mode, fn in modes.items():
        for grid, unroll in ((4096, 8), (2048, 16), (1024, 16)):
            ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(6)]
            for e0, e1 in ev:
                assert fn(big.data_ptr(), 1 << 30, grid, unroll, sink.data_ptr(), e0.handle, e1.handle, stream) == 0
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_ms(b) * 1e3 for a, b in ev[1:]]))
            big_rates[f"{mode}_grid{grid}_u{unroll}"] = round((1 << 30) / (us * 1e-6) / 1e9, 1)
    out["hbm_read_1GiB_GB/s"] = max(big_rates.values())
    out["hbm_read_1GiB_sweep_GB/s"] = big_rates
    del big
    fsink = torch.zeros(4096 * 256, dtype=torch.float32, device=dev)

    def mfma_rate(fn, flop_per_inst, iters=4000):
        best_tf, best_grid = 0.0, 0
        for grid in (256, 512, 1024, 2048):
            ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(3)]
            for e0, e1 in ev:
                assert fn(grid, iters, e0, e1) == 0, "MFMA peak launch failed"
            torch.cuda.synchronize()
            ms = float(np.median([a.elapsed_ms(b) for a, b in ev[1:]]))
            tf = grid * 4 * iters * 4 * flop_per_inst / (ms * 1e-3) / 1e12
            if tf > best_tf:
                best_tf, best_grid = tf, grid
        return round(best_tf, 1), best_grid
    fp4, g4 = mfma_rate(lambda g, it, e0, e1: L.peak_mfma_fp4(g, it, fsink.data_ptr(), e0.handle, e1.handle, stream),
                        peaks.FLOP_FP4_MFMA)
    b16s, gs = mfma_rate(lambda g, it, e0, e1: L.peak_mfma_bf16(g, it, 0, fsink.data_ptr(), e0.handle, e1.handle,
                                                                stream), peaks.FLOP_BF16_SMALL)
    b16b, gb = mfma_rate(lambda g, it, e0, e1: L.peak_mfma_bf16(g, it, 1, fsink.data_ptr(), e0.handle, e1.handle,
                                                                stream), peaks.FLOP_BF16_BIG)
    ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(21)]
    for e0, e1 in ev:  # the floor of a launch's measured duration (4 workgroups of 1024 threads)
        assert L.peak_empty(4, 1024, sink.data_ptr(), e0.handle, e1.handle, stream) == 0
    torch.cuda.synchronize()
    out["empty_kernel_us"] = round(float(np.median([a.elapsed_ms(b) * 1e3 for a, b in ev[1:]])), 2)
    # VALU issue: 64 x 256 adds per wave, one workgroup per CU of 1, 4 or 16 waves
    valu = {}
    for block in (64, 256, 1024):
        ev = [(csa.HipEvent(), csa.HipEvent()) for _ in range(6)]
        for e0, e1 in ev:
            assert L.peak_valu(256, block, 64, sink.data_ptr(), e0.handle, e1.handle, stream) == 0
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_ms(b) * 1e3 for a, b in ev[1:]]))
        per_wave = 64 * 256
        valu[f"waves_per_cu_{block // 64}"] = {
            "us": round(us, 2),
            "ns_per_instr_per_wave": round((us - out["empty_kernel_us"]) * 1e3 / per_wave, 3)}
    out["valu_issue"] = valu
    out["fp4_mfma_TFLOP/s"] = fp4
    out["bf16_mfma_16x16x32_TFLOP/s"] = b16s
    out["bf16_mfma_32x32x16_TFLOP/s"] = b16b
    out["bf16_mfma_TFLOP/s"] = max(b16s, b16b)
    out["mfma_grids"] = {"fp4": g4, "bf16_16x16x32": gs, "bf16_32x32x16": gb}
    out["datasheet"] = {"hbm_GB/s": HBM_PEAK_GBS, "fp4_TFLOP/s": FP4_PEAK_TFLOPS, "bf16_TFLOP/s": BF16_PEAK_TFLOPS}
    log(f"measured peaks: {out}")
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    """Threads the oracle may use: the CPUs this process may run on, at most 16
    (a one-GPU machine's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(wl, host, log, min_seconds: float = 10.0, single_seconds: float = 4.0):
    """The oracle, as it stands, on the decode queries of the same workload:
    every host thread this process may use (the 4 queries repeated to fill
    them), then one thread alone.  The oracle's fp64 HCA caches are built first
    and not timed, as the GPU's pooled caches are not."""
    import oracle
    n = wl.n_q
    seqs = np.repeat(np.arange(wl.B), np.diff(host["q_off"]))
    scale = 1.0 / math.sqrt(wl.d)
    threads = host_threads()

    def seq_rows(b):
        t0, t1 = int(host["tok_off"][b]), int(host["tok_off"][b + 1])
        return host["kv"][t0:t1], host["z"][t0:t1]

    log(f"cpu baseline: building oracle HCA caches for {n} queries")
    with ThreadPoolExecutor(max_workers=min(threads, n)) as ex:
        hp = list(ex.map(lambda r: oracle.pool(*seq_rows(seqs[r]), wl.m_hca), range(n)))

    def one(r):
        b = seqs[r]
        kv, z = seq_rows(b)
        p0, p1 = int(host["pool_off"][b]), int(host["pool_off"][b + 1])
        t = int(host["q_pos"][r])
        oracle.csa_query(kv, z, host["q"][r], t, wl.m, wl.W, wl.k, scale, host["qc"][r], host["qs"][r],
                         host["w"][r], host["kc"][p0:p1], host["ks"][p0:p1])
        oracle.hca_query(kv, z, host["q"][r], t, wl.m_hca, wl.W_hca, scale, hpooled=hp[r])

    tasks = [i % n for i in range(max(threads, n))]
    log(f"cpu baseline: the oracle on {len(tasks)} query tasks with {threads} threads, at least {min_seconds} s")
    t = time.time()
    done = 0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while done == 0 or time.time() - t < min_seconds:
            list(ex.map(one, tasks))
            done += len(tasks)
    dt = time.time() - t
    t = time.time()
    single = 0
    while single == 0 or time.time() - t < single_seconds:
        one(single % n)
        single += 1
    dt1 = time.time() - t
    log(f"cpu baseline: {done} queries in {dt:.2f} s on {threads} threads; {single} in {dt1:.2f} s on one")
    return {"value": round(done / dt, 4), "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} decode queries of {wl.name} ({n} distinct, repeated to fill {threads} threads; CSA: "
                      f"exact MXFP4 scores of every visible pooled entry, full-sort top-{wl.k}, fp64 pooling of the "
                      f"selected blocks, attention; HCA: attention over the oracle's prebuilt fp64 cache)",
            "seconds": round(dt, 3), "single_thread": {"value": round(single / dt1, 4), "queries": single,
                                                        "seconds": round(dt1, 3)},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
