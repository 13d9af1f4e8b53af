"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same seeded inputs, and compare.

Tolerances: top-k indices bit-exact; fp32 outputs max-abs <= 1e-5; bf16
outputs max-abs <= 2e-2 and relative L2 (over the whole output) <= 5e-3.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

import oracle
import synth

FP32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return synth.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def torch_to_np(t) -> np.ndarray:
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def check_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    g = as_f64(got) if got.dtype != np.float64 else got
    finite = np.isfinite(want)
    assert np.array_equal(np.isfinite(g), finite), f"{what}: non-finite pattern differs"
    assert np.array_equal(g[~finite], want[~finite]), f"{what}: non-finite values differ"
    diff = g[finite] - want[finite]
    err = np.abs(diff)
    max_abs = float(err.max()) if err.size else 0.0
    if dtype == "f32":
        assert max_abs <= FP32_MAX_ABS, f"{what}: max-abs {max_abs:.3g} > {FP32_MAX_ABS}"
    else:
        den = float(np.linalg.norm(want[finite]))
        rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(err))
        assert max_abs <= BF16_MAX_ABS, f"{what}: max-abs {max_abs:.3g} > {BF16_MAX_ABS}"
        assert rel <= BF16_REL_L2, f"{what}: rel-L2 {rel:.3g} > {BF16_REL_L2}"
    return max_abs


def seq_slices(host, b):
    t0, t1 = int(host["tok_off"][b]), int(host["tok_off"][b + 1])
    p0, p1 = int(host["pool_off"][b]), int(host["pool_off"][b + 1])
    q0, q1 = int(host["q_off"][b]), int(host["q_off"][b + 1])
    return (t0, t1), (p0, p1), (q0, q1)


def oracle_topk_row(host, wl: synth.Workload, row: int, b: int, k: int, m: int) -> np.ndarray:
    (_, _), (p0, p1), _ = seq_slices(host, b)
    t = int(host["q_pos"][row])
    n_vis = min((t + 1) // m, p1 - p0)
    S, ex = oracle.index_scores(host["qc"][row], host["qs"][row], host["w"][row],
                                host["kc"][p0:p0 + n_vis], host["ks"][p0:p0 + n_vis])
    assert ex.all(), "fp32 exactness precondition violated by the generated inputs"
    return oracle.topk(S, k)


def row_seq(host) -> List[int]:
    q_off = host["q_off"]
    out = []
    for b in range(len(q_off) - 1):
        out += [b] * int(q_off[b + 1] - q_off[b])
    return out
