"""Run by tests/test_gpu_debug_checks.py in a process of its own with
CSA_LIBRARY=debug, so that the binding loads libcsa_debug.so: the kernels
with device-side index checks.  Prints one JSON line with what it found."""
import json
import math
import sys

import numpy as np
import torch

import oracle
import synth
from tests import _parity as P


def main():
    import long_context_compressed_05_amd as csa
    assert csa.LIB_PATH.endswith("libcsa_debug.so"), csa.LIB_PATH
    csa.lib()
    out = {"lib": csa.LIB_PATH.rsplit("/", 1)[-1]}
    assert csa.csa_debug_checks() == 0
    from long_context_compressed_05_amd.step import Layer, Params, to_device
    # (1) the fused decode step on ragged rows: no violation, top-k against the oracle
    wl = synth.Workload("debug_decode", [1030, 4099, 2049], [1029, 4098, 2048], H=64, dtype="bf16", k=64, W=128,
                        m=4, m_hca=128, seed=77)
    host = synth.make_inputs(wl)
    layer = Layer.from_host(Params(H=wl.H, d=wl.d, m=wl.m, k=wl.k, W=wl.W, m_hca=wl.m_hca), host, "cuda")
    layer.build_caches()
    dq = to_device({k: host[k] for k in ("q", "qc", "qs", "w")})
    idx, co, cl, ho, hl = layer.decode_fused(dq["q"], dq["qc"], dq["qs"], dq["w"])
    layer.check_fused()
    torch.cuda.synchronize()
    got = P.torch_to_np(idx)
    seqs = P.row_seq(host)
    for r in range(wl.n_q):
        assert np.array_equal(got[r], P.oracle_topk_row(host, wl, r, seqs[r], wl.k, wl.m)), f"row {r}"
    out["fused_violations"] = csa.csa_debug_checks()
    # (2) csa_sparse_attn with valid indices, then with two out-of-range ones in
    # row 0 (sequence 0's pooled count + 3, a row of sequence 1's segment in
    # memory): counted, and the result equals that of padding (-1) there
    pool_off = torch.from_numpy(host["pool_off"]).cuda()
    batch = csa.Batch.from_host(host["tok_off"], host["q_off"], host["q_pos"])
    scale = 1 / math.sqrt(wl.d)
    sidx = idx.clone()
    o_ok, l_ok = csa.csa_sparse_attn(batch, pool_off, dq["q"], layer.pooled, layer.kv, sidx, wl.W, scale)
    torch.cuda.synchronize()
    out["valid_violations"] = csa.csa_debug_checks()
    P0 = int(host["pool_off"][1] - host["pool_off"][0])
    bad = sidx.clone()
    bad[0, 3] = P0 + 3
    bad[0, 7] = P0 + 3
    pad = sidx.clone()
    pad[0, 3] = -1
    pad[0, 7] = -1
    # padding must come after the valid entries: move the -1 entries to the end
    row = pad[0][pad[0] >= 0]
    pad[0] = torch.cat([row, torch.full((wl.k - row.numel(),), -1, dtype=pad.dtype, device=pad.device)])
    rowb = bad[0][(bad[0] >= 0) & (bad[0] < P0)]
    bad[0] = torch.cat([rowb, torch.tensor([P0 + 3, P0 + 3], dtype=bad.dtype, device=bad.device),
                        torch.full((wl.k - rowb.numel() - 2,), -1, dtype=bad.dtype, device=bad.device)])
    o_bad, l_bad = csa.csa_sparse_attn(batch, pool_off, dq["q"], layer.pooled, layer.kv, bad, wl.W, scale)
    torch.cuda.synchronize()
    out["bad_violations"] = csa.csa_debug_checks()
    o_pad, l_pad = csa.csa_sparse_attn(batch, pool_off, dq["q"], layer.pooled, layer.kv, pad, wl.W, scale)
    torch.cuda.synchronize()
    out["pad_violations"] = csa.csa_debug_checks()
    out["bad_equals_pad"] = bool(torch.equal(o_bad, o_pad) and torch.equal(l_bad, l_pad))
    out["other_rows_unchanged"] = bool(torch.equal(o_bad[1:], o_ok[1:]))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
    sys.exit(0)
