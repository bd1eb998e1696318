"""Full-size workloads on the GPU, in the launch configuration bench.py times,
checked against the fp64 oracle on stratified sampled query rows (first
rows, rows around w0 and around every multiple of w_pretrained, last rows,
seeded random rows; all heads).  Decode is checked in full.

Tolerance: max abs error 2e-2 on O and LSE (bf16 outputs).
"""
import concurrent.futures as cf
import os

import numpy as np
import pytest

import oracle
import zero_shot_rope_bifocal_amd as jl
from zero_shot_rope_bifocal_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
TOL = 2e-2


def _torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _say(*a):
    print("[case]", *a, flush=True)
    log = os.environ.get("JL_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            print(os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], *a, file=f)


def oracle_rows_parallel(q_rows, k, v, rows, L, wp, w0, theta, Hq, Hkv):
    """Oracle on the given rows, one KV head (and its query heads) per thread."""
    rep = Hq // Hkv

    def one(hk):
        hs = slice(hk * rep, (hk + 1) * rep)
        return oracle.bifocal_sequence(q_rows[:, hs], k[:, hk:hk + 1], v[:, hk:hk + 1], rows, L, wp, w0, theta)

    with cf.ThreadPoolExecutor(min(Hkv, 16)) as ex:
        parts = list(ex.map(one, range(Hkv)))
    return np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=1)


def run_and_check_prefill(name, n_edge=32, n_rand=96):
    torch = _torch()
    w = W.WORKLOADS[name]
    _say(name, "generating")
    inp = W.workload_inputs(name)
    dev = "cuda"
    q = W.to_device(inp["q"], "bf16", dev)
    k = W.to_device(inp["k"], "bf16", dev)
    v = W.to_device(inp["v"], "bf16", dev)
    cu = torch.from_numpy(inp["cu_q"]).to(dev)
    maxL = max(inp["lens"])
    _say(name, "gpu prefill")
    out, lse = jl.prefill(q, k, v, cu, maxL, w["w_pretrained"], w["w0"], w["theta"], return_lse=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    del q, k, v
    worst = 0.0
    for b, L in enumerate(inp["lens"]):
        a = int(inp["cu_q"][b])
        rows = W.sample_rows(L, w["w0"], w["w_pretrained"], seed=100 + b, n_edge=n_edge, n_rand=n_rand)
        _say(name, f"seq {b} L={L}: oracle on {rows.size} rows")
        qr = W.as_f64(inp["q"][a + rows], "bf16")
        kb = W.as_f64(inp["k"][a:a + L], "bf16")
        vb = W.as_f64(inp["v"][a:a + L], "bf16")
        o_ref, l_ref = oracle_rows_parallel(qr, kb, vb, rows, L, w["w_pretrained"], w["w0"], w["theta"],
                                            w["Hq"], w["Hkv"])
        idx = torch.from_numpy(a + rows).to(dev)
        o_gpu = out.index_select(0, idx).float().cpu().numpy()
        l_gpu = lse.index_select(1, idx).cpu().numpy().T
        eo = float(np.max(np.abs(o_gpu - o_ref)))
        el = float(np.max(np.abs(l_gpu - l_ref)))
        _say(name, f"seq {b}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        worst = max(worst, eo, el)
    assert worst <= TOL, worst


def test_short_fidelity_prefill_G1():
    """L = w_pretrained = 32768: G = 1, so the result is classic RoPE causal
    attention (the oracle's G = 1 reduction is pinned on the CPU)."""
    run_and_check_prefill("short_bf16")


def test_long_prefill_128k():
    run_and_check_prefill("long_bf16")


def test_ragged_varlen_prefill():
    run_and_check_prefill("ragged_bf16", n_edge=24, n_rand=64)


def test_decode_16x128k_full():
    torch = _torch()
    w = W.WORKLOADS["decode_bf16"]
    _say("decode_bf16 generating")
    inp = W.workload_inputs("decode_bf16")
    q = W.to_device(inp["q"], "bf16")
    k = W.to_device(inp["k"], "bf16")
    v = W.to_device(inp["v"], "bf16")
    seq = torch.from_numpy(inp["seq_L"]).cuda()
    _say("decode_bf16 gpu")
    out, lse = jl.decode(q, k, v, seq, w["w_pretrained"], w["w0"], w["theta"], return_lse=True)
    torch.cuda.synchronize()
    o_gpu = out.float().cpu().numpy()
    l_gpu = lse.cpu().numpy()
    del q, k, v
    worst = 0.0
    for b in range(w["B"]):
        L = int(inp["seq_L"][b])
        qb = W.as_f64(inp["q"][b:b + 1], "bf16")
        kb = W.as_f64(inp["k"][b, :L], "bf16")
        vb = W.as_f64(inp["v"][b, :L], "bf16")
        o_ref, l_ref = oracle_rows_parallel(qb, kb, vb, np.array([L - 1]), L, w["w_pretrained"], w["w0"],
                                            w["theta"], w["Hq"], w["Hkv"])
        eo = float(np.max(np.abs(o_gpu[b] - o_ref[0])))
        el = float(np.max(np.abs(l_gpu[b] - l_ref[0])))
        worst = max(worst, eo, el)
        if b % 4 == 0:
            _say(f"decode seq {b}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    _say(f"decode worst {worst:.3e}")
    assert worst <= TOL, worst
