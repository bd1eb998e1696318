"""The inclusion-exclusion route (three attention passes merged by their LSE,
the pages' own algorithm in "Inference Efficiency Mechanisms") on the GPU vs
the fp64 oracle's bifocal attention, and a cancellation study against the
tile-routed kernels.

Tolerances as in test_gpu_parity: fp32 1e-4, bf16 2e-2 (max abs, O and LSE).
"""
import os

import numpy as np
import pytest

import oracle
import zero_shot_rope_bifocal_amd as jl
from zero_shot_rope_bifocal_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


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


def _run(fn, inp, wp, w0, theta, prerotated=False, q=None, k=None):
    torch = _torch()
    dt = inp["dtype"]
    qd = W.to_device(inp["q"] if q is None else q, dt)
    kd = W.to_device(inp["k"] if k is None else k, dt)
    vd = W.to_device(inp["v"], dt)
    cu_q = torch.from_numpy(inp["cu_q"]).cuda()
    cu_k = torch.from_numpy(inp["cu_k"]).cuda()
    out, lse = fn(qd, kd, vd, cu_q, max(inp["q_lens"]), wp, w0, theta, cu_seqlens_k=cu_k,
                  max_seqlen_k=max(inp["lens"]), return_lse=True, prerotated=prerotated)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64).T


def _oracle(inp, wp, w0, theta):
    dt = inp["dtype"]
    cq, ck = inp["cu_q"], inp["cu_k"]
    outs, lses = [], []
    for b, (L, Lq) in enumerate(zip(inp["lens"], inp["q_lens"])):
        o, s = oracle.bifocal_sequence(W.as_f64(inp["q"][cq[b]:cq[b + 1]], dt), W.as_f64(inp["k"][ck[b]:ck[b + 1]], dt),
                                       W.as_f64(inp["v"][ck[b]:ck[b + 1]], dt), np.arange(L - Lq, L), L, wp, w0, theta)
        outs.append(o)
        lses.append(s)
    return np.concatenate(outs), np.concatenate(lses)


CASES = [
    # (lens, q_lens, Hq, Hkv, d, dtype, wp, w0, theta, seed)
    ([1500], None, 8, 2, 128, "bf16", 512, 128, 1e6, 81),                # G = 3, GQA 4
    ([777, 64, 1, 1300], None, 8, 2, 128, "bf16", 256, 200, 1e4, 82),    # ragged varlen
    ([1000], None, 4, 2, 64, "bf16", 300, 0, 1e4, 83),                   # w0 = 0: window passes empty
    ([900], None, 4, 4, 128, "bf16", 128, 5000, 1e4, 84),                # w0 >= L: full pass cancels out
    ([1200, 700], [130, 700], 16, 2, 128, "bf16", 256, 100, 1e4, 85),    # chunk of a longer prefill, GQA 8
    ([513, 70], None, 2, 1, 64, "f32", 128, 33, 1e4, 86),
    ([300], None, 4, 2, 128, "f32", 64, 50, 1e4, 87),
    ([65], None, 4, 1, 128, "bf16", 32, 1, 10.0, 88),                    # window 1
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_prefill_ie_matches_oracle(case):
    _torch()
    lens, q_lens, Hq, Hkv, d, dt, wp, w0, theta, seed = case
    _say("prefill_ie", case)
    inp = W.prefill_inputs(lens, Hq, Hkv, d, dt, seed, q_lens=q_lens)
    o_gpu, l_gpu = _run(jl.prefill_ie, inp, wp, w0, theta)
    o_ref, l_ref = _oracle(inp, wp, w0, theta)
    eo, el = np.max(np.abs(o_gpu - o_ref)), np.max(np.abs(l_gpu - l_ref))
    _say(f"max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert np.all(np.isfinite(o_gpu))
    assert eo <= TOL[dt], eo
    assert el <= TOL[dt], el


def test_prefill_ie_prerotated_matches_routed():
    """With a pre-rotated cache both routes apply the same correction rotation."""
    _torch()
    _say("prefill_ie prerotated")
    L, wp, w0, theta = 1100, 256, 90, 1e4
    inp = W.prefill_inputs([L], 8, 2, 128, "bf16", 89)
    pos = np.arange(L)
    rot = lambda x: np.stack([oracle.rope_rotate(x[:, h], pos, theta) for h in range(x.shape[1])], axis=1)  # noqa: E731
    q = W.bf16_bits(rot(W.as_f64(inp["q"], "bf16")).astype(np.float32))
    k = W.bf16_bits(rot(W.as_f64(inp["k"], "bf16")).astype(np.float32))
    o_ie, l_ie = _run(jl.prefill_ie, inp, wp, w0, theta, prerotated=True, q=q, k=k)
    o_rt, l_rt = _run(jl.prefill, inp, wp, w0, theta, prerotated=True, q=q, k=k)
    o_ref, l_ref = oracle.bifocal_sequence_prerotated(W.as_f64(q, "bf16"), W.as_f64(k, "bf16"),
                                                      W.as_f64(inp["v"], "bf16"), pos, L, wp, w0, theta)
    for name, o, s in (("ie", o_ie, l_ie), ("routed", o_rt, l_rt)):
        eo, el = np.max(np.abs(o - o_ref)), np.max(np.abs(s - l_ref))
        _say(f"{name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= TOL["bf16"] and el <= TOL["bf16"], (name, eo, el)


def planted_cancellation(L, d, wp, w0, theta, c, dt, seed=90):
    """One head; the last query has all its energy in the fastest rotation
    pair (angle = position in radians).  The window keys whose local angle
    to that query is nearly opposite to their grouped-position angle are set
    to c * R(f(i) - f(j)) q_i: at the grouped positions they align with the
    query (logit c / sqrt(d)), at the true positions they point away.  So the
    window holds almost all of the full grouped-position mass (pass 2) and
    pass 3 takes it out again: w2 - w3 cancels, kappa = exp(LSE_2 - LSE)
    large."""
    inp = W.prefill_inputs([L], 1, 1, d, dt, seed)
    G = oracle.group_size(L, wp)
    i = L - 1
    qi = np.zeros(d)
    qi[0] = 1.0
    q = W.as_f64(inp["q"], dt)
    k = W.as_f64(inp["k"], dt)
    q[i, 0] = qi
    for j in range(max(0, i - w0 + 1), i):
        if np.cos((j - i) - (j // G - i // G)) < -0.8:
            k[j, 0] = c * oracle.rope_rotate(qi[None], np.array([i // G - j // G]), theta)[0]
    store = (lambda x: W.bf16_bits(x.astype(np.float32))) if dt == "bf16" else (lambda x: x.astype(np.float32))
    inp["q"], inp["k"] = store(q), store(k)
    return inp


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_ie_cancellation_study(dt):
    """Error on the planted row as kappa grows: the routed kernel never forms
    w2 - w3 and stays within tolerance; the merged route loses ~eps * kappa
    and is wrong (or not finite) at the largest plant."""
    _torch()
    L, d, wp, w0, theta = 1024, 64, 256, 64, 1e4
    errs = []
    for c in (16, 64, 96, 128, 160):
        inp = planted_cancellation(L, d, wp, w0, theta, c, dt)
        o_ref, l_ref = _oracle(inp, wp, w0, theta)
        _, l2 = oracle.bifocal_sequence(W.as_f64(inp["q"][-1:], dt), W.as_f64(inp["k"], dt), W.as_f64(inp["v"], dt),
                                        np.array([L - 1]), L, wp, 0, theta)   # w0 = 0: the full grouped pass
        kappa = float(np.exp(l2[0, 0] - l_ref[-1, 0]))
        row = []
        for fn in (jl.prefill, jl.prefill_ie):
            o, s = _run(fn, inp, wp, w0, theta)
            e = max(np.max(np.abs(o[-1] - o_ref[-1])), np.max(np.abs(s[-1] - l_ref[-1])))
            row.append(float(e) if np.isfinite(e) else float("inf"))
        _say(f"{dt} c={c} kappa={kappa:.2e}: routed err {row[0]:.2e}  inclusion-exclusion err {row[1]:.2e}")
        errs.append((kappa, *row))
    assert all(r <= TOL[dt] for _, r, _ in errs), errs
    assert errs[-1][2] > TOL[dt], errs
