"""Pre-rotated convention (queries and keys handed over already rotated at
their true positions, the usual RoPE cache) on the GPU vs the fp64 oracle's
correction-rotation formulation.  The stored rotated values are generated on
the host from seeded raw inputs (fp64 rotation, then rounded to the storage
type); the oracle reads exactly the stored values.

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


def _store(x64, dt):
    """fp64 values -> the stored representation of dtype dt."""
    return W.bf16_bits(x64.astype(np.float32)) if dt == "bf16" else x64.astype(np.float32)


def _rotate_rows(x, pos, theta):
    """R(pos[i]) applied to every head of row i; x [n, H, d] fp64."""
    return np.stack([oracle.rope_rotate(x[:, h], pos, theta) for h in range(x.shape[1])], axis=1)


PREFILL_CASES = [
    # (lens, q_lens, Hq, Hkv, d, dtype, wp, w0, theta, seed)
    ([3000, 1000], None, 8, 2, 128, "bf16", 512, 300, 1e6, 61),
    ([1500], [400], 4, 4, 64, "bf16", 256, 0, 1e4, 62),            # chunk of a longer prefill, all remote
    ([900, 65], None, 4, 2, 64, "f32", 128, 100, 1e4, 63),
    ([700], None, 2, 1, 128, "bf16", 128, 2000, 1e4, 64),         # w0 >= L: all local, no rotation at all
]




def _random_prefill_cases(n, seed):
    """Seeded extra cases: ragged lengths, optional query chunks, GQA ratios
    1..8, d 64 / 128, windows from 0 to beyond L."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        lens = [int(x) for x in rng.integers(2, 1300, size=B)]
        q_lens = None if i % 2 else [int(rng.integers(1, L + 1)) for L in lens]
        Hkv = int(rng.choice([1, 2]))
        ratio = int(rng.choice([1, 2, 3, 4, 8]))
        Lmax = max(lens)
        out.append((lens, q_lens, Hkv * ratio, Hkv, int(rng.choice([64, 128])), "bf16" if i % 3 else "f32",
                    int(rng.integers(max(1, Lmax // 6), Lmax + 100)), int(rng.choice([0, 1, int(rng.integers(2, 300)), Lmax + 3])),
                    float(rng.choice([1e4, 1e6])), 300 + i))
    return out


PREFILL_CASES += _random_prefill_cases(6, 2026)


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[f"case{i}" for i in range(len(PREFILL_CASES))])
def test_prefill_prerotated(case):
    torch = _torch()
    lens, q_lens, Hq, Hkv, d, dt, wp, w0, theta, seed = case
    _say("prefill prerotated", case)
    inp = W.prefill_inputs(lens, Hq, Hkv, d, dt, seed, q_lens=q_lens)
    cq, ck = inp["cu_q"], inp["cu_k"]
    qs, ks = [], []
    for b, (L, Lq) in enumerate(zip(inp["lens"], inp["q_lens"])):
        qs.append(_rotate_rows(W.as_f64(inp["q"][cq[b]:cq[b + 1]], dt), np.arange(L - Lq, L), theta))
        ks.append(_rotate_rows(W.as_f64(inp["k"][ck[b]:ck[b + 1]], dt), np.arange(L), theta))
    q_st, k_st = _store(np.concatenate(qs), dt), _store(np.concatenate(ks), dt)
    q = W.to_device(q_st, dt)
    k = W.to_device(k_st, dt)
    v = W.to_device(inp["v"], dt)
    cu_q = torch.from_numpy(cq).cuda()
    cu_k = torch.from_numpy(ck).cuda()
    out, lse = jl.prefill(q, k, v, cu_q, max(inp["q_lens"]), wp, w0, theta, cu_seqlens_k=cu_k,
                          max_seqlen_k=max(inp["lens"]), return_lse=True, prerotated=True)
    torch.cuda.synchronize()
    o_gpu = out.float().cpu().numpy()
    l_gpu = lse.cpu().numpy().T
    worst = 0.0
    for b, (L, Lq) in enumerate(zip(inp["lens"], inp["q_lens"])):
        o_ref, l_ref = oracle.bifocal_sequence_prerotated(
            W.as_f64(q_st[cq[b]:cq[b + 1]], dt), W.as_f64(k_st[ck[b]:ck[b + 1]], dt),
            W.as_f64(inp["v"][ck[b]:ck[b + 1]], dt), np.arange(L - Lq, L), L, wp, w0, theta)
        worst = max(worst, np.max(np.abs(o_gpu[cq[b]:cq[b + 1]] - o_ref)),
                    np.max(np.abs(l_gpu[cq[b]:cq[b + 1]] - l_ref)))
    _say(f"max err {worst:.3e}")
    assert np.all(np.isfinite(o_gpu))
    assert worst <= TOL[dt], worst


DECODE_CASES = [
    # (B, S, seq_L, Hq, Hkv, d, dtype, wp, w0, theta, seed)
    (4, 3000, [3000, 1, 2049, 777], 32, 8, 128, "bf16", 512, 256, 1e6, 71),
    (2, 1000, [1000, 333], 8, 2, 64, "bf16", 200, 0, 1e4, 72),
    (3, 800, [800, 65, 5], 8, 2, 128, "f32", 100, 50, 1e4, 73),
    (7, 1024, [255, 256, 257, 512, 513, 768, 769], 8, 2, 128, "bf16", 256, 64, 1e4, 75),  # G 1..4
]




def _random_decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        S = int(rng.integers(8, 2500))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        ratio = int(rng.choice([1, 2, 4, 6, 8]))
        out.append((B, S, [int(x) for x in rng.integers(1, S + 1, size=B)], Hkv * ratio, Hkv, int(rng.choice([64, 128])),
                    "bf16" if i % 3 else "f32", int(rng.integers(max(1, S // 6), S + 100)),
                    int(rng.choice([0, 1, int(rng.integers(2, 500)), S + 3])), float(rng.choice([1e4, 1e6])), 400 + i))
    return out


DECODE_CASES += _random_decode_cases(6, 2027)


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"case{i}" for i in range(len(DECODE_CASES))])
def test_decode_prerotated(case):
    torch = _torch()
    B, S, seq_L, Hq, Hkv, d, dt, wp, w0, theta, seed = case
    _say("decode prerotated", case)
    inp = W.decode_inputs(B, S, Hq, Hkv, d, dt, seed, seq_L=seq_L)
    q64 = W.as_f64(inp["q"], dt)
    k64 = W.as_f64(inp["k"], dt)
    q_rot = np.stack([_rotate_rows(q64[b:b + 1], [int(seq_L[b]) - 1], theta)[0] for b in range(B)])
    k_rot = np.stack([_rotate_rows(k64[b], np.arange(S), theta) for b in range(B)])
    q_st, k_st = _store(q_rot, dt), _store(k_rot, dt)
    q = W.to_device(q_st, dt)
    k = W.to_device(k_st, dt)
    v = W.to_device(inp["v"], dt)
    seq = torch.from_numpy(inp["seq_L"]).cuda()
    out, lse = jl.decode(q, k, v, seq, wp, w0, theta, return_lse=True, prerotated=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.bifocal_decode_prerotated(W.as_f64(q_st, dt), W.as_f64(k_st, dt), W.as_f64(inp["v"], dt),
                                                    inp["seq_L"], wp, w0, theta)
    err_o = np.max(np.abs(out.float().cpu().numpy() - o_ref))
    err_l = np.max(np.abs(lse.cpu().numpy() - l_ref))
    _say(f"max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= TOL[dt], err_o
    assert err_l <= TOL[dt], err_l


def test_prerotated_matches_raw_convention():
    """The same attention handed over raw and pre-rotated (fp32, so the stored
    rotation adds only fp32 rounding) agrees on the GPU."""
    torch = _torch()
    _say("prerotated vs raw")
    L, Hq, Hkv, d, wp, w0, theta = 1200, 4, 2, 64, 256, 100, 1e4
    inp = W.prefill_inputs([L], Hq, Hkv, d, "f32", 74)
    pos = np.arange(L)
    q_rot = _rotate_rows(W.as_f64(inp["q"], "f32"), pos, theta).astype(np.float32)
    k_rot = _rotate_rows(W.as_f64(inp["k"], "f32"), pos, theta).astype(np.float32)
    cu = torch.from_numpy(inp["cu_q"]).cuda()
    v = torch.from_numpy(inp["v"]).cuda()
    raw = jl.prefill(torch.from_numpy(inp["q"]).cuda(), torch.from_numpy(inp["k"]).cuda(), v, cu, L, wp, w0, theta)
    rot = jl.prefill(torch.from_numpy(q_rot).cuda(), torch.from_numpy(k_rot).cuda(), v, cu, L, wp, w0, theta,
                     prerotated=True)
    torch.cuda.synchronize()
    err = float((raw - rot).abs().max())
    _say(f"max|raw - prerotated| = {err:.3e}")
    assert err <= 1e-4
