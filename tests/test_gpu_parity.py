"""HIP path vs the fp64 oracle, element by element, at sizes the oracle
finishes in seconds (several tiles, ragged tails, GQA, edge cases).

Tolerances (stated on outputs after upcast): fp32 max abs error 1e-4 on O and
1e-4 on LSE; bf16 max abs error 2e-2 on O and LSE.  Integer maps are compared
bit-exactly.
"""
import hashlib
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


def run_prefill(inp, wp, w0, theta, max_q=None, max_k=None):
    torch = _torch()
    dt = inp["dtype"]
    q = W.to_device(inp["q"], dt)
    k = W.to_device(inp["k"], dt)
    v = W.to_device(inp["v"], dt)
    cu_q = torch.from_numpy(inp["cu_q"]).cuda()
    cu_k = torch.from_numpy(inp["cu_k"]).cuda()
    mq = max(inp["q_lens"]) if max_q is None else max_q
    mk = max(inp["lens"]) if max_k is None else max_k
    out, lse = jl.prefill(q, k, v, cu_q, mq, wp, w0, theta, cu_seqlens_k=cu_k, max_seqlen_k=mk,
                          return_lse=True)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_prefill(inp, wp, w0, theta, rows=None):
    dt = inp["dtype"]
    out, lse = [], []
    cq, ck = inp["cu_q"], inp["cu_k"]
    for b, (L, Lq) in enumerate(zip(inp["lens"], inp["q_lens"])):
        if Lq == 0:
            continue
        q = W.as_f64(inp["q"][cq[b]:cq[b + 1]], dt)
        k = W.as_f64(inp["k"][ck[b]:ck[b + 1]], dt)
        v = W.as_f64(inp["v"][ck[b]:ck[b + 1]], dt)
        pos = np.arange(L - Lq, L)
        o, s = oracle.bifocal_sequence(q, k, v, pos, L, wp, w0, theta)
        out.append(o)
        lse.append(s)
    return np.concatenate(out), np.concatenate(lse)


def check_prefill(inp, wp, w0, theta):
    dt = inp["dtype"]
    o_gpu, lse_gpu = run_prefill(inp, wp, w0, theta)
    o_ref, lse_ref = oracle_prefill(inp, wp, w0, theta)
    err_o = np.max(np.abs(o_gpu - o_ref))
    err_l = np.max(np.abs(lse_gpu.T - lse_ref))
    _say(f"max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert np.all(np.isfinite(o_gpu))
    assert err_o <= TOL[dt], err_o
    assert err_l <= TOL[dt], err_l


# ---------------------------------------------------------------- integers

@pytest.mark.parametrize("lens,q_lens,wp", [
    ([2048], None, 512), ([20000, 70000, 131072], None, 32768), ([5, 0, 1025, 64], None, 512),
    ([1000, 300], [7, 300], 128), ([1], None, 1),
])
def test_remote_positions_bit_exact(lens, q_lens, wp):
    torch = _torch()
    _say("remote_positions", lens, q_lens, wp)
    q_lens = lens if q_lens is None else q_lens
    cu_q = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32).cuda()
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32).cuda()
    pos, f, G = jl.remote_positions(cu_q, wp, cu_seqlens_k=cu_k)
    want_pos, want_f, want_G = [], [], []
    for L, Lq in zip(lens, q_lens):
        g = oracle.group_size(L, wp)
        p = np.arange(L - Lq, L)
        want_pos.append(p)
        want_f.append(oracle.remote_positions(p, g))
        want_G.append(g)
    assert np.array_equal(pos.cpu().numpy(), np.concatenate(want_pos))
    assert np.array_equal(f.cpu().numpy(), np.concatenate(want_f))
    assert G.cpu().numpy().tolist() == want_G


@pytest.mark.parametrize("Lq,L,w0,BM,BN", [
    (2048, 2048, 128, 64, 64), (2048, 2048, 128, 128, 64), (1000, 1000, 0, 64, 64),
    (1000, 1000, 5000, 64, 64), (777, 2000, 300, 64, 64), (8, 8, 3, 2, 2), (7, 7, 3, 2, 2),
    (4096, 4096, 2048, 64, 64), (300, 300, 64, 256, 64), (1, 1, 0, 64, 64),
])
def test_tile_classes_bit_exact(Lq, L, w0, BM, BN):
    _torch()
    _say("tile_classes", Lq, L, w0, BM, BN)
    got = jl.tile_classes(Lq, L, w0, BM, BN).cpu().numpy()
    want = oracle.tile_classes(Lq, L, L - Lq, w0, BM, BN)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- prefill

def test_prefill_f32_tiny_config():
    """2 heads, head_dim 64, L 2048, w_pretrained 512 (G = 4), w0 128, theta 1e4."""
    _torch()
    w = W.WORKLOADS["tiny_f32"]
    _say("tiny_f32 full")
    inp = W.workload_inputs("tiny_f32")
    check_prefill(inp, w["w_pretrained"], w["w0"], w["theta"])


PREFILL_CASES = [
    # (lens, Hq, Hkv, d, dtype, wp, w0, theta, seed)
    ([1500], 8, 2, 128, "bf16", 512, 128, 1e6, 11),          # G = 3, GQA 4
    ([777, 64, 1, 1300], 8, 2, 128, "bf16", 256, 200, 1e4, 12),  # ragged varlen, G = 4/1/1/6
    ([1000], 8, 2, 128, "bf16", 256, 0, 1e4, 13),           # w0 = 0: all remote
    ([900], 4, 4, 128, "bf16", 128, 5000, 1e4, 14),         # w0 >= L: all local, MHA
    ([1100], 6, 3, 128, "bf16", 2048, 100, 1e4, 15),         # G = 1, GQA 2
    ([1000], 4, 2, 64, "bf16", 300, 64, 1e4, 16),            # head_dim 64
    ([640], 16, 2, 128, "bf16", 100, 37, 1e6, 17),           # GQA 8: two head groups
    ([513, 70], 2, 1, 64, "f32", 128, 33, 1e4, 18),          # fp32, GQA 2, d 64
    ([300], 4, 2, 128, "f32", 64, 50, 1e4, 19),              # fp32, d 128
    ([65], 4, 1, 128, "bf16", 32, 1, 10.0, 20),               # window 1, tiny theta
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[f"case{i}" for i in range(len(PREFILL_CASES))])
def test_prefill_matches_oracle(case):
    _torch()
    lens, Hq, Hkv, d, dt, wp, w0, theta, seed = case
    _say("prefill", case)
    inp = W.prefill_inputs(lens, Hq, Hkv, d, dt, seed)
    check_prefill(inp, wp, w0, theta)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_chunked_prefill_matches_oracle(dt):
    """Queries at the last positions of longer sequences (a prefill chunk
    against an existing cache); G comes from the full length."""
    _torch()
    _say("chunked prefill", dt)
    inp = W.prefill_inputs([1200, 700, 90], 8, 2, 128, dt, 21, q_lens=[130, 700, 1])
    check_prefill(inp, 256, 100, 1e4)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_contract_breaks_left_unwritten(dt):
    """Sequences whose lengths exceed the bounds passed (Lq > max_seqlen_q,
    L > max_seqlen_k) are skipped: their rows of o and lse keep what the
    caller stored; the valid sequence matches the oracle."""
    torch = _torch()
    wp, w0, theta = 128, 60, 1e4
    inp = W.prefill_inputs([300, 250, 400], 8, 2, 128, dt, 46, q_lens=[100, 200, 50])
    _say("prefill contract breaks", dt)
    q = W.to_device(inp["q"], dt)
    k = W.to_device(inp["k"], dt)
    v = W.to_device(inp["v"], dt)
    cu_q = torch.from_numpy(inp["cu_q"]).cuda()
    cu_k = torch.from_numpy(inp["cu_k"]).cuda()
    out = torch.full_like(q, 7.0)
    lse = torch.full((8, q.shape[0]), 5.0, dtype=torch.float32, device=q.device)
    # sequence 1: Lq = 200 > max_seqlen_q = 150; sequence 2: L = 400 > max_seqlen_k = 300
    jl.prefill(q, k, v, cu_q, 150, wp, w0, theta, cu_seqlens_k=cu_k, max_seqlen_k=300, out=out, lse=lse,
               return_lse=True)
    torch.cuda.synchronize()
    o_gpu = out.float().cpu().numpy().astype(np.float64)
    l_gpu = lse.cpu().numpy().astype(np.float64)
    assert np.all(o_gpu[100:] == 7.0) and np.all(l_gpu[:, 100:] == 5.0)
    qq = W.as_f64(inp["q"][:100], dt)
    o_ref, l_ref = oracle.bifocal_sequence(qq, W.as_f64(inp["k"][:300], dt), W.as_f64(inp["v"][:300], dt),
                                           np.arange(200, 300), 300, wp, w0, theta)
    err_o = np.max(np.abs(o_gpu[:100] - o_ref))
    err_l = np.max(np.abs(l_gpu[:, :100].T - l_ref))
    _say(f"seq 0: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= TOL[dt] and err_l <= TOL[dt], (err_o, err_l)


def test_prefill_peaked_keys():
    _torch()
    _say("peaked keys")
    inp = W.prefill_inputs([1536], 8, 2, 128, "bf16", 22, peaked_rows=16, peak_seed=5, peak_scale=4.0)
    check_prefill(inp, 512, 128, 1e6)


@pytest.mark.parametrize("rise", [6.0, 16.0])  # log2 climb ~ rise * 8 / sqrt(128) / ln 2
def test_prefill_rising_scores(rise):
    """Scores that climb along the keys of every row: one feature of the
    lowest-frequency rotation pair (features d/2 - 1 and d - 1, nearly
    position-independent over 2048 keys) carries a query weight of 8 and a
    key weight growing linearly to `rise` (a total climb of about 6 or 16
    log2 units), so each row's maximum rises tile after tile by a fraction
    of a log2 unit.  The fast path then keeps a
    stale maximum over many tiles with probabilities far above 1 before the
    slow path rescales; the result must still match the oracle."""
    _torch()
    _say("rising scores", rise)
    inp = W.prefill_inputs([2048], 4, 1, 128, "bf16", 23)
    q = W.bits_to_f32(inp["q"]) * np.float32(0.25)
    k = W.bits_to_f32(inp["k"]) * np.float32(0.25)
    q[:, :, 127] = 8.0
    k[:, 0, 127] = np.linspace(0.0, rise, 2048, dtype=np.float32)
    inp["q"], inp["k"] = W.bf16_bits(q), W.bf16_bits(k)
    check_prefill(inp, 512, 256, 1e4)


def test_prefill_inputs_untouched_and_deterministic():
    torch = _torch()
    _say("prefill determinism")
    inp = W.prefill_inputs([700, 300], 8, 2, 128, "bf16", 23)
    q = W.to_device(inp["q"], "bf16")
    k = W.to_device(inp["k"], "bf16")
    v = W.to_device(inp["v"], "bf16")
    cu = torch.from_numpy(inp["cu_q"]).cuda()
    h0 = [hashlib.sha256(t.view(torch.int16).cpu().numpy().tobytes()).hexdigest() for t in (q, k, v)]
    o1 = jl.prefill(q, k, v, cu, 700, 256, 64, 1e4)
    o2 = jl.prefill(q, k, v, cu, 700, 256, 64, 1e4)
    torch.cuda.synchronize()
    h1 = [hashlib.sha256(t.view(torch.int16).cpu().numpy().tobytes()).hexdigest() for t in (q, k, v)]
    assert h0 == h1
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ---------------------------------------------------------------- decode

def run_decode(inp, wp, w0, theta, max_L=None):
    torch = _torch()
    dt = inp["dtype"]
    q = W.to_device(inp["q"], dt)
    k = W.to_device(inp["k"], dt)
    v = W.to_device(inp["v"], dt)
    seq = torch.from_numpy(inp["seq_L"]).cuda()
    out, lse = jl.decode(q, k, v, seq, wp, w0, theta, max_L=max_L, return_lse=True)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_decode(inp, wp, w0, theta):
    dt = inp["dtype"]
    o_gpu, lse_gpu = run_decode(inp, wp, w0, theta)
    o_ref, lse_ref = oracle.bifocal_decode(W.as_f64(inp["q"], dt), W.as_f64(inp["k"], dt),
                                           W.as_f64(inp["v"], dt), inp["seq_L"], wp, w0, theta)
    err_o = np.max(np.abs(o_gpu - o_ref))
    err_l = np.max(np.abs(lse_gpu - lse_ref))
    _say(f"max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert np.all(np.isfinite(o_gpu))
    assert err_o <= TOL[dt], err_o
    assert err_l <= TOL[dt], err_l


DECODE_CASES = [
    # (B, S, seq_L, Hq, Hkv, d, dtype, wp, w0, theta, seed)
    (4, 3000, [3000, 1, 2049, 777], 32, 8, 128, "bf16", 512, 256, 1e6, 31),
    (3, 1500, [1500, 1024, 15], 8, 8, 128, "bf16", 256, 0, 1e4, 32),       # all remote, MHA
    (2, 900, [900, 450], 16, 2, 64, "bf16", 128, 2000, 1e4, 33),          # all local, GQA 8, d 64
    (2, 1000, [1000, 999], 12, 4, 128, "bf16", 300, 77, 1e4, 34),          # GQA 3
    (3, 800, [800, 65, 5], 8, 2, 128, "f32", 100, 50, 1e4, 35),
    (2, 700, [700, 300], 4, 4, 64, "f32", 64, 0, 1e4, 36),
    (1, 5000, [5000], 64, 4, 128, "bf16", 1024, 512, 1e6, 37),            # GQA 16
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[f"case{i}" for i in range(len(DECODE_CASES))])
def test_decode_matches_oracle(case):
    _torch()
    B, S, seq_L, Hq, Hkv, d, dt, wp, w0, theta, seed = case
    _say("decode", case)
    inp = W.decode_inputs(B, S, Hq, Hkv, d, dt, seed, seq_L=seq_L)
    check_decode(inp, wp, w0, theta)


# Decode cases aimed at which cos/sin rows the decode writes: neighbours of
# equal length (their window is written once), overlapping windows that start
# off the 32-row run grid, a sequence shorter than w_pretrained, and empty
# windows (w0 = 0, where the query's own row is written on its own); d 128
# (one run per wavefront) and d 64 (two runs per wavefront), both dtypes.
TABLE_ROW_CASES = [
    # (B, S, seq_L, Hq, Hkv, d, dtype, wp, w0, theta, seed)
    (6, 2400, [2400, 2400, 2333, 2301, 2400, 90], 16, 4, 128, "bf16", 600, 250, 1e4, 41),
    (6, 2400, [2400, 2400, 2333, 2301, 2400, 90], 16, 4, 128, "f32", 600, 250, 1e4, 42),
    (4, 1300, [1300, 1300, 1299, 7], 8, 2, 64, "bf16", 256, 0, 1e4, 43),
    (4, 1300, [1300, 1300, 1299, 7], 8, 2, 64, "f32", 256, 0, 1e4, 44),
]


@pytest.mark.parametrize("case", TABLE_ROW_CASES, ids=[f"rows{i}" for i in range(len(TABLE_ROW_CASES))])
def test_decode_table_rows(case):
    _torch()
    B, S, seq_L, Hq, Hkv, d, dt, wp, w0, theta, seed = case
    _say("decode table rows", case)
    inp = W.decode_inputs(B, S, Hq, Hkv, d, dt, seed, seq_L=seq_L)
    check_decode(inp, wp, w0, theta)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_invalid_lengths_left_unwritten(dt):
    """A sequence whose length breaks 1 <= L <= max_L is skipped by every
    decode kernel (its o and lse keep what the caller stored there); the
    other sequences of the batch match the oracle."""
    torch = _torch()
    B, S, Hq, Hkv, d, wp, w0, theta = 4, 600, 8, 2, 128, 256, 100, 1e4
    good = [600, 600, 300, 17]
    inp = W.decode_inputs(B, S, Hq, Hkv, d, dt, 45, seq_L=good)
    q = W.to_device(inp["q"], dt)
    k = W.to_device(inp["k"], dt)
    v = W.to_device(inp["v"], dt)
    lens = np.array([600, 0, 300, 601], dtype=np.int32)  # sequence 1: L = 0; sequence 3: L > max_L
    _say("decode invalid lengths", dt, lens.tolist())
    out = torch.full_like(q, 7.0)
    lse = torch.full((B, Hq), 5.0, dtype=torch.float32, device=q.device)
    jl.decode(q, k, v, torch.from_numpy(lens).cuda(), wp, w0, theta, max_L=S, out=out, lse=lse, return_lse=True)
    torch.cuda.synchronize()
    o_gpu = out.float().cpu().numpy().astype(np.float64)
    l_gpu = lse.cpu().numpy().astype(np.float64)
    for b in (1, 3):
        assert np.all(o_gpu[b] == 7.0) and np.all(l_gpu[b] == 5.0), b
    o_ref, l_ref = oracle.bifocal_decode(W.as_f64(inp["q"], dt), W.as_f64(inp["k"], dt), W.as_f64(inp["v"], dt),
                                         inp["seq_L"], wp, w0, theta)
    for b in (0, 2):
        err_o = np.max(np.abs(o_gpu[b] - o_ref[b]))
        err_l = np.max(np.abs(l_gpu[b] - l_ref[b]))
        _say(f"seq {b}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
        assert err_o <= TOL[dt] and err_l <= TOL[dt], (b, err_o, err_l)


def test_decode_strided_cache_and_untouched():
    """A cache laid out [S, B, Hkv, d] (non-default strides) is read in place
    and both caches are left byte-identical."""
    torch = _torch()
    _say("decode strided")
    B, S, Hq, Hkv, d = 3, 1200, 8, 2, 128
    inp = W.decode_inputs(B, S, Hq, Hkv, d, "bf16", 38, seq_L=[1200, 600, 33])
    k = W.to_device(inp["k"], "bf16").permute(1, 0, 2, 3).contiguous().permute(1, 0, 2, 3)
    v = W.to_device(inp["v"], "bf16").permute(1, 0, 2, 3).contiguous().permute(1, 0, 2, 3)
    q = W.to_device(inp["q"], "bf16")
    seq = torch.from_numpy(inp["seq_L"]).cuda()
    digest = lambda t: hashlib.sha256(t.contiguous().view(torch.int16).cpu().numpy().tobytes()).hexdigest()  # noqa: E731
    hk, hv = digest(k), digest(v)
    out = jl.decode(q, k, v, seq, 256, 100, 1e4)
    torch.cuda.synchronize()
    assert digest(k) == hk and digest(v) == hv
    o_ref, _ = oracle.bifocal_decode(W.as_f64(inp["q"], "bf16"), W.as_f64(inp["k"], "bf16"),
                                     W.as_f64(inp["v"], "bf16"), inp["seq_L"], 256, 100, 1e4)
    err = np.max(np.abs(out.float().cpu().numpy() - o_ref))
    _say(f"max|dO|={err:.3e}")
    assert err <= TOL["bf16"]


def test_decode_equals_last_prefill_row():
    """Decode of the newest token equals the last row of the prefill of the
    same sequence (both on the GPU)."""
    torch = _torch()
    _say("decode vs prefill")
    L, Hq, Hkv, d = 1300, 8, 2, 128
    inp = W.prefill_inputs([L], Hq, Hkv, d, "f32", 39)
    o_p, _ = run_prefill(inp, 256, 100, 1e4)
    q = torch.from_numpy(inp["q"][L - 1:L]).cuda()
    k = torch.from_numpy(inp["k"]).cuda().unsqueeze(0)
    v = torch.from_numpy(inp["v"]).cuda().unsqueeze(0)
    seq = torch.tensor([L], dtype=torch.int32).cuda()
    o_d = jl.decode(q, k, v, seq, 256, 100, 1e4).cpu().numpy()
    assert np.max(np.abs(o_d[0] - o_p[L - 1])) < 1e-5


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_steps_across_G_boundaries(dt):
    """Decode steps on one unchanged cache as the length crosses multiples of
    w_pretrained: G goes 1, 1, 2, 2, 3, 3, 4 without any key being rewritten."""
    torch = _torch()
    wp, w0, theta, S = 256, 64, 1e4, 1024
    seq_L = [wp - 1, wp, wp + 1, 2 * wp, 2 * wp + 1, 3 * wp, 3 * wp + 1]
    _say("decode across G boundaries", dt, seq_L)
    one = W.decode_inputs(1, S, 8, 2, 128, dt, 38)
    B = len(seq_L)
    inp = dict(q=np.repeat(one["q"], B, axis=0), k=np.repeat(one["k"], B, axis=0),
               v=np.repeat(one["v"], B, axis=0), seq_L=np.asarray(seq_L, dtype=np.int32), dtype=dt)
    check_decode(inp, wp, w0, theta)
    # One cache buffer shared by every step (batch stride 0 view).
    k = W.to_device(one["k"], dt).expand(B, -1, -1, -1)
    v = W.to_device(one["v"], dt).expand(B, -1, -1, -1)
    q = W.to_device(one["q"], dt).expand(B, -1, -1).contiguous()
    seq = torch.from_numpy(inp["seq_L"]).cuda()
    out = jl.decode(q, k, v, seq, wp, w0, theta)
    o_sep, _ = run_decode(inp, wp, w0, theta)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy().astype(np.float64), o_sep)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prepare_once_attend_several_windows(dt):
    """One prepared workspace (rotated key copies, V^T, table) serves attends
    with different local windows, each matching the oracle."""
    torch = _torch()
    L, wp, theta = 1300, 256, 1e4
    _say("prepare once, attend twice", dt)
    inp = W.prefill_inputs([L], 8, 2, 128, dt, 24)
    q = W.to_device(inp["q"], dt)
    k = W.to_device(inp["k"], dt)
    v = W.to_device(inp["v"], dt)
    cu = torch.from_numpy(inp["cu_q"]).cuda()
    ws = jl.prefill_prepare(k, v, cu, L, wp, theta, Hq=8)
    for w0 in (64, 500):
        out, lse = jl.prefill_attend(q, k, v, cu, L, wp, w0, theta, ws, return_lse=True)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle_prefill(inp, wp, w0, theta)
        eo = float(np.max(np.abs(out.float().cpu().numpy() - o_ref)))
        el = float(np.max(np.abs(lse.cpu().numpy().T - l_ref)))
        _say(f"w0={w0}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= TOL[dt] and el <= TOL[dt], (w0, eo, el)


def test_chunked_prefill_across_G_boundary_same_cache():
    """Two prefill chunks over one unchanged key/value buffer: the first ends
    at L = w_pretrained (G = 1), the second at L = w_pretrained + 150 (G = 2);
    each attends to the cache as it stands, with G taken from its own length."""
    torch = _torch()
    wp, w0, theta, Hq, Hkv, d = 256, 40, 1e4, 8, 2, 128
    Lmax = wp + 150
    _say("chunks across G boundary")
    full = W.prefill_inputs([Lmax], Hq, Hkv, d, "bf16", 25)
    k = W.to_device(full["k"], "bf16")
    v = W.to_device(full["v"], "bf16")
    for L, Lq in ((wp, 100), (Lmax, Lmax - wp)):
        q_np = full["q"][L - Lq:L]
        q = W.to_device(q_np, "bf16")
        cu_q = torch.tensor([0, Lq], dtype=torch.int32, device="cuda")
        cu_k = torch.tensor([0, L], dtype=torch.int32, device="cuda")
        out, lse = jl.prefill(q, k[:L], v[:L], cu_q, Lq, wp, w0, theta, cu_seqlens_k=cu_k, max_seqlen_k=L,
                              return_lse=True)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.bifocal_sequence(W.as_f64(q_np, "bf16"), W.as_f64(full["k"][:L], "bf16"),
                                               W.as_f64(full["v"][:L], "bf16"), np.arange(L - Lq, L), L, wp, w0,
                                               theta)
        eo = float(np.max(np.abs(out.float().cpu().numpy() - o_ref)))
        el = float(np.max(np.abs(lse.cpu().numpy().T - l_ref)))
        _say(f"L={L} (G={jl.group_size(L, wp)}): max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= TOL["bf16"] and el <= TOL["bf16"], (L, eo, el)


# ---------------------------------------------------------------- sweeps

def _random_prefill_configs(n, seed):
    """Seeded small configurations: ragged lengths (some not multiples of 64,
    some shorter than one tile), GQA ratios 1..8 including odd ones, head_dim
    64 / 128, windows from 0 to beyond L and group sizes from 1 to ~8."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(1, 1400, size=B)]
        Hkv = int(rng.choice([1, 2, 3]))
        ratio = int(rng.choice([1, 2, 3, 4, 5, 8]))
        d = int(rng.choice([64, 128]))
        dt = "bf16" if i % 4 else "f32"
        Lmax = max(lens)
        wp = int(rng.integers(max(1, Lmax // 8), Lmax + 200))
        w0 = int(rng.choice([0, 1, int(rng.integers(2, 400)), Lmax + 5]))
        theta = float(rng.choice([1e4, 1e6]))
        out.append((lens, Hkv * ratio, Hkv, d, dt, wp, w0, theta, 100 + i))
    return out


@pytest.mark.parametrize("case", _random_prefill_configs(12, 2024), ids=[f"r{i}" for i in range(12)])
def test_prefill_random_configs(case):
    _torch()
    lens, Hq, Hkv, d, dt, wp, w0, theta, seed = case
    _say("random prefill", case)
    inp = W.prefill_inputs(lens, Hq, Hkv, d, dt, seed)
    check_prefill(inp, wp, w0, theta)


def _random_decode_configs(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B = int(rng.integers(1, 5))
        S = int(rng.integers(16, 3000))
        seq_L = [int(x) for x in rng.integers(1, S + 1, size=B)]
        Hkv = int(rng.choice([1, 2, 4, 8]))
        ratio = int(rng.choice([1, 2, 3, 4, 6, 8]))
        d = int(rng.choice([64, 128]))
        dt = "bf16" if i % 4 else "f32"
        wp = int(rng.integers(max(1, S // 8), S + 200))
        w0 = int(rng.choice([0, 1, int(rng.integers(2, 600)), S + 5]))
        theta = float(rng.choice([1e4, 1e6]))
        out.append((B, S, seq_L, Hkv * ratio, Hkv, d, dt, wp, w0, theta, 200 + i))
    return out


@pytest.mark.parametrize("case", _random_decode_configs(12, 2025), ids=[f"r{i}" for i in range(12)])
def test_decode_random_configs(case):
    _torch()
    B, S, seq_L, Hq, Hkv, d, dt, wp, w0, theta, seed = case
    _say("random decode", case)
    inp = W.decode_inputs(B, S, Hq, Hkv, d, dt, seed, seq_L=seq_L)
    check_decode(inp, wp, w0, theta)
