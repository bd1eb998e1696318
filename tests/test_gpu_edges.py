"""GPU cases aimed at what random inputs at small group sizes cannot show.

* The bf16 decode's integer map (its own fp32 quotient for f(j) = floor(j/G),
  eq. f) exported by jl_bifocal_decode_key_rows, bit-exact against j // G for
  G from 1 to beyond 2^20.
* Group sizes in the hundreds to thousands (small w_pretrained), both dtypes.
* Planted keys at distance w0 - 1 and w0 of chosen queries (tests/planted.py),
  where one pair routed to the wrong side of the window edge moves the output
  by ~2 (checked on the CPU by tests/test_planted_sensitivity.py).
* The two configurations the benchmark times as plain RoPE: prefill with
  G = 1 and w0 = 0, and a pre-rotated decode with every key in the window.
* The bf16 operand range: keys near the half limit match the oracle; keys,
  values or queries beyond it give NaN in the rows that use them and leave the
  other rows exact.
* The prepared-table decode gives the same bits as the decode that builds
  its own rows.

Tolerances as everywhere: max abs error 1e-4 (fp32) and 2e-2 (bf16) on O and
LSE; integer maps bit-exact.
"""
import numpy as np
import pytest

import oracle
import zero_shot_rope_bifocal_amd as jl
from zero_shot_rope_bifocal_amd import workloads as W

import planted
from test_gpu_parity import TOL, _say, _torch, check_decode, check_prefill, oracle_prefill, run_prefill

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- integers

def _want_rows(seq_L, max_L, wp, w0, prerot):
    want = np.full((len(seq_L), max_L), -2 ** 31, dtype=np.int64)
    for b, L in enumerate(seq_L):
        if not 1 <= L <= max_L:
            continue
        G = oracle.group_size(L, wp)
        j = np.arange(L, dtype=np.int64)
        f = oracle.remote_positions(j, G)
        local = (L - 1) - j < w0
        if prerot:
            want[b, :L] = np.where(local, 0, ~(j - f))
        else:
            want[b, :L] = np.where(local, j, f)
    return want


@pytest.mark.parametrize("prerot", [False, True])
@pytest.mark.parametrize("Hkv", [8, 3])
def test_decode_key_rows_bit_exact(prerot, Hkv):
    """G from 1 to 2^21 (w_pretrained 1 makes G = L), lengths not multiples of
    16 or of the split size, windows 0, 1, 100 and beyond L."""
    torch = _torch()
    rng = np.random.default_rng(77)
    max_L = 1 << 21
    seq_L = [max_L, (1 << 20) + 3, (1 << 20) - 1, 300001, 65537, 4099, 1000, 17, 1, 0]
    wps = [1, 1, 1, 7, 3, 2, 1000, 5, 1, 4]
    for w0 in (0, 1, 100, max_L + 1):
        for b in range(len(seq_L)):
            L, wp = seq_L[b], wps[b]
            sl = torch.tensor([L], dtype=torch.int32, device="cuda")
            Lm = max(L, 1)
            got = jl.decode_key_rows(sl, Lm, Hkv, wp, w0, prerotated=prerot).cpu().numpy().astype(np.int64)
            want = _want_rows([L], Lm, wp, w0, prerot)
            _say("key rows", dict(L=L, wp=wp, w0=w0, Hkv=Hkv, prerot=prerot))
            assert np.array_equal(got, want), (L, wp, w0, np.argwhere(got != want)[:5])
    # a batch with random group sizes in one call
    seq_L = [int(x) for x in rng.integers(1, 200000, size=12)]
    wps = [int(x) for x in rng.integers(1, 3000, size=12)]
    for wp in wps[:4]:
        sl = torch.tensor(seq_L, dtype=torch.int32, device="cuda")
        got = jl.decode_key_rows(sl, max(seq_L), Hkv, wp, 77, prerotated=prerot).cpu().numpy().astype(np.int64)
        assert np.array_equal(got, _want_rows(seq_L, max(seq_L), wp, 77, prerot)), wp


# ---------------------------------------------------------------- large G

LARGE_G_PREFILL = [
    # (lens, Hq, Hkv, d, dtype, wp, w0, theta, seed)
    ([3000], 8, 2, 128, "bf16", 3, 100, 1e4, 71),          # G = 1000
    ([3000, 1111], 8, 2, 128, "f32", 10, 64, 1e4, 72),     # G = 300 / 112
    ([2500], 4, 1, 64, "bf16", 1, 200, 1e6, 73),           # G = 2500 (every remote key at f = 0)
    ([4096], 8, 4, 128, "bf16", 7, 1, 1e4, 74),            # G = 586, window 1
]


@pytest.mark.parametrize("case", LARGE_G_PREFILL, ids=[f"g{i}" for i in range(len(LARGE_G_PREFILL))])
def test_prefill_large_group_size(case):
    _torch()
    lens, Hq, Hkv, d, dt, wp, w0, theta, seed = case
    _say("prefill large G", case, [oracle.group_size(L, wp) for L in lens])
    check_prefill(W.prefill_inputs(lens, Hq, Hkv, d, dt, seed), wp, w0, theta)


LARGE_G_DECODE = [
    # (B, S, seq_L, Hq, Hkv, d, dtype, wp, w0, theta, seed)
    (3, 5000, [5000, 4097, 1500], 32, 8, 128, "bf16", 2, 300, 1e6, 75),   # G = 2500 / 2049 / 750
    (2, 4096, [4096, 3333], 8, 2, 128, "f32", 1, 100, 1e4, 76),          # G = L
    (2, 3000, [3000, 2999], 16, 4, 64, "bf16", 9, 0, 1e4, 77),           # G = 334, all remote
]


@pytest.mark.parametrize("case", LARGE_G_DECODE, ids=[f"g{i}" for i in range(len(LARGE_G_DECODE))])
def test_decode_large_group_size(case):
    _torch()
    B, S, seq_L, Hq, Hkv, d, dt, wp, w0, theta, seed = case
    _say("decode large G", case)
    check_decode(W.decode_inputs(B, S, Hq, Hkv, d, dt, seed, seq_L=seq_L), wp, w0, theta)


# One sequence, so the key ranges are as many as the split rules allow: with
# one KV head the bf16 kernel runs 8 waves per head and the combine merges
# its maximum of 1024 partial states; with 8 KV heads, 512 ranges of one wave
# each (the 128K decode at batch 1); the fp32 kernel at its own slot count.
MOST_PARTS = [
    # (B, S, seq_L, Hq, Hkv, d, dtype, wp, w0, theta, seed)
    (1, 40000, [40000], 4, 1, 128, "bf16", 8192, 2048, 1e6, 91),
    (1, 40000, [40000], 4, 1, 128, "f32", 8192, 2048, 1e6, 92),
    (1, 131072, [131072], 32, 8, 128, "bf16", 32768, 2048, 1e6, 93),
]


@pytest.mark.parametrize("case", MOST_PARTS, ids=[f"p{i}" for i in range(len(MOST_PARTS))])
def test_decode_most_partial_states(case):
    _torch()
    B, S, seq_L, Hq, Hkv, d, dt, wp, w0, theta, seed = case
    _say("decode, most key ranges", case[:3], case[3:])
    check_decode(W.decode_inputs(B, S, Hq, Hkv, d, dt, seed, seq_L=seq_L), wp, w0, theta)


# ---------------------------------------------------------------- window edge

EDGE_PREFILL = [
    # (L, Hq, Hkv, d, dtype, wp, w0, theta)
    (1100, 8, 2, 128, "bf16", 256, 100, 1e4),
    (1100, 8, 2, 128, "bf16", 256, 64, 1e4),   # window edge on a tile boundary
    (1300, 4, 4, 64, "bf16", 300, 129, 1e4),
    (900, 8, 2, 128, "bf16", 128, 1, 1e4),     # window 1: only the diagonal is local
    (1100, 4, 2, 128, "f32", 256, 100, 1e4),
]


@pytest.mark.parametrize("case", EDGE_PREFILL, ids=[f"e{i}" for i in range(len(EDGE_PREFILL))])
def test_prefill_planted_window_edge(case):
    _torch()
    L, Hq, Hkv, d, dt, wp, w0, theta = case
    inp, rows = planted.edge_prefill(L, Hq, Hkv, d, dt, wp, w0, theta, seed=81)
    _say("prefill window edge", case, f"{len(rows)} planted rows")
    assert len(rows) >= 5
    o_gpu, lse_gpu = run_prefill(inp, wp, w0, theta)
    o_ref, lse_ref = oracle_prefill(inp, wp, w0, theta)
    err_rows = np.max(np.abs(o_gpu[rows] - o_ref[rows]))
    err_o = np.max(np.abs(o_gpu - o_ref))
    err_l = np.max(np.abs(lse_gpu.T - lse_ref))
    _say(f"planted rows max|dO|={err_rows:.3e}; all rows max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}")
    assert err_o <= TOL[dt] and err_l <= TOL[dt], (err_o, err_l)


EDGE_DECODE = [
    # (seq_L, S, Hq, Hkv, d, dtype, wp, w0, theta)
    ([1500, 900, 1234, 777], 1500, 32, 8, 128, "bf16", 128, 100, 1e4),
    ([2048, 2047, 1000, 1025], 2048, 8, 2, 128, "bf16", 256, 64, 1e4),
    ([3000, 2000], 3000, 16, 2, 64, "bf16", 100, 1, 1e6),
    ([1500, 900, 1234, 777], 1500, 8, 2, 128, "f32", 128, 100, 1e4),
]


@pytest.mark.parametrize("case", EDGE_DECODE, ids=[f"e{i}" for i in range(len(EDGE_DECODE))])
def test_decode_planted_window_edge(case):
    _torch()
    seq_L, S, Hq, Hkv, d, dt, wp, w0, theta = case
    inp, planted_b = planted.edge_decode(seq_L, S, Hq, Hkv, d, dt, wp, w0, theta, seed=82)
    _say("decode window edge", case, "planted sequences", planted_b)
    assert len(planted_b) == len(seq_L)
    check_decode(inp, wp, w0, theta)


# ---------------------------------------------------------------- plain RoPE configurations

@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_plain_rope_configuration(dt):
    """w_pretrained = L (G = 1) and w0 = 0: every pair at its true position
    through the all-remote route; equals textbook RoPE causal attention."""
    _torch()
    lens = [1500, 700]
    _say("prefill plain-RoPE config", dt)
    inp = W.prefill_inputs(lens, 8, 2, 128, dt, 83)
    check_prefill(inp, max(lens), 0, 1e6)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_decode_plain_rope_configuration(dt):
    """Pre-rotated cache with w0 >= max_L: the plain path (bf16: no table, no
    key rotation, stored keys on the bf16 MFMA) against the oracle's
    pre-rotated attention, which then is textbook attention on the stored
    vectors."""
    torch = _torch()
    B, S, Hq, Hkv, d, wp, theta = 3, 2000, 32, 8, 128, 300, 1e6
    seq_L = [2000, 1999, 37]
    inp = W.decode_inputs(B, S, Hq, Hkv, d, dt, 84, seq_L=seq_L)
    _say("decode plain-RoPE config", dt)
    for w0 in (S, S + 1000):
        q = W.to_device(inp["q"], dt)
        k = W.to_device(inp["k"], dt)
        v = W.to_device(inp["v"], dt)
        seq = torch.from_numpy(inp["seq_L"]).cuda()
        out, lse = jl.decode(q, k, v, seq, wp, w0, theta, return_lse=True, prerotated=True)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.bifocal_decode_prerotated(W.as_f64(inp["q"], dt), W.as_f64(inp["k"], dt),
                                                        W.as_f64(inp["v"], dt), inp["seq_L"], wp, w0, theta)
        eo = float(np.max(np.abs(out.float().cpu().numpy() - o_ref)))
        el = float(np.max(np.abs(lse.cpu().numpy() - l_ref)))
        _say(f"w0={w0}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= TOL[dt] and el <= TOL[dt], (w0, eo, el)


# ---------------------------------------------------------------- bf16 range

def _prefill_bits(q, k, v, L, Hq, Hkv, d, wp, w0, theta):
    return dict(q=W.bf16_bits(q), k=W.bf16_bits(k), v=W.bf16_bits(v),
                cu_q=np.array([0, L], np.int32), cu_k=np.array([0, L], np.int32),
                lens=[L], q_lens=[L], dtype="bf16", Hq=Hq, Hkv=Hkv, d=d)


def _near_limit_keys(k, q, rows, d):
    """Keys of `rows` get +-40000 (the supported bound is 46300) on rotation
    pair 3, where every query is zero: rotated, they stay below the half
    limit, so they add exactly nothing to the scores (an overflow would turn
    0 * inf into NaN).  They also get +-4000 on pair 5, where the queries
    are scaled by 1e-3, so those large components do score (logit terms of
    order 0.5) and are checked for accuracy."""
    h = d // 2
    for f in (3, 3 + h):
        k[rows, :, f] = np.where(k[rows, :, f] < 0, -40000.0, 40000.0)
        q[..., f] = 0.0
    for f in (5, 5 + h):
        k[rows, :, f] = np.where(k[rows, :, f] < 0, -4000.0, 4000.0)
        q[..., f] *= 1e-3


def test_prefill_keys_near_half_limit():
    _torch()
    L, Hq, Hkv, d, wp, w0, theta = 1000, 8, 2, 128, 256, 100, 1e4
    base = W.prefill_inputs([L], Hq, Hkv, d, "f32", 85)
    k, q = base["k"].copy(), base["q"].copy()
    _near_limit_keys(k, q, np.random.default_rng(85).choice(L, 40, replace=False), d)
    inp = _prefill_bits(q, k, base["v"], L, Hq, Hkv, d, wp, w0, theta)
    _say("prefill keys near the half limit")
    check_prefill(inp, wp, w0, theta)


def test_decode_keys_near_half_limit():
    _torch()
    B, S, Hq, Hkv, d, wp, w0, theta = 2, 1200, 8, 2, 128, 256, 100, 1e4
    base = W.decode_inputs(B, S, Hq, Hkv, d, "f32", 86, seq_L=[1200, 999])
    k, q = base["k"].copy(), base["q"].copy()
    for b in range(B):
        _near_limit_keys(k[b], q[b:b + 1], np.arange(0, S, 7), d)
    inp = dict(base, q=W.bf16_bits(q), k=W.bf16_bits(k), v=W.bf16_bits(base["v"]), dtype="bf16")
    _say("decode keys near the half limit")
    check_decode(inp, wp, w0, theta)


@pytest.mark.parametrize("which", ["k", "v", "q"])
def test_prefill_out_of_range_gives_nan(which):
    """One element of 1e6 (beyond half range) in key or value row j (KV head
    0) or in query row j (head 0): every output row >= j of the heads that
    attend it is NaN; rows of the other KV head and rows well before j match
    the oracle."""
    torch = _torch()
    L, Hq, Hkv, d, wp, w0, theta, j = 1000, 8, 2, 128, 256, 100, 1e4, 700
    base = W.prefill_inputs([L], Hq, Hkv, d, "f32", 87)
    arrs = dict(q=base["q"].copy(), k=base["k"].copy(), v=base["v"].copy())
    arrs[which][j, 0, 5] = 1e6
    inp = _prefill_bits(arrs["q"], arrs["k"], arrs["v"], L, Hq, Hkv, d, wp, w0, theta)
    _say("prefill out of range", which)
    o_gpu, lse_gpu = run_prefill(inp, wp, w0, theta)
    o_ref, lse_ref = oracle_prefill(inp, wp, w0, theta)
    if which == "q":
        # only query row j of head 0 uses the value
        assert np.all(np.isnan(o_gpu[j, 0])) and np.isnan(lse_gpu[0, j])
        mask = np.ones(o_gpu.shape[:2], bool)
        mask[j, 0] = False
        eo = np.max(np.abs(o_gpu[mask] - o_ref[mask]))
        _say(f"untouched rows max|dO|={eo:.3e}")
        assert np.isfinite(eo) and eo <= TOL["bf16"], eo
        return
    heads = list(range(Hq // Hkv))  # query heads reading KV head 0
    others = [h for h in range(Hq) if h not in heads]
    assert np.all(np.isnan(o_gpu[j:, heads].reshape(L - j, -1).max(axis=1))), "rows >= j not NaN"
    if which == "k":
        assert np.all(np.isnan(lse_gpu[heads][:, j:]))
    before = slice(0, j - 256)
    eo = max(np.max(np.abs(o_gpu[:, others] - o_ref[:, others])), np.max(np.abs(o_gpu[before] - o_ref[before])))
    _say(f"untouched rows max|dO|={eo:.3e}")
    assert np.isfinite(eo) and eo <= TOL["bf16"], eo


@pytest.mark.parametrize("which", ["k", "q"])
def test_decode_out_of_range_gives_nan(which):
    """A key element (or query element) of 1e6 in sequence 0, KV head 1: the
    query heads of that KV group (or that head) come out NaN; every other
    head and sequence matches the oracle."""
    torch = _torch()
    B, S, Hq, Hkv, d, wp, w0, theta = 2, 1500, 8, 2, 128, 256, 100, 1e4
    base = W.decode_inputs(B, S, Hq, Hkv, d, "f32", 88, seq_L=[1500, 1300])
    q, k = base["q"].copy(), base["k"].copy()
    for pos in (10, 1450):  # one remote and one local key (or just the query)
        if which == "k":
            k[0, pos, 1, 3] = -1e6
    if which == "q":
        q[0, 5, 3] = 1e6
    inp = dict(base, q=W.bf16_bits(q), k=W.bf16_bits(k), v=W.bf16_bits(base["v"]), dtype="bf16")
    _say("decode out of range", which)
    qd, kd, vd = (W.to_device(inp[n], "bf16") for n in ("q", "k", "v"))
    out, lse = jl.decode(qd, kd, vd, torch.from_numpy(inp["seq_L"]).cuda(), wp, w0, theta, return_lse=True)
    torch.cuda.synchronize()
    o_gpu = out.float().cpu().numpy()
    bad = [4, 5, 6, 7] if which == "k" else [5]
    assert np.all(np.isnan(o_gpu[0, bad])) and np.all(np.isnan(lse.cpu().numpy()[0, bad]))
    o_ref, _ = oracle.bifocal_decode(W.as_f64(inp["q"], "bf16"), W.as_f64(inp["k"], "bf16"),
                                     W.as_f64(inp["v"], "bf16"), inp["seq_L"], wp, w0, theta)
    good0 = [h for h in range(Hq) if h not in bad]
    eo = max(np.max(np.abs(o_gpu[0, good0] - o_ref[0, good0])), np.max(np.abs(o_gpu[1] - o_ref[1])))
    _say(f"untouched heads max|dO|={eo:.3e}")
    assert eo <= TOL["bf16"], eo


def test_decode_large_values_unlimited():
    """Decode values go to the bf16 matrix cores as they are: a value element
    of 1e5 gives the oracle's result (relative tolerance on that feature)."""
    torch = _torch()
    B, S, Hq, Hkv, d, wp, w0, theta = 1, 1000, 8, 2, 128, 256, 100, 1e4
    base = W.decode_inputs(B, S, Hq, Hkv, d, "f32", 89)
    v = base["v"].copy()
    v[0, 500, 0, 9] = 1e5
    inp = dict(base, q=W.bf16_bits(base["q"]), k=W.bf16_bits(base["k"]), v=W.bf16_bits(v), dtype="bf16")
    qd, kd, vd = (W.to_device(inp[n], "bf16") for n in ("q", "k", "v"))
    out = jl.decode(qd, kd, vd, torch.from_numpy(inp["seq_L"]).cuda(), wp, w0, theta)
    torch.cuda.synchronize()
    o_gpu = out.float().cpu().numpy().astype(np.float64)
    o_ref, _ = oracle.bifocal_decode(W.as_f64(inp["q"], "bf16"), W.as_f64(inp["k"], "bf16"),
                                     W.as_f64(inp["v"], "bf16"), inp["seq_L"], wp, w0, theta)
    rel = np.max(np.abs(o_gpu - o_ref) / np.maximum(1.0, np.abs(o_ref)))
    _say(f"max rel |dO| = {rel:.3e}")
    assert rel <= TOL["bf16"], rel


# ---------------------------------------------------------------- prepared table

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("prerot", [False, True])
def test_decode_with_table_matches_decode(dt, prerot):
    """decode_with_table over one prepared table (covering more positions than
    max_L) gives exactly the bits of decode, which builds its rows per call,
    for two calls with different lengths and windows; and matches the oracle."""
    torch = _torch()
    B, S, Hq, Hkv, d, wp, theta = 3, 2500, 16, 4, 128, 512, 1e6
    table = jl.rope_table(S + 300, d, theta)
    for seq_L, w0 in (([2500, 1700, 3], 200), ([1024, 1025, 2047], 0)):
        inp = W.decode_inputs(B, S, Hq, Hkv, d, dt, 90, seq_L=seq_L)
        q, k, v = (W.to_device(inp[n], dt) for n in ("q", "k", "v"))
        seq = torch.from_numpy(inp["seq_L"]).cuda()
        o1, l1 = jl.decode(q, k, v, seq, wp, w0, theta, return_lse=True, prerotated=prerot)
        o2, l2 = jl.decode_with_table(q, k, v, seq, wp, w0, table, S + 300, return_lse=True, prerotated=prerot)
        torch.cuda.synchronize()
        _say("decode_with_table", dt, prerot, seq_L, w0)
        assert torch.equal(o1.view(torch.int16) if dt == "bf16" else o1, o2.view(torch.int16) if dt == "bf16" else o2)
        assert torch.equal(l1, l2)
        ref = oracle.bifocal_decode_prerotated if prerot else oracle.bifocal_decode
        o_ref, _ = ref(W.as_f64(inp["q"], dt), W.as_f64(inp["k"], dt), W.as_f64(inp["v"], dt), inp["seq_L"], wp,
                       w0, theta)
        eo = float(np.max(np.abs(o2.float().cpu().numpy() - o_ref)))
        assert eo <= TOL[dt], eo
