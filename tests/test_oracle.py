"""Pins of the fp64 oracle against what the pages and mathematics fix.

CPU only.  Each test checks the oracle against something other than itself:
hand-derived integers from eq. G / eq. f, a closed-form tiny case, the
textbook special cases (G = 1, w0 >= L, w0 = 0), a brute-force relative-angle
evaluation, the complex-number form of RoPE, and the pages' inclusion-exclusion
identity.  The last test plants plausible mistakes in a copy of the oracle and
checks that at least one pin catches each.
"""
import json
import math
import os
import types

import numpy as np
import pytest

import oracle
import oracle.bifocal as ob
from pins import brute_bifocal, classic_rope_attention, complex_rope

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- integers

def test_group_size_golden():
    g = _load("group_size.json")
    for c in g["group_size"]:
        assert oracle.group_size(c["L"], c["w_pretrained"]) == c["G"], c


def test_remote_map_golden():
    g = _load("group_size.json")
    for c in g["remote_map"]:
        G = oracle.group_size(c["L"], c["w_pretrained"])
        f = oracle.remote_positions(np.arange(c["L"]), G)
        assert f.tolist() == c["f"]
    for c in g["max_remote_position"]:
        G = oracle.group_size(c["L"], c["w_pretrained"])
        assert int(oracle.remote_positions([c["L"] - 1], G)[0]) == c["max_f"]


@pytest.mark.parametrize("L,wp", [(2048, 512), (32768, 32768), (131072, 32768),
                                  (20000, 32768), (70000, 32768), (1024, 512),
                                  (1025, 512), (65536, 32768), (65537, 32768),
                                  (1, 1), (7, 1), (100, 3)])
def test_remote_positions_in_distribution(L, wp):
    """Every remote rotation index lies on the pre-training grid [0, wp), and
    every causal remote angle difference is below wp."""
    G = oracle.group_size(L, wp)
    f = oracle.remote_positions(np.arange(L), G)
    assert f.min() == 0 and f.max() <= wp - 1
    assert np.all(np.diff(f) >= 0)
    assert f[-1] - f[0] < wp
    # minimal compression: with G - 1 the grid would overflow
    if G > 1:
        assert (L - 1) // (G - 1) >= wp


def test_group_size_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.group_size(10, 0)
    with pytest.raises(ValueError):
        oracle.group_size(-1, 4)


# ---------------------------------------------------------------- rotation

def test_rope_frequencies_golden():
    """theta_k at every k (not only k = 0) against hand-derived powers of ten."""
    for c in _load("rope_pairs.json")["frequencies"]:
        got = oracle.rope_frequencies(c["d"], c["theta"])
        assert np.allclose(got, c["theta_k"], rtol=1e-14, atol=0), (c, got)


def test_rope_rotation_golden_higher_pairs():
    """R(p) of a one-hot vector in a pair k >= 1 lands on (cos a, sin a) at the
    pair's two features, a = p * theta_k a whole number of radians."""
    for c in _load("rope_pairs.json")["rotations"]:
        x = np.zeros((1, c["d"]))
        x[0, c["one_hot"]] = 1.0
        got = oracle.rope_rotate(x, [c["p"]], c["theta"])[0]
        want = np.zeros(c["d"])
        want[c["cos_at"]] = math.cos(c["angle_rad"])
        want[c["sin_at"]] = c.get("sin_sign", 1) * math.sin(c["angle_rad"])
        assert np.allclose(got, want, rtol=0, atol=1e-12), (c, got)


def test_rope_matches_complex_form():
    rng = np.random.default_rng(0)
    for d in (2, 8, 64, 128):
        x = _rand(rng, 50, d)
        pos = rng.integers(0, 131072, size=50)
        for theta in (1.0, 1e4, 1e6):
            a = oracle.rope_rotate(x, pos, theta)
            b = complex_rope(x, pos, theta)
            # fp64 angles carry a relative error of a few ulp: bound scales with p
            assert np.max(np.abs(a - b)) < 1e-15 * (1 + pos.max())


def test_rope_closed_form_single_frequency():
    # d = 2: the only frequency is theta^0 = 1, so R(a)(1, 0) = (cos a, sin a)
    for a in (0, 1, 2, 5, 1000, 131071):
        r = oracle.rope_rotate(np.array([[1.0, 0.0]]), [a], 12345.0)[0]
        assert abs(r[0] - math.cos(a)) < 1e-15 and abs(r[1] - math.sin(a)) < 1e-15


def test_rope_composition_and_norm():
    rng = np.random.default_rng(1)
    x = _rand(rng, 40, 64)
    a = rng.integers(0, 40000, size=40)
    b = rng.integers(0, 40000, size=40)
    lhs = oracle.rope_rotate(oracle.rope_rotate(x, a, 1e6), b, 1e6)
    rhs = oracle.rope_rotate(x, a + b, 1e6)
    assert np.max(np.abs(lhs - rhs)) < 1e-11
    assert np.allclose(np.linalg.norm(lhs, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)


def test_correction_rotation_identity():
    """R(f(p) - p) R(p) x = R(f(p)) x: the remote vector is rebuilt from the
    true-position one, which stays untouched."""
    rng = np.random.default_rng(2)
    L, wp = 131072, 32768
    G = oracle.group_size(L, wp)
    pos = np.concatenate([np.arange(8), rng.integers(0, L, size=56)])
    x = _rand(rng, pos.size, 128)
    base = oracle.rope_rotate(x, pos, 1e6)
    keep = base.copy()
    rebuilt = oracle.correction_rotation(base, pos, G, 1e6)
    direct = complex_rope(x, pos // G, 1e6)
    # two rotations with angles up to ~L: a few ulp of 2L of angle error
    assert np.max(np.abs(rebuilt - direct)) < 1e-15 * (1 + 2 * L)
    assert np.array_equal(base, keep)


# ---------------------------------------------------------------- attention

def test_closed_form_case():
    g = _load("closed_form_d2.json")
    L = g["L"]
    q = np.zeros((L, 1, 2))
    q[:, 0, 0] = 1.0
    k = q.copy()
    v = np.eye(L).reshape(L, 1, L)
    o, lse = oracle.bifocal_sequence(q, k, v, np.arange(L), L, g["w_pretrained"],
                                     g["w0"], g["theta"])
    sc = 1.0 / math.sqrt(2.0)
    for i, row in enumerate(g["angle_diff"]):
        logits = [sc * math.cos(a) for a in row]
        m = max(logits)
        w = [math.exp(s - m) for s in logits]
        tot = sum(w)
        want = [x / tot for x in w] + [0.0] * (L - len(w))
        assert np.max(np.abs(o[i, 0] - np.array(want))) < 1e-15
        assert abs(lse[i, 0] - (m + math.log(tot))) < 1e-15


BRUTE_CASES = [
    # (L, d, Hq, Hkv, wp, w0, theta)
    (9, 2, 1, 1, 4, 2, 1.0),
    (12, 4, 2, 1, 5, 3, 100.0),
    (16, 8, 4, 2, 4, 5, 1e4),
    (16, 8, 2, 2, 16, 4, 1e4),      # G = 1
    (13, 4, 2, 2, 3, 0, 10.0),      # w0 = 0: all remote
    (11, 8, 2, 1, 2, 11, 1e6),      # w0 >= L: all local, G = 6
    (16, 4, 3, 1, 1, 1, 50.0),      # wp = 1: G = L, f = 0
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_matches_brute_force(case):
    L, d, Hq, Hkv, wp, w0, theta = case
    rng = np.random.default_rng(hash(case) % 2**32)
    q, k, v = _rand(rng, L, Hq, d), _rand(rng, L, Hkv, d), _rand(rng, L, Hkv, d)
    o, lse = oracle.bifocal_sequence(q, k, v, np.arange(L), L, wp, w0, theta)
    ob_, lb = brute_bifocal(q, k, v, np.arange(L), L, wp, w0, theta)
    assert np.max(np.abs(o - ob_)) < 1e-12
    assert np.max(np.abs(lse - lb)) < 1e-12


def test_g1_reproduces_classic_rope():
    """L <= w_pretrained gives G = 1: classic RoPE causal attention exactly."""
    rng = np.random.default_rng(3)
    for L, wp, w0 in ((64, 64, 16), (40, 512, 0), (33, 33, 5)):
        q, k, v = _rand(rng, L, 4, 16), _rand(rng, L, 2, 16), _rand(rng, L, 2, 16)
        o, _ = oracle.bifocal_sequence(q, k, v, np.arange(L), L, wp, w0, 1e4)
        c = classic_rope_attention(q, k, v, np.arange(L), theta=1e4)
        assert np.max(np.abs(o - c)) < 1e-12


def test_wide_window_reproduces_classic_rope():
    """w0 >= L: every pair is local, whatever G is."""
    rng = np.random.default_rng(4)
    L = 48
    q, k, v = _rand(rng, L, 2, 8), _rand(rng, L, 1, 8), _rand(rng, L, 1, 8)
    o, _ = oracle.bifocal_sequence(q, k, v, np.arange(L), L, 8, L, 1e4)
    c = classic_rope_attention(q, k, v, np.arange(L), theta=1e4)
    assert np.max(np.abs(o - c)) < 1e-12


def test_zero_window_is_grouped_rope():
    """w0 = 0: every pair uses the grouped positions f(p)."""
    rng = np.random.default_rng(5)
    L, wp = 50, 8
    G = oracle.group_size(L, wp)
    q, k, v = _rand(rng, L, 2, 8), _rand(rng, L, 2, 8), _rand(rng, L, 2, 8)
    o, _ = oracle.bifocal_sequence(q, k, v, np.arange(L), L, wp, 0, 1e4)
    c = classic_rope_attention(q, k, v, np.arange(L), k_pos=np.arange(L) // G, theta=1e4)
    assert np.max(np.abs(o - c)) < 1e-12


def test_local_band_logits_are_classic():
    """Routing check on logits: a row's output changes only through remote
    keys when the remote rotation is perturbed (theta of the remote branch),
    i.e. local-band pairs do not depend on f at all."""
    rng = np.random.default_rng(6)
    L, wp, w0 = 40, 10, 7
    q, k = _rand(rng, L, 1, 8), _rand(rng, L, 1, 8)
    # V = identity over keys so O row = attention weights
    v = np.eye(L).reshape(L, 1, L)
    o, _ = oracle.bifocal_sequence(q, k, v, np.arange(L), L, wp, w0, 1e4)
    # rows < w0 have only local keys -> equal to classic RoPE weights
    c = classic_rope_attention(q, k, v, np.arange(L), theta=1e4)
    assert np.max(np.abs(o[:w0] - c[:w0])) < 1e-12
    # for later rows the ratio of two local weights equals the classic ratio
    for i in range(w0, L):
        a, b = i, i - w0 + 1
        assert abs(math.log(o[i, 0, a] / o[i, 0, b]) - math.log(c[i, 0, a] / c[i, 0, b])) < 1e-10


@pytest.mark.parametrize("L,wp,w0", [(40, 8, 6), (64, 16, 0), (64, 16, 64), (70, 7, 13), (33, 33, 4)])
def test_inclusion_exclusion_identity(L, wp, w0):
    """The pages' three-pass merge equals mask-select."""
    rng = np.random.default_rng(L * 1000 + w0)
    q, k, v = _rand(rng, L, 4, 16), _rand(rng, L, 2, 16), _rand(rng, L, 2, 16)
    o, lse = oracle.bifocal_sequence(q, k, v, np.arange(L), L, wp, w0, 1e4)
    o2, lse2 = oracle.bifocal_sequence_ie(q, k, v, np.arange(L), L, wp, w0, 1e4)
    assert np.max(np.abs(o - o2) / (1 + np.abs(o))) < 1e-10
    assert np.max(np.abs(lse - lse2)) < 1e-10


PREROT_CASES = [
    # (L, d, Hq, Hkv, wp, w0, theta)
    (40, 8, 4, 2, 8, 6, 1e4),       # G = 5, straddling window
    (33, 16, 2, 1, 33, 5, 1e4),     # G = 1
    (29, 8, 2, 2, 4, 0, 100.0),     # w0 = 0: all remote
    (25, 4, 2, 1, 3, 30, 1e6),      # w0 >= L: all local
]


@pytest.mark.parametrize("case", PREROT_CASES)
def test_prerotated_cache_matches_raw_inputs(case):
    """Queries and keys handed over already rotated at their true positions
    (the usual RoPE cache) give the bifocal result of the raw vectors: the
    correction rotation R(f(p) - p) composes with R(p) to R(f(p))."""
    L, d, Hq, Hkv, wp, w0, theta = case
    rng = np.random.default_rng(L * 31 + d)
    q, k, v = _rand(rng, L, Hq, d), _rand(rng, L, Hkv, d), _rand(rng, L, Hkv, d)
    pos = np.arange(L)
    q_rot = np.stack([complex_rope(q[:, h], pos, theta) for h in range(Hq)], axis=1)
    k_rot = np.stack([complex_rope(k[:, h], pos, theta) for h in range(Hkv)], axis=1)
    o1, l1 = oracle.bifocal_sequence_prerotated(q_rot, k_rot, v, pos, L, wp, w0, theta)
    o2, l2 = brute_bifocal(q, k, v, pos, L, wp, w0, theta)
    assert np.max(np.abs(o1 - o2)) < 1e-10
    assert np.max(np.abs(l1 - l2)) < 1e-10


def test_prerotated_wide_window_is_plain_attention():
    """w0 >= L over a pre-rotated cache: textbook causal softmax attention of
    the stored vectors, no rotation at all."""
    rng = np.random.default_rng(8)
    L, d = 21, 8
    q, k, v = _rand(rng, L, 2, d), _rand(rng, L, 1, d), _rand(rng, L, 1, d)
    o, lse = oracle.bifocal_sequence_prerotated(q, k, v, np.arange(L), L, 4, L, 1e4)
    for h in range(2):
        s = (q[:, h] @ k[:, 0].T) / math.sqrt(d)
        s[np.triu_indices(L, 1)] = -np.inf
        w = np.exp(s - s.max(axis=1, keepdims=True))
        ref = (w @ v[:, 0]) / w.sum(axis=1, keepdims=True)
        assert np.max(np.abs(o[:, h] - ref)) < 1e-12


def test_prerotated_decode_is_last_row():
    rng = np.random.default_rng(9)
    L, d = 30, 8
    q, k, v = _rand(rng, L, 4, d), _rand(rng, L, 2, d), _rand(rng, L, 2, d)
    full, _ = oracle.bifocal_sequence_prerotated(q, k, v, np.arange(L), L, 7, 4, 1e4)
    dec, _ = oracle.bifocal_decode_prerotated(q[L - 1:L], k[None], v[None], [L], 7, 4, 1e4)
    assert np.max(np.abs(dec[0] - full[L - 1])) < 1e-12


def test_decode_is_last_prefill_row():
    rng = np.random.default_rng(7)
    B, S, Hq, Hkv, d = 3, 40, 4, 2, 16
    kc, vc = _rand(rng, B, S, Hkv, d), _rand(rng, B, S, Hkv, d)
    q = _rand(rng, B, Hq, d)
    seq_L = [40, 17, 1]
    o, lse = oracle.bifocal_decode(q, kc, vc, seq_L, 8, 5, 1e4)
    for b, L in enumerate(seq_L):
        qf = np.zeros((L, Hq, d))
        qf[L - 1] = q[b]
        op, lp = oracle.bifocal_sequence(qf, kc[b, :L], vc[b, :L], np.arange(L), L, 8, 5, 1e4)
        assert np.max(np.abs(o[b] - op[L - 1])) < 1e-13
        ob_, _ = brute_bifocal(q[b:b + 1], kc[b, :L], vc[b, :L], [L - 1], L, 8, 5, 1e4)
        assert np.max(np.abs(o[b] - ob_[0])) < 1e-12


def test_varlen_prefill_is_per_sequence():
    rng = np.random.default_rng(8)
    lens = [5, 0, 17, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v = _rand(rng, T, 2, 8), _rand(rng, T, 1, 8), _rand(rng, T, 1, 8)
    o, lse = oracle.bifocal_prefill(q, k, v, cu, 4, 3, 1e4)
    for b, L in enumerate(lens):
        if L == 0:
            continue
        a = cu[b]
        ob_, lb = brute_bifocal(q[a:a + L], k[a:a + L], v[a:a + L], np.arange(L), L, 4, 3, 1e4)
        assert np.max(np.abs(o[a:a + L] - ob_)) < 1e-12
        assert np.max(np.abs(lse[a:a + L] - lb)) < 1e-12


def test_sampled_rows_match_full():
    rng = np.random.default_rng(9)
    L = 80
    q, k, v = _rand(rng, L, 2, 8), _rand(rng, L, 1, 8), _rand(rng, L, 1, 8)
    o, lse = oracle.bifocal_sequence(q, k, v, np.arange(L), L, 16, 9, 1e4)
    rows = np.array([0, 3, 8, 9, 40, 79])
    o2, l2 = oracle.bifocal_rows(q, k, v, rows, L, 16, 9, 1e4)
    assert np.array_equal(o[rows], o2) and np.array_equal(lse[rows], l2)


def test_chunked_queries_match_full():
    """Queries at offset positions (a chunk at the end) see the same result as
    the corresponding rows of the full prefill."""
    rng = np.random.default_rng(10)
    L, n = 60, 13
    q, k, v = _rand(rng, L, 2, 8), _rand(rng, L, 2, 8), _rand(rng, L, 2, 8)
    o, _ = oracle.bifocal_sequence(q, k, v, np.arange(L), L, 16, 7, 1e4)
    oc, _ = oracle.bifocal_sequence(q[L - n:], k, v, np.arange(L - n, L), L, 16, 7, 1e4)
    assert np.array_equal(o[L - n:], oc)


# ---------------------------------------------------------------- tiles

def test_tile_classes_golden():
    for c in _load("tile_classes.json")["cases"]:
        got = oracle.tile_classes(c["Lq"], c["L"], c["q_offset"], c["w0"], c["BM"], c["BN"])
        assert got.tolist() == c["classes"], c


# ---------------------------------------------------------------- mutation

def _pins_pass(mod) -> bool:
    """Runs a compact set of the pins above against a (possibly mutated)
    copy of the oracle module; True if every pin holds."""
    try:
        for c in _load("group_size.json")["group_size"]:
            if mod.group_size(c["L"], c["w_pretrained"]) != c["G"]:
                return False
        g = _load("closed_form_d2.json")
        L = g["L"]
        q = np.zeros((L, 1, 2)); q[:, 0, 0] = 1.0
        v = np.eye(L).reshape(L, 1, L)
        o, _ = mod.bifocal_sequence(q, q.copy(), v, np.arange(L), L, g["w_pretrained"], g["w0"], g["theta"])
        sc = 1.0 / math.sqrt(2.0)
        for i, row in enumerate(g["angle_diff"]):
            w = [math.exp(sc * math.cos(a)) for a in row]
            want = np.array([x / sum(w) for x in w] + [0.0] * (L - len(w)))
            if np.max(np.abs(o[i, 0] - want)) > 1e-12:
                return False
        for case in BRUTE_CASES:
            Lb, d, Hq, Hkv, wp, w0, theta = case
            rng = np.random.default_rng(11)
            q, k, v = _rand(rng, Lb, Hq, d), _rand(rng, Lb, Hkv, d), _rand(rng, Lb, Hkv, d)
            o, lse = mod.bifocal_sequence(q, k, v, np.arange(Lb), Lb, wp, w0, theta)
            ob_, lb = brute_bifocal(q, k, v, np.arange(Lb), Lb, wp, w0, theta)
            if np.max(np.abs(o - ob_)) > 1e-10 or np.max(np.abs(lse - lb)) > 1e-10:
                return False
        for c in _load("tile_classes.json")["cases"]:
            got = mod.tile_classes(c["Lq"], c["L"], c["q_offset"], c["w0"], c["BM"], c["BN"])
            if got.tolist() != c["classes"]:
                return False
    except Exception:
        return False
    return True


MUTATIONS = [
    ("dist < w0, s_loc, s_rem", "dist <= w0, s_loc, s_rem"),                 # window off by one
    ("x1 * c - x2 * s, x2 * c + x1 * s", "x1 * c + x2 * s, x2 * c - x1 * s"),  # rotation sign
    ("return max(1, -(-L // w_pretrained))", "return max(1, L // w_pretrained)"),  # floor for ceil
    ("vh = v[:, hk]", "vh = v[:, (hk + 1) % Hkv]"),                          # wrong KV head for V
    ("s = np.where(dist < 0, -np.inf, s)", "s = np.where(dist < -1, -np.inf, s)"),  # causal off by one
    ("-2.0 * k / d)", "-1.0 * k / d)"),                                      # frequency formula
    ("kr = rope_rotate(k[:, hk], fk, theta)", "kr = rope_rotate(k[:, hk], kpos, theta)"),  # keys not grouped
    ("out[r0:r1, h] = (p @ vh) / l", "out[r0:r1, h] = (p @ vh)"),            # dropped normalisation
    ("lse[r0:r1, h] = (m + np.log(l))[:, 0]", "lse[r0:r1, h] = m[:, 0]"),    # dropped LSE term
    ("ql = rope_rotate(q[:, h], q_pos, theta)\n            qr = rope_rotate(q[:, h], fq, theta)",
     "ql = rope_rotate(q[:, h], q_pos + 1, theta)\n            qr = rope_rotate(q[:, h], fq, theta)"),  # query position shift
    ("qr = rope_rotate(q[:, h], fq, theta)", "qr = rope_rotate(q[:, h], q_pos, theta)"),  # queries not grouped
    ("near = (dist < w0)[causal]", "near = (dist <= w0)[causal]"),          # tile window off by one
    ("if (~causal).any():", "if (~causal).all():"),                          # diag flag
]


def test_unmutated_oracle_passes_pins():
    assert _pins_pass(ob)


@pytest.mark.parametrize("old,new", MUTATIONS)
def test_planted_mistake_is_caught(old, new):
    src = open(ob.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    assert not _pins_pass(mod), f"mutation not caught: {new}"
