"""Inputs with planted keys at the edge of the local window, for tests.

For a query at position i the local window holds the keys at distances
0 .. w0-1 ("Dynamic Bifocal RoPE": classic RoPE at the true positions); the
key at distance w0 already takes the grouped positions f(x) = floor(x / G).
Random N(0, 1) inputs cannot show a pair routed to the wrong side of that
edge: one misrouted key among thousands moves the output by ~1e-3.  Here,
for each chosen query row i, the keys j1 = i - (w0 - 1) (local) and
j2 = i - w0 (remote) are built so that each scores LOGIT (natural units)
with query i in its own branch and far less in the other one, and their
values carry +2 and -2 on one feature: the row's output then depends on
both routing decisions at order 1.

Construction (fp64, then rounded like every other input): query i is
a * e_k on one rotation pair k (feature k of the first half), key j1 is
c * R_k((i - j1) theta_k) e_k and key j2 is c * R_k((f(i) - f(j2)) theta_k) e_k,
with a * c * scale = LOGIT, where R_k turns the pair (k, k + d/2).  Each
planted row gets its own pair k, chosen so that the wrong branch's angle
leaves cos <= 0.6, i.e. a logit drop of 0.4 LOGIT or more (with w0 = 1
the local key is the diagonal, which scores the same in both branches, so
only the remote edge key is observable there).  The expected
outputs always come from the oracle; this module only builds inputs.
"""
from __future__ import annotations

import math

import numpy as np

from zero_shot_rope_bifocal_amd import workloads as W

LOGIT = 12.0


def _freq(d, theta, k):
    return float(theta) ** (-2.0 * k / d)


def _pick_pairs(rows, w0, G, d, theta, max_cos=0.6):
    """Per planted row: a rotation pair whose wrong-branch angle for both
    edge keys leaves cos <= max_cos (rows without one are dropped)."""
    used, out = set(), []
    for i in rows:
        j1, j2 = i - (w0 - 1), i - w0
        best = None
        # prefer a pair no other planted row uses (no crosstalk between
        # planted rows); at w0 = 1 only the fastest pairs qualify, so they are
        # shared (the oracle scores the crosstalk like everything else)
        for k in sorted(range(d // 2), key=lambda k: k in used):
            if best is not None and k in used:
                break
            t = _freq(d, theta, k)
            # the diagonal (w0 = 1) scores the same in both branches: nothing
            # to observe there
            c1 = math.cos(((i // G - j1 // G) - (i - j1)) * t) if j1 != i else -1.0
            c2 = math.cos(((i - j2) - (i // G - j2 // G)) * t)
            worst = max(c1, c2)
            if worst <= max_cos and (best is None or worst < best[1]):
                best = (k, worst)
        if best is not None:
            used.add(best[0])
            out.append((i, best[0]))
    return out


def _plant_row(q_row, k_rows, v_rows, i, pair, w0, G, d, theta, feat, scale, a=4.0):
    """Writes the planted query (all heads of q_row) and its two edge keys and
    values (all KV heads) into float32 arrays indexed by position."""
    c = LOGIT / (scale * a)
    h = d // 2
    t = _freq(d, theta, pair)
    j1, j2 = i - (w0 - 1), i - w0
    q_row[i] = 0.0
    q_row[i, :, pair] = a
    for j, ang in ((j1, (i - j1) * t), (j2, (i // G - j2 // G) * t)):
        k_rows[j] = 0.0
        k_rows[j, :, pair] = c * math.cos(ang)
        k_rows[j, :, pair + h] = c * math.sin(ang)
    v_rows[j1, :, feat] = 2.0
    v_rows[j2, :, feat] = -2.0


def _round(x, dtype):
    return W.bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def edge_prefill(L, Hq, Hkv, d, dtype, wp, w0, theta, seed, spacing=37):
    """One sequence of length L (raw inputs) with planted edge keys for query
    rows w0, w0 + spacing, ...; returns (inputs dict as prefill_inputs,
    planted rows)."""
    assert w0 >= 1 and L > w0
    G = max(1, -(-L // wp))
    inp = W.prefill_inputs([L], Hq, Hkv, d, "f32", seed)
    q = inp["q"] * np.float32(0.25)
    k = inp["k"] * np.float32(0.25)
    v = inp["v"] * np.float32(0.25)
    rows = list(range(w0, L, spacing))
    planted = _pick_pairs(rows, w0, G, d, theta)
    scale = 1.0 / math.sqrt(d)
    for n, (i, pair) in enumerate(planted):
        _plant_row(q, k, v, i, pair, w0, G, d, theta, n % d, scale)
    inp.update(q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype), dtype=dtype)
    return inp, [i for i, _ in planted]


def edge_decode(seq_L, S, Hq, Hkv, d, dtype, wp, w0, theta, seed):
    """Decode caches [B, S, Hkv, d] (raw) where each sequence's query (at
    seq_L[b] - 1) has planted edge keys at distances w0 - 1 and w0."""
    B = len(seq_L)
    inp = W.decode_inputs(B, S, Hq, Hkv, d, "f32", seed, seq_L=seq_L)
    q = inp["q"] * np.float32(0.25)
    k = inp["k"] * np.float32(0.25)
    v = inp["v"] * np.float32(0.25)
    scale = 1.0 / math.sqrt(d)
    planted = []
    for b, L in enumerate(seq_L):
        i = L - 1
        if i < w0:
            continue
        G = max(1, -(-L // wp))
        got = _pick_pairs([i], w0, G, d, theta)
        if not got:
            continue
        pair = got[0][1]
        qb = q[b][None]  # position axis of length 1, holding position i
        # write through a view indexed by position: query slot 0 stands for i
        qpos = np.zeros((i + 1, Hq, d), np.float32)
        _plant_row(qpos, k[b], v[b], i, pair, w0, G, d, theta, b % d, scale)
        qb[0] = qpos[i]
        planted.append(b)
    inp.update(q=_round(q, dtype), k=_round(k, dtype), v=_round(v, dtype), dtype=dtype)
    return inp, planted
