"""Independent formulations used to pin the oracle (tests only).

Nothing here reuses the oracle's code paths:

* ``brute_bifocal`` scores every pair with the relative-angle form of the RoPE
  inner product, <R(a)q, R(b)k> = sum_k (q_k k_k + q_{k+h} k_{k+h}) cos((a-b) t_k)
  - (q_{k+h} k_k - q_k k_{k+h}) sin((a-b) t_k), h = d/2, in pure Python with
  ``math.fsum`` and an explicit softmax.  The oracle instead rotates each
  vector by its absolute angle and uses numpy matrix products.
* ``classic_rope_attention`` is textbook RoPE causal attention written with
  complex numbers (pair (x_k, x_{k+h}) as x_k + i x_{k+h}, rotation as a
  multiplication by exp(i p t_k)).
"""
from __future__ import annotations

import math

import numpy as np


def brute_bifocal(q, k, v, q_pos, L, w_pretrained, w0, theta, scale=None):
    """q: [n, Hq, d]; k: [L, Hkv, d]; v: [L, Hkv, dv]; returns (O, LSE) as
    numpy fp64.  Pure-Python per-pair loop: tiny inputs only."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, Hq, d = q.shape
    Hkv = k.shape[1]
    h = d // 2
    G = max(1, (L + w_pretrained - 1) // w_pretrained)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    freqs = [float(theta) ** (-2.0 * t / d) for t in range(h)]
    out = np.zeros((n, Hq, v.shape[2]))
    lse = np.zeros((n, Hq))
    for r in range(n):
        i = int(q_pos[r])
        for hq in range(Hq):
            hk = hq // (Hq // Hkv)
            qv = [float(x) for x in q[r, hq]]
            logits = []
            for j in range(i + 1):
                kv = [float(x) for x in k[j, hk]]
                if i - j < w0:
                    a, b = i, j
                else:
                    a, b = i // G, j // G
                terms = []
                for t in range(h):
                    phi = (a - b) * freqs[t]
                    re = qv[t] * kv[t] + qv[t + h] * kv[t + h]
                    im = qv[t + h] * kv[t] - qv[t] * kv[t + h]
                    terms.append(re * math.cos(phi))
                    terms.append(-im * math.sin(phi))
                logits.append(scale * math.fsum(terms))
            m = max(logits)
            w = [math.exp(s - m) for s in logits]
            tot = math.fsum(w)
            for e in range(v.shape[2]):
                out[r, hq, e] = math.fsum(w[j] * float(v[j, hk, e]) for j in range(i + 1)) / tot
            lse[r, hq] = m + math.log(tot)
    return out, lse


def complex_rope(x, positions, theta):
    """Textbook RoPE via complex multiplication; x [n, d] real -> [n, d]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    t = np.array([float(theta) ** (-2.0 * j / d) for j in range(h)])
    z = x[:, :h] + 1j * x[:, h:]
    z = z * np.exp(1j * np.outer(np.asarray(positions, dtype=np.float64), t))
    return np.concatenate([z.real, z.imag], axis=1)


def classic_rope_attention(q, k, v, q_pos, k_pos=None, theta=10000.0, scale=None):
    """Standard causal RoPE attention of one sequence with an arbitrary
    integer position per token (default: keys at 0 .. L-1).  Causality is by
    token index (key index <= query's own index in ``q_pos`` order of the
    sequence), which is what the bifocal method keeps."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, Hq, d = q.shape
    L, Hkv, _ = k.shape
    q_idx = np.asarray(q_pos, dtype=np.int64)
    if k_pos is None:
        k_pos = np.arange(L)
        qp = q_idx
    else:
        qp = np.asarray(k_pos)[q_idx]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((n, Hq, v.shape[2]))
    for hq in range(Hq):
        hk = hq // (Hq // Hkv)
        qr = complex_rope(q[:, hq], qp, theta)
        kr = complex_rope(k[:, hk], k_pos, theta)
        s = scale * np.einsum("nd,ld->nl", qr, kr)
        allowed = np.arange(L)[None, :] <= q_idx[:, None]
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, hq] = p @ v[:, hk]
    return out
