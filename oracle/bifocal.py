"""Plain fp64 CPU oracle for dynamic bifocal RoPE attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import this module:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.  It shares no code, table or constant with the HIP library
and imports nothing from it.

Source of the method: "Jet-Long: Efficient Long-Context Extension with Dynamic
Bifocal RoPE" (gist.science summaries, paper 2607.07740), section "Dynamic
Bifocal RoPE" (the equations for the group size G and the remote map f) and
section "Inference Efficiency Mechanisms" (the correction rotation and the
inclusion-exclusion merge).

What is computed, written out as its plain definition (no tiling, no online
softmax, no merge):

* G = max(1, ceil(L / w_pretrained)) from the current length L, in exact
  integers (eq. G); f(x) = floor(x / G) (eq. f).
* Classic RoPE at true positions for pairs closer than w0 (the local window);
  RoPE at the grouped positions f(p_i), f(p_j) for every other causal pair.
* Full local and remote logit rows, mask-select by distance, causal softmax,
  times V.

Readings where the pages are silent:
* RoPE itself is not defined on the pages: standard RoPE with
  theta_k = theta^(-2k/d), rotate-half pairing (dims k and k + d/2).
* The remote branch rotates each token by f of its own absolute position, with
  no extra offset.
* The local window holds distances 0 .. w0-1; w0 = 0 makes every pair remote.
* Softmax scale 1/sqrt(d), no temperature.
* GQA: query head h reads KV head h // (Hq / Hkv).
* In decode L counts the new token, whose K/V is already in the cache; the
  query sits at position L - 1.

Every function here is pinned by ``tests/test_oracle_*.py`` against values the
pages' formulas fix (hand-derived integers and a closed-form case), textbook
special cases (G = 1 gives classic RoPE attention) and a brute-force
relative-angle evaluation on tiny inputs.
"""
from __future__ import annotations

import numpy as np

# tile classes (shared vocabulary with the tests; the values are a labelling
# choice, not part of the method)
SKIP, LOCAL, REMOTE, STRADDLE = 0, 1, 2, 3
DIAG = 4  # flag bit: the tile holds at least one pair with key after query


def group_size(L: int, w_pretrained: int) -> int:
    """G = max(1, ceil(L / w_pretrained)) in exact integers (eq. G of the
    "Dynamic Bifocal RoPE" section)."""
    L = int(L)
    w_pretrained = int(w_pretrained)
    if L < 0 or w_pretrained < 1:
        raise ValueError("need L >= 0 and w_pretrained >= 1")
    return max(1, -(-L // w_pretrained))


def remote_positions(positions, G: int) -> np.ndarray:
    """f(x) = floor(x / G) for non-negative integer positions (eq. f)."""
    p = np.asarray(positions, dtype=np.int64)
    if np.any(p < 0):
        raise ValueError("positions must be non-negative")
    return p // int(G)


def rope_frequencies(d: int, theta: float) -> np.ndarray:
    """theta_k = theta^(-2k/d), k = 0 .. d/2-1, fp64 (standard RoPE; the pages
    name RoPE without defining it)."""
    if d % 2:
        raise ValueError("head_dim must be even")
    k = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * k / d)


def rope_rotate(x: np.ndarray, positions, theta: float) -> np.ndarray:
    """R(p) x for rows of x, rotate-half pairing, in fp64.

    x: [n, ..., d]; positions: [n] integers.  Pair (x_k, x_{k+d/2}) turns by
    the angle p * theta_k.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    inv = rope_frequencies(d, theta)
    p = np.asarray(positions, dtype=np.int64).astype(np.float64)
    ang = p[:, None] * inv[None, :]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (h,)
    c = np.cos(ang).reshape(shape)
    s = np.sin(ang).reshape(shape)
    x1 = x[..., :h]
    x2 = x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _row_block(L: int) -> int:
    return max(1, (1 << 23) // max(L, 1))


def bifocal_sequence(q, k, v, q_pos, L: int, w_pretrained: int, w0: int,
                     theta: float, scale: float | None = None):
    """Bifocal attention of one sequence, fp64, by mask-select.

    q: [n, Hq, d] queries at integer positions q_pos [n] (each < L);
    k: [L, Hkv, d], v: [L, Hkv, dv] keys/values at positions 0 .. L-1.
    Returns (O [n, Hq, dv], LSE [n, Hq]) with LSE the natural-log
    log-sum-exp of the selected, scaled logits of each row.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n, Hq, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != L or v.shape[0] != L:
        raise ValueError("k and v must hold L rows")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if n and (q_pos.min() < 0 or q_pos.max() >= L):
        raise ValueError("query positions must lie in [0, L)")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = group_size(L, w_pretrained)
    kpos = np.arange(L, dtype=np.int64)
    fq = remote_positions(q_pos, G)
    fk = remote_positions(kpos, G)
    rep = Hq // Hkv
    out = np.zeros((n, Hq, v.shape[2]), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    for hk in range(Hkv):
        kl = rope_rotate(k[:, hk], kpos, theta)       # classic RoPE keys
        kr = rope_rotate(k[:, hk], fk, theta)         # grouped-position keys
        vh = v[:, hk]
        for h in range(hk * rep, (hk + 1) * rep):
            ql = rope_rotate(q[:, h], q_pos, theta)
            qr = rope_rotate(q[:, h], fq, theta)
            blk = _row_block(L)
            for r0 in range(0, n, blk):
                r1 = min(n, r0 + blk)
                s_loc = scale * (ql[r0:r1] @ kl.T)
                s_rem = scale * (qr[r0:r1] @ kr.T)
                dist = q_pos[r0:r1, None] - kpos[None, :]
                s = np.where(dist < w0, s_loc, s_rem)
                s = np.where(dist < 0, -np.inf, s)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                l = p.sum(axis=1, keepdims=True)
                out[r0:r1, h] = (p @ vh) / l
                lse[r0:r1, h] = (m + np.log(l))[:, 0]
    return out, lse


def bifocal_prefill(q, k, v, cu_seqlens, w_pretrained: int, w0: int,
                    theta: float, scale: float | None = None):
    """Packed varlen prefill: sequence b owns rows cu_seqlens[b] ..
    cu_seqlens[b+1]-1 of q, k, v, at positions 0 .. L_b-1.  Returns
    (O [T, Hq, dv], LSE [T, Hq])."""
    cu = [int(c) for c in cu_seqlens]
    q = np.asarray(q)
    T, Hq, _ = q.shape
    out = np.zeros((T, Hq, np.asarray(v).shape[2]), dtype=np.float64)
    lse = np.zeros((T, Hq), dtype=np.float64)
    for b in range(len(cu) - 1):
        a, e = cu[b], cu[b + 1]
        L = e - a
        if L == 0:
            continue
        o, s = bifocal_sequence(q[a:e], k[a:e], v[a:e], np.arange(L), L,
                                w_pretrained, w0, theta, scale)
        out[a:e] = o
        lse[a:e] = s
    return out, lse


def bifocal_rows(q, k, v, rows, L: int, w_pretrained: int, w0: int,
                 theta: float, scale: float | None = None):
    """Prefill output of one sequence restricted to the query rows ``rows``
    (row index = position).  q: [L, Hq, d] (only the listed rows are read)."""
    rows = np.asarray(rows, dtype=np.int64)
    return bifocal_sequence(np.asarray(q)[rows], k, v, rows, L, w_pretrained,
                            w0, theta, scale)


def bifocal_decode(q, k_cache, v_cache, seq_L, w_pretrained: int, w0: int,
                   theta: float, scale: float | None = None):
    """One new query per sequence.  q: [B, Hq, d]; caches [B, S_max, Hkv, d];
    seq_L[b] keys are valid (the new token included); the query sits at
    position seq_L[b] - 1.  Returns (O [B, Hq, dv], LSE [B, Hq])."""
    q = np.asarray(q)
    B, Hq, _ = q.shape
    out = np.zeros((B, Hq, np.asarray(v_cache).shape[3]), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    for b in range(B):
        L = int(seq_L[b])
        o, s = bifocal_sequence(q[b:b + 1], k_cache[b, :L], v_cache[b, :L],
                                [L - 1], L, w_pretrained, w0, theta, scale)
        out[b] = o[0]
        lse[b] = s[0]
    return out, lse


def masked_attention(qr, kr, v, mask, scale):
    """Softmax attention of rotated rows qr [n, d] against kr [L, d] over the
    pairs where mask [n, L] is true.  Rows with no pair return O = 0 and
    LSE = -inf.  fp64."""
    s = scale * (qr @ kr.T)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(empty[:, None], 0.0, (p @ v) / np.where(l > 0, l, 1.0))
        lse = np.where(empty, -np.inf, m[:, 0] + np.log(np.where(l[:, 0] > 0, l[:, 0], 1.0)))
    return o, lse


def bifocal_sequence_ie(q, k, v, q_pos, L: int, w_pretrained: int, w0: int,
                        theta: float, scale: float | None = None):
    """The pages' own route to the same result ("Inclusion-Exclusion Attention
    Merge"): three plain attention passes merged with their log-sum-exp
    statistics.  Pass 1: local window with base (true-position) q/k.  Pass 2:
    full causal attention with remote q/k.  Pass 3: local window with remote
    q/k, subtracted.  Returns (O, LSE) like ``bifocal_sequence``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n, Hq, d = q.shape
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = group_size(L, w_pretrained)
    kpos = np.arange(L, dtype=np.int64)
    dist = q_pos[:, None] - kpos[None, :]
    causal = dist >= 0
    window = causal & (dist < w0)
    rep = Hq // Hkv
    out = np.zeros((n, Hq, v.shape[2]))
    lse = np.zeros((n, Hq))
    for hk in range(Hkv):
        kl = rope_rotate(k[:, hk], kpos, theta)
        kr = rope_rotate(k[:, hk], remote_positions(kpos, G), theta)
        for h in range(hk * rep, (hk + 1) * rep):
            ql = rope_rotate(q[:, h], q_pos, theta)
            qr = rope_rotate(q[:, h], remote_positions(q_pos, G), theta)
            o1, s1 = masked_attention(ql, kl, v[:, hk], window, scale)
            o2, s2 = masked_attention(qr, kr, v[:, hk], causal, scale)
            o3, s3 = masked_attention(qr, kr, v[:, hk], window, scale)
            M = np.maximum(s1, s2)
            w1 = np.exp(s1 - M)
            w2 = np.exp(s2 - M)
            w3 = np.exp(s3 - M)
            den = w1 + w2 - w3
            out[:, h] = (w1[:, None] * o1 + w2[:, None] * o2 - w3[:, None] * o3) / den[:, None]
            lse[:, h] = M + np.log(den)
    return out, lse


def correction_rotation(x_rot, positions, G: int, theta: float):
    """Remote vectors rebuilt from vectors already rotated at their true
    positions p: R(f(p) - p) R(p) x = R(f(p)) x ("On-the-Fly Correction
    Rotation").  The stored rotated vectors are read only."""
    p = np.asarray(positions, dtype=np.int64)
    return rope_rotate(x_rot, remote_positions(p, G) - p, theta)


def bifocal_sequence_prerotated(q_rot, k_rot, v, q_pos, L: int, w_pretrained: int,
                                w0: int, theta: float, scale: float | None = None):
    """Bifocal attention of one sequence whose queries and keys arrive already
    rotated at their true positions (q_rot = R(p_i) q, k_rot = R(p_j) k, the
    usual RoPE cache).  Local logits are q_rot . k_rot as stored; remote
    logits use the correction rotation R(f(p) - p) on both sides ("On-the-Fly
    Correction Rotation"), so the stored vectors are never rewritten.  Same
    arguments and returns as bifocal_sequence, fp64, mask-select."""
    q_rot = np.asarray(q_rot, dtype=np.float64)
    k_rot = np.asarray(k_rot, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n, Hq, d = q_rot.shape
    Hkv = k_rot.shape[1]
    if k_rot.shape[0] != L or v.shape[0] != L:
        raise ValueError("k and v must hold L rows")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if n and (q_pos.min() < 0 or q_pos.max() >= L):
        raise ValueError("query positions must lie in [0, L)")
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    G = group_size(L, w_pretrained)
    kpos = np.arange(L, dtype=np.int64)
    rep = Hq // Hkv
    out = np.zeros((n, Hq, v.shape[2]), dtype=np.float64)
    lse = np.zeros((n, Hq), dtype=np.float64)
    for hk in range(Hkv):
        kl = k_rot[:, hk]                                  # as stored
        kr = correction_rotation(k_rot[:, hk], kpos, G, theta)
        vals = v[:, hk]
        for h in range(hk * rep, (hk + 1) * rep):
            ql = q_rot[:, h]
            qr = correction_rotation(q_rot[:, h], q_pos, G, theta)
            blk = _row_block(L)
            for r0 in range(0, n, blk):
                r1 = min(n, r0 + blk)
                gap = q_pos[r0:r1, None] - kpos[None, :]         # causal distance
                logit = np.where(gap >= w0, scale * (qr[r0:r1] @ kr.T), scale * (ql[r0:r1] @ kl.T))
                logit[gap < 0] = -np.inf
                top = logit.max(axis=1, keepdims=True)
                wgt = np.exp(logit - top)
                z = wgt.sum(axis=1, keepdims=True)
                out[r0:r1, h] = (wgt @ vals) / z
                lse[r0:r1, h] = top[:, 0] + np.log(z[:, 0])
    return out, lse


def bifocal_decode_prerotated(q_rot, k_cache_rot, v_cache, seq_L, w_pretrained: int,
                              w0: int, theta: float, scale: float | None = None):
    """Decode over a pre-rotated cache (see bifocal_sequence_prerotated); the
    new query, rotated at its position seq_L[b] - 1, is q_rot[b]."""
    q_rot = np.asarray(q_rot)
    B, Hq, _ = q_rot.shape
    out = np.zeros((B, Hq, np.asarray(v_cache).shape[3]), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    for b in range(B):
        L = int(seq_L[b])
        o, s = bifocal_sequence_prerotated(q_rot[b:b + 1], k_cache_rot[b, :L], v_cache[b, :L],
                                           [L - 1], L, w_pretrained, w0, theta, scale)
        out[b] = o[0]
        lse[b] = s[0]
    return out, lse


def tile_classes(Lq: int, L: int, q_offset: int, w0: int, BM: int, BN: int):
    """Class of every (query block, key tile) of one sequence, decided pair by
    pair.  Query rows are positions q_offset .. q_offset+Lq-1 in blocks of BM
    rows; keys are positions 0 .. L-1 in tiles of BN.  A tile is SKIP if no
    pair in it is causal (key at or before query); LOCAL if every causal pair
    is closer than w0; REMOTE if none is; STRADDLE otherwise.  The DIAG bit is
    set on a non-SKIP tile that also holds a pair with the key after the
    query.  Returns uint8 [ceil(Lq/BM), ceil(L/BN)]."""
    nqb = -(-Lq // BM)
    nkb = -(-L // BN)
    out = np.zeros((nqb, nkb), dtype=np.uint8)
    for a in range(nqb):
        qi = q_offset + np.arange(a * BM, min(Lq, (a + 1) * BM))
        for b in range(nkb):
            kj = np.arange(b * BN, min(L, (b + 1) * BN))
            dist = qi[:, None] - kj[None, :]
            causal = dist >= 0
            if not causal.any():
                out[a, b] = SKIP
                continue
            near = (dist < w0)[causal]
            if near.all():
                c = LOCAL
            elif not near.any():
                c = REMOTE
            else:
                c = STRADDLE
            if (~causal).any():
                c |= DIAG
            out[a, b] = c
    return out
