"""Named workloads and their seeded synthetic inputs.

This module holds no arithmetic of the attention method: it only draws
i.i.d. N(0, 1) numbers from seeded numpy PCG64 generators, rounds them to
bfloat16 (round to nearest even) where the workload is bf16, and packs
variable-length batches.  The HIP path and the CPU oracle both read the same
arrays.

The shapes stand in for the setting the Jet-Long pages evaluate (section
"Experimental Results": Qwen3 models with a 32K native window extended to
128K); the pages give no head counts, so 32 query / 8 KV heads of dimension
128 are used.  No benchmark item of any evaluation suite is reproduced.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

WORKLOADS = {
    # tiny fp32 prefill: parity at 1e-4
    "tiny_f32": dict(kind="prefill", dtype="f32", lens=[2048], Hq=2, Hkv=2, d=64,
                     w_pretrained=512, w0=128, theta=1e4, seed=1),
    # L = w_pretrained: G = 1, must equal classic RoPE causal attention
    "short_bf16": dict(kind="prefill", dtype="bf16", lens=[32768], Hq=32, Hkv=8, d=128,
                       w_pretrained=32768, w0=2048, theta=1e6, seed=2),
    # 128K prefill, G = 4, 64 key rows scaled x4 for peaked attention
    "long_bf16": dict(kind="prefill", dtype="bf16", lens=[131072], Hq=32, Hkv=8, d=128,
                      w_pretrained=32768, w0=2048, theta=1e6, seed=3,
                      peaked_rows=64, peak_seed=1003, peak_scale=4.0),
    # decode: 16 sequences, full 128K caches, G = 4
    "decode_bf16": dict(kind="decode", dtype="bf16", B=16, L=131072, Hq=32, Hkv=8, d=128,
                        w_pretrained=32768, w0=2048, theta=1e6, seed=4),
    # ragged varlen prefill, G = 1 / 3 / 4
    "ragged_bf16": dict(kind="prefill", dtype="bf16", lens=[20000, 70000, 131072], Hq=32, Hkv=8,
                        d=128, w_pretrained=32768, w0=2048, theta=1e6, seed=5),
}

_CHUNK = 1 << 22
_THREADS = min(16, os.cpu_count() or 1)


def _bf16_from_f32(x: np.ndarray) -> np.ndarray:
    u = x.view(np.uint32)
    return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even.  The
    inputs are finite, so the 32-bit sum cannot overflow and no NaN handling
    is needed."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    fx, fo = x.reshape(-1), out.reshape(-1)
    for a in range(0, fx.size, _CHUNK):
        fo[a:a + _CHUNK] = _bf16_from_f32(fx[a:a + _CHUNK])
    return out


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> their exact float32 values."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _normals(seed: int, stream: int, shape, bf16: bool) -> np.ndarray:
    """N(0, 1) draws for one array of a workload.  Element chunk c (2^22
    elements, row-major order) comes from PCG64 seeded with
    SeedSequence(seed, spawn_key=(stream, c)), so the values do not depend on
    how many threads fill the array."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)

    def fill(c):
        a = c * _CHUNK
        m = min(_CHUNK, n - a)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, c))))
        x = rng.standard_normal(m, dtype=np.float32)
        out[a:a + m] = _bf16_from_f32(x) if bf16 else x

    nchunks = -(-n // _CHUNK)
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with cf.ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def normals_range(seed: int, stream: int, start: int, count: int, bf16: bool) -> np.ndarray:
    """Elements [start, start + count) (row-major order) of the array that
    ``_normals(seed, stream, shape, bf16)`` returns, drawing only the chunks
    that hold them."""
    out = np.empty(count, dtype=np.uint16 if bf16 else np.float32)
    c0, c1 = start // _CHUNK, (start + count + _CHUNK - 1) // _CHUNK
    for c in range(c0, c1):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, c))))
        x = rng.standard_normal(_CHUNK, dtype=np.float32)
        a, b = max(start, c * _CHUNK), min(start + count, (c + 1) * _CHUNK)
        out[a - start:b - start] = (_bf16_from_f32(x) if bf16 else x)[a - c * _CHUNK:b - c * _CHUNK]
    return out


def _peak_rows(L0, peaked_rows, peak_seed):
    return np.sort(np.random.default_rng(peak_seed).choice(L0, peaked_rows, replace=False))


def _scale_rows(k, rows, scale, bf16):
    if bf16:
        k[rows] = bf16_bits(bits_to_f32(k[rows]) * np.float32(scale))
    else:
        k[rows] *= np.float32(scale)


def prefill_kv(name: str):
    """(k, v) of a named one-sequence prefill workload, exactly as
    ``workload_inputs(name)`` holds them, without drawing the queries."""
    w = WORKLOADS[name]
    L, bf16 = w["lens"][0], w["dtype"] == "bf16"
    k = _normals(w["seed"], 1, (L, w["Hkv"], w["d"]), bf16)
    v = _normals(w["seed"], 2, (L, w["Hkv"], w["d"]), bf16)
    if w.get("peaked_rows", 0):
        _scale_rows(k, _peak_rows(L, w["peaked_rows"], w["peak_seed"]), w["peak_scale"], bf16)
    return k, v


def prefill_q_rows(name: str, row0: int, nrows: int):
    """Query rows [row0, row0 + nrows) of a named prefill workload."""
    w = WORKLOADS[name]
    n = w["Hq"] * w["d"]
    x = normals_range(w["seed"], 0, row0 * n, nrows * n, w["dtype"] == "bf16")
    return x.reshape(nrows, w["Hq"], w["d"])


def decode_sequence(name: str, b: int):
    """(q [1, Hq, d], k [1, S, Hkv, d], v [1, S, Hkv, d]) of sequence b of a
    named decode workload, exactly as ``workload_inputs(name)`` holds them."""
    w = WORKLOADS[name]
    bf16 = w["dtype"] == "bf16"
    nq, nk = w["Hq"] * w["d"], w["L"] * w["Hkv"] * w["d"]
    q = normals_range(w["seed"], 0, b * nq, nq, bf16).reshape(1, w["Hq"], w["d"])
    k = normals_range(w["seed"], 1, b * nk, nk, bf16).reshape(1, w["L"], w["Hkv"], w["d"])
    v = normals_range(w["seed"], 2, b * nk, nk, bf16).reshape(1, w["L"], w["Hkv"], w["d"])
    return q, k, v


def prefill_inputs(lens, Hq, Hkv, d, dtype, seed, peaked_rows=0, peak_seed=0, peak_scale=1.0,
                   q_lens=None):
    """Packed batch: q [Tq, Hq, d], k/v [Tk, Hkv, d] drawn as streams 0, 1, 2
    of ``seed`` (see ``_normals``).  bf16 arrays are uint16 bit patterns, f32
    arrays float32.  ``q_lens`` (default = lens) takes each sequence's queries
    from its last q_lens[b] positions (the other query rows are never
    drawn).  ``peaked_rows`` key rows of the first sequence, chosen by
    ``default_rng(peak_seed)``, are multiplied by ``peak_scale`` in every KV
    head and feature (a power of two: exact in bf16)."""
    lens = [int(x) for x in lens]
    q_lens = lens if q_lens is None else [int(x) for x in q_lens]
    bf16 = dtype == "bf16"
    Tq, Tk = sum(q_lens), sum(lens)
    q = _normals(seed, 0, (Tq, Hq, d), bf16)
    k = _normals(seed, 1, (Tk, Hkv, d), bf16)
    v = _normals(seed, 2, (Tk, Hkv, d), bf16)
    peaks = None
    if peaked_rows:
        peaks = _peak_rows(lens[0], peaked_rows, peak_seed)
        _scale_rows(k, peaks, peak_scale, bf16)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return dict(q=q, k=k, v=v, cu_q=cu_q, cu_k=cu_k, lens=lens, q_lens=q_lens, peaks=peaks,
                dtype=dtype, Hq=Hq, Hkv=Hkv, d=d)


def decode_inputs(B, S, Hq, Hkv, d, dtype, seed, seq_L=None):
    """q [B, Hq, d], caches [B, S, Hkv, d] (streams 0, 1, 2 of ``seed``) and seq_L."""
    bf16 = dtype == "bf16"
    q = _normals(seed, 0, (B, Hq, d), bf16)
    k = _normals(seed, 1, (B, S, Hkv, d), bf16)
    v = _normals(seed, 2, (B, S, Hkv, d), bf16)
    if seq_L is None:
        seq_L = [S] * B
    return dict(q=q, k=k, v=v, seq_L=np.asarray(seq_L, dtype=np.int32), dtype=dtype,
                Hq=Hq, Hkv=Hkv, d=d)


def workload_inputs(name: str):
    w = WORKLOADS[name]
    if w["kind"] == "decode":
        return decode_inputs(w["B"], w["L"], w["Hq"], w["Hkv"], w["d"], w["dtype"], w["seed"])
    return prefill_inputs(w["lens"], w["Hq"], w["Hkv"], w["d"], w["dtype"], w["seed"],
                          w.get("peaked_rows", 0), w.get("peak_seed", 0), w.get("peak_scale", 1.0))


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of a generated array (bf16 bits or float32)."""
    return (bits_to_f32(a) if dtype == "bf16" else a).astype(np.float64)


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Uploads a generated array as a torch tensor (bfloat16 or float32)."""
    import torch
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def sample_rows(L: int, w0: int, w_pretrained: int, seed: int, n_edge: int = 64, n_rand: int = 256):
    """Stratified query rows of one sequence: first rows, rows around w0,
    around every multiple of w_pretrained, the last rows and seeded random
    rows."""
    rows = set(range(min(L, n_edge)))
    for c in [w0] + list(range(w_pretrained, L, w_pretrained)):
        rows.update(range(max(0, c - n_edge // 2), min(L, c + n_edge // 2)))
    rows.update(range(max(0, L - n_edge), L))
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, L, size=n_rand).tolist())
    return np.array(sorted(rows), dtype=np.int64)
