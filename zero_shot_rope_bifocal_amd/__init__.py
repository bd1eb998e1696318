"""MI355X (gfx950) dynamic bifocal RoPE attention.

Thin Python binding over ``libjetlong.so`` (C ABI in ``include/jetlong.h``).
It only marshals arguments: every step of the computation runs in the HIP
kernels.  PyTorch supplies device memory and the current stream.  There is no
fallback: if the library is missing every call raises.

Method: "Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal
RoPE" (gist.science summaries of arXiv 2607.07740), section "Dynamic Bifocal
RoPE" (eq. G, eq. f) and section "Inference Efficiency Mechanisms".
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "JL_F32", "JL_BF16", "JL_FLAG_PREROTATED", "JetLongError", "library_path", "lib",
    "group_size", "prefill", "prefill_prepare", "prefill_attend", "prefill_ie", "decode", "prefill_workspace_size",
    "prefill_ie_workspace_size", "decode_workspace_size",
    "remote_positions", "tile_classes", "prefill_tile_shape", "version",
    "rope_table", "rope_table_size", "decode_with_table", "decode_with_table_workspace_size", "decode_key_rows",
]

JL_F32, JL_BF16 = 0, 1
JL_FLAG_PREROTATED = 1
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class JetLongError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"jetlong status {code}: {msg}")
        self.code = code


def library_path() -> str:
    return os.environ.get("JETLONG_LIB", os.path.join(_HERE, "libjetlong.so"))


def lib() -> ctypes.CDLL:
    """Loads libjetlong.so (built by ``zero_shot_rope_bifocal_amd.build``)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m zero_shot_rope_bifocal_amd.build`")
    L = ctypes.CDLL(path)
    c_int, c_i64, c_sz, c_vp, c_d, c_f = (ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                                         ctypes.c_void_p, ctypes.c_double, ctypes.c_float)
    L.jl_bifocal_group_size.argtypes = [c_i64, c_i64]
    L.jl_bifocal_group_size.restype = c_i64
    L.jl_bifocal_prefill_workspace_size.argtypes = [c_int] * 7
    L.jl_bifocal_prefill_workspace_size.restype = c_sz
    L.jl_bifocal_prefill.argtypes = ([c_vp] * 5 + [c_int] + [c_vp] * 2 + [c_int] * 10 +
                                     [c_d, c_f, c_vp, c_sz, c_vp])
    L.jl_bifocal_prefill.restype = c_int
    L.jl_bifocal_prefill_prepare.argtypes = [c_vp, c_vp, c_int, c_vp] + [c_int] * 6 + [c_d, c_vp, c_sz, c_vp]
    L.jl_bifocal_prefill_prepare.restype = c_int
    L.jl_bifocal_prefill_attend.argtypes = L.jl_bifocal_prefill.argtypes
    L.jl_bifocal_prefill_attend.restype = c_int
    L.jl_bifocal_decode_workspace_size.argtypes = [c_int] * 6
    L.jl_bifocal_decode_workspace_size.restype = c_sz
    L.jl_bifocal_decode.argtypes = ([c_vp] * 3 + [c_i64] * 3 + [c_vp, c_vp, c_int, c_vp] +
                                    [c_int] * 7 + [c_d, c_f, c_vp, c_sz, c_vp])
    L.jl_bifocal_decode.restype = c_int
    c_u = ctypes.c_uint
    L.jl_bifocal_prefill_ex.argtypes = L.jl_bifocal_prefill.argtypes + [c_u]
    L.jl_bifocal_prefill_ex.restype = c_int
    L.jl_bifocal_prefill_prepare_ex.argtypes = L.jl_bifocal_prefill_prepare.argtypes + [c_u]
    L.jl_bifocal_prefill_prepare_ex.restype = c_int
    L.jl_bifocal_prefill_attend_ex.argtypes = L.jl_bifocal_prefill_attend.argtypes + [c_u]
    L.jl_bifocal_prefill_attend_ex.restype = c_int
    L.jl_bifocal_decode_ex.argtypes = L.jl_bifocal_decode.argtypes + [c_u]
    L.jl_bifocal_decode_ex.restype = c_int
    L.jl_bifocal_prefill_ie_workspace_size.argtypes = [c_int] * 8
    L.jl_bifocal_prefill_ie_workspace_size.restype = c_sz
    L.jl_bifocal_prefill_ie.argtypes = L.jl_bifocal_prefill_ex.argtypes
    L.jl_bifocal_prefill_ie.restype = c_int
    L.jl_bifocal_rope_table_size.argtypes = [c_int, c_int]
    L.jl_bifocal_rope_table_size.restype = c_sz
    L.jl_bifocal_rope_table.argtypes = [c_int, c_int, c_d, c_vp, c_sz, c_vp]
    L.jl_bifocal_rope_table.restype = c_int
    L.jl_bifocal_decode_with_table_workspace_size.argtypes = [c_int] * 6
    L.jl_bifocal_decode_with_table_workspace_size.restype = c_sz
    L.jl_bifocal_decode_with_table.argtypes = ([c_vp] * 3 + [c_i64] * 3 + [c_vp, c_vp, c_int, c_vp] +
                                               [c_int] * 7 + [c_f, c_vp, c_sz, c_int, c_vp, c_sz, c_vp, c_u])
    L.jl_bifocal_decode_with_table.restype = c_int
    L.jl_bifocal_decode_with_table_noalloc.argtypes = ([c_vp] * 3 + [c_i64] * 3 + [c_vp, c_vp, c_int, c_vp] +
                                                       [c_int] * 7 + [c_f, c_vp, c_sz, c_int, c_vp, c_u])
    L.jl_bifocal_decode_with_table_noalloc.restype = c_int
    L.jl_bifocal_decode_key_rows.argtypes = [c_vp] + [c_int] * 5 + [c_u, c_vp, c_vp]
    L.jl_bifocal_decode_key_rows.restype = c_int
    L.jl_bifocal_remote_positions.argtypes = [c_vp, c_vp, c_int, c_int, c_int, c_vp, c_vp, c_vp, c_vp]
    L.jl_bifocal_remote_positions.restype = c_int
    L.jl_bifocal_tile_classes.argtypes = [c_int] * 5 + [c_vp, c_vp]
    L.jl_bifocal_tile_classes.restype = c_int
    L.jl_bifocal_prefill_tile_shape.argtypes = [c_int] * 4 + [ctypes.POINTER(c_int)] * 2
    L.jl_bifocal_prefill_tile_shape.restype = c_int
    L.jl_status_string.argtypes = [c_int]
    L.jl_status_string.restype = ctypes.c_char_p
    L.jl_last_error.argtypes = []
    L.jl_last_error.restype = ctypes.c_char_p
    L.jl_version.argtypes = []
    L.jl_version.restype = ctypes.c_char_p
    _LIB = L
    return L


def _check(code: int):
    if code != 0:
        L = lib()
        raise JetLongError(code, f"{L.jl_status_string(code).decode()}: {L.jl_last_error().decode()}")


def version() -> str:
    return lib().jl_version().decode()


def group_size(L: int, w_pretrained: int) -> int:
    g = lib().jl_bifocal_group_size(int(L), int(w_pretrained))
    if g < 0:
        _check(int(g))
    return int(g)


# ---------------------------------------------------------------- torch glue

def _torch():
    import torch  # noqa: WPS433  (plumbing only: memory and streams)
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return JL_BF16
    if t.dtype == torch.float32:
        return JL_F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


def prefill_workspace_size(dtype: int, B: int, total_k: int, max_seqlen_k: int, Hq: int, Hkv: int,
                           head_dim: int) -> int:
    return int(lib().jl_bifocal_prefill_workspace_size(dtype, B, total_k, max_seqlen_k, Hq, Hkv, head_dim))


def prefill_ie_workspace_size(dtype: int, B: int, total_q: int, total_k: int, max_seqlen_k: int, Hq: int,
                              Hkv: int, head_dim: int) -> int:
    return int(lib().jl_bifocal_prefill_ie_workspace_size(dtype, B, total_q, total_k, max_seqlen_k, Hq, Hkv,
                                                          head_dim))


def decode_workspace_size(dtype: int, B: int, max_L: int, Hq: int, Hkv: int, head_dim: int) -> int:
    return int(lib().jl_bifocal_decode_workspace_size(dtype, B, max_L, Hq, Hkv, head_dim))


def prefill(q, k, v, cu_seqlens_q, max_seqlen_q: int, w_pretrained: int, w0: int, rope_theta: float,
            cu_seqlens_k=None, max_seqlen_k: int | None = None, softmax_scale: float = 0.0,
            out=None, lse=None, workspace=None, return_lse: bool = False, prerotated: bool = False):
    """Packed varlen bifocal prefill.  q [Tq, Hq, d], k/v [Tk, Hkv, d] (cuda,
    float32 or bfloat16, contiguous); cu_seqlens int32 cuda [B+1].  Queries of
    sequence b sit at its last Lq_b positions.  prerotated: q and k hold
    R(p) q, R(p) k (a RoPE cache).  Returns out (and lse [Hq, Tq] float32 when
    asked)."""
    return _prefill(False, q, k, v, cu_seqlens_q, max_seqlen_q, w_pretrained, w0, rope_theta, cu_seqlens_k,
                    max_seqlen_k, softmax_scale, out, lse, workspace, return_lse, prerotated)


def prefill_ie(q, k, v, cu_seqlens_q, max_seqlen_q: int, w_pretrained: int, w0: int, rope_theta: float,
               cu_seqlens_k=None, max_seqlen_k: int | None = None, softmax_scale: float = 0.0,
               out=None, lse=None, workspace=None, return_lse: bool = False, prerotated: bool = False):
    """``prefill`` computed by the inclusion-exclusion merge of three attention
    passes (a comparison route; same arguments and result)."""
    return _prefill(True, q, k, v, cu_seqlens_q, max_seqlen_q, w_pretrained, w0, rope_theta, cu_seqlens_k,
                    max_seqlen_k, softmax_scale, out, lse, workspace, return_lse, prerotated)


def _prefill(ie, q, k, v, cu_seqlens_q, max_seqlen_q, w_pretrained, w0, rope_theta, cu_seqlens_k, max_seqlen_k,
             softmax_scale, out, lse, workspace, return_lse, prerotated):
    torch = _torch()
    _need_cuda(q, k, v, cu_seqlens_q, cu_seqlens_k)
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    if cu_seqlens_q.dtype != torch.int32 or (cu_seqlens_k is not None and cu_seqlens_k.dtype != torch.int32):
        raise TypeError("cu_seqlens must be int32")
    dt = _dtype_code(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    B = cu_seqlens_q.numel() - 1
    if max_seqlen_k is None:
        if cu_seqlens_k is not None:
            raise ValueError("max_seqlen_k is required with cu_seqlens_k")
        max_seqlen_k = max_seqlen_q
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    need = (prefill_ie_workspace_size(dt, B, Tq, Tk, max_seqlen_k, Hq, Hkv, d) if ie
            else prefill_workspace_size(dt, B, Tk, max_seqlen_k, Hq, Hkv, d))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    entry = lib().jl_bifocal_prefill_ie if ie else lib().jl_bifocal_prefill_ex
    code = entry(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), dt, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        B, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, d, int(w_pretrained), int(w0),
        float(rope_theta), float(softmax_scale), _ptr(workspace), workspace.numel(), _stream(q.device),
        JL_FLAG_PREROTATED if prerotated else 0)
    _check(code)
    return (out, lse) if return_lse else out


def prefill_prepare(k, v, cu_seqlens_k, max_seqlen_k: int, w_pretrained: int, rope_theta: float,
                    Hq: int | None = None, workspace=None, prerotated: bool = False):
    """First stage of ``prefill``: fills and returns a workspace holding the
    cos/sin table and (bf16) the rotated keys and transposed values."""
    torch = _torch()
    _need_cuda(k, v, cu_seqlens_k)
    if cu_seqlens_k.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    dt = _dtype_code(k)
    Tk, Hkv, d = k.shape
    B = cu_seqlens_k.numel() - 1
    need = prefill_workspace_size(dt, B, Tk, max_seqlen_k, Hq or Hkv, Hkv, d)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=k.device)
    _check(lib().jl_bifocal_prefill_prepare_ex(_ptr(k), _ptr(v), dt, _ptr(cu_seqlens_k), B, Tk, int(max_seqlen_k),
                                               Hkv, d, int(w_pretrained), float(rope_theta), _ptr(workspace),
                                               workspace.numel(), _stream(k.device),
                                               JL_FLAG_PREROTATED if prerotated else 0))
    return workspace


def prefill_attend(q, k, v, cu_seqlens_q, max_seqlen_q: int, w_pretrained: int, w0: int,
                   rope_theta: float, workspace, cu_seqlens_k=None, max_seqlen_k: int | None = None,
                   softmax_scale: float = 0.0, out=None, lse=None, return_lse: bool = False,
                   prerotated: bool = False):
    """Second stage of ``prefill`` over a workspace from ``prefill_prepare``
    made with the same keys, values, key-side arguments and ``prerotated``."""
    torch = _torch()
    _need_cuda(q, k, v, cu_seqlens_q, cu_seqlens_k, workspace)
    dt = _dtype_code(q)
    Tq, Hq, d = q.shape
    Tk, Hkv, _ = k.shape
    B = cu_seqlens_q.numel() - 1
    if max_seqlen_k is None:
        max_seqlen_k = max_seqlen_q
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((Hq, Tq), dtype=torch.float32, device=q.device)
    _check(lib().jl_bifocal_prefill_attend_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), dt, _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        B, Tq, Tk, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, d, int(w_pretrained), int(w0),
        float(rope_theta), float(softmax_scale), _ptr(workspace), workspace.numel(), _stream(q.device),
        JL_FLAG_PREROTATED if prerotated else 0))
    return (out, lse) if return_lse else out


def decode(q, k_cache, v_cache, seq_L, w_pretrained: int, w0: int, rope_theta: float,
           max_L: int | None = None, softmax_scale: float = 0.0, out=None, lse=None, workspace=None,
           return_lse: bool = False, prerotated: bool = False):
    """One query per sequence against an untouched cache.  q [B, Hq, d];
    caches [B, S_max, Hkv, d] with d contiguous (any strides on the other
    axes, same for both); seq_L int32 cuda [B] counts the new token.
    prerotated: q and the key cache hold vectors rotated at their positions."""
    torch = _torch()
    _need_cuda(q, k_cache, v_cache, seq_L)
    if seq_L.dtype != torch.int32:
        raise TypeError("seq_L must be int32")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if k_cache.stride(3) != 1 or not q.is_contiguous():
        raise ValueError("head_dim must be contiguous")
    dt = _dtype_code(q)
    B, Hq, d = q.shape
    _, S, Hkv, _ = k_cache.shape
    if max_L is None:
        max_L = S
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = decode_workspace_size(dt, B, max_L, Hq, Hkv, d)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    sb, ss, sh, _ = k_cache.stride()
    code = lib().jl_bifocal_decode_ex(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), sb, ss, sh, _ptr(out), _ptr(lse), dt, _ptr(seq_L),
        B, int(max_L), Hq, Hkv, d, int(w_pretrained), int(w0), float(rope_theta),
        float(softmax_scale), _ptr(workspace), workspace.numel(), _stream(q.device),
        JL_FLAG_PREROTATED if prerotated else 0)
    _check(code)
    return (out, lse) if return_lse else out


def rope_table_size(max_pos: int, head_dim: int) -> int:
    return int(lib().jl_bifocal_rope_table_size(int(max_pos), int(head_dim)))


def rope_table(max_pos: int, head_dim: int, rope_theta: float, device="cuda", table=None):
    """Prepared cos/sin table of positions 0 .. max_pos-1 (uint8 cuda tensor)
    for ``decode_with_table``; build once, reuse for every decode step."""
    torch = _torch()
    need = rope_table_size(max_pos, head_dim)
    if table is None or table.numel() < need:
        table = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _check(lib().jl_bifocal_rope_table(int(max_pos), int(head_dim), float(rope_theta), _ptr(table), table.numel(),
                                       _stream(table.device)))
    return table


def decode_with_table_workspace_size(dtype: int, B: int, max_L: int, Hq: int, Hkv: int, head_dim: int) -> int:
    return int(lib().jl_bifocal_decode_with_table_workspace_size(dtype, B, max_L, Hq, Hkv, head_dim))


def decode_with_table(q, k_cache, v_cache, seq_L, w_pretrained: int, w0: int, table, table_rows: int,
                      max_L: int | None = None, softmax_scale: float = 0.0, out=None, lse=None, workspace=None,
                      return_lse: bool = False, prerotated: bool = False):
    """``decode`` reading a prepared cos/sin table (``rope_table``) that covers
    ``table_rows`` >= max_L positions and was built with the wanted theta."""
    torch = _torch()
    _need_cuda(q, k_cache, v_cache, seq_L, table)
    if seq_L.dtype != torch.int32:
        raise TypeError("seq_L must be int32")
    if k_cache.stride() != v_cache.stride() or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must share shape and strides")
    if k_cache.stride(3) != 1 or not q.is_contiguous():
        raise ValueError("head_dim must be contiguous")
    dt = _dtype_code(q)
    B, Hq, d = q.shape
    _, S, Hkv, _ = k_cache.shape
    if max_L is None:
        max_L = S
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = decode_with_table_workspace_size(dt, B, max_L, Hq, Hkv, d)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    sb, ss, sh, _ = k_cache.stride()
    _check(lib().jl_bifocal_decode_with_table(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), sb, ss, sh, _ptr(out), _ptr(lse), dt, _ptr(seq_L),
        B, int(max_L), Hq, Hkv, d, int(w_pretrained), int(w0), float(softmax_scale), _ptr(table), table.numel(),
        int(table_rows), _ptr(workspace), workspace.numel(), _stream(q.device),
        JL_FLAG_PREROTATED if prerotated else 0))
    return (out, lse) if return_lse else out


def decode_key_rows(seq_L, max_L: int, Hkv: int, w_pretrained: int, w0: int, prerotated: bool = False):
    """int32 cuda [B, max_L]: the signed cos/sin row the bf16 decode kernel
    rotates each key with (~r for row r with sin negated); entries past
    seq_L[b] are -2**31 (not written by the library)."""
    torch = _torch()
    _need_cuda(seq_L)
    B = seq_L.numel()
    out = torch.full((max(B, 1), max(int(max_L), 1)), -2 ** 31, dtype=torch.int32, device=seq_L.device)
    _check(lib().jl_bifocal_decode_key_rows(_ptr(seq_L), B, int(max_L), int(Hkv), int(w_pretrained), int(w0),
                                            JL_FLAG_PREROTATED if prerotated else 0, _ptr(out),
                                            _stream(seq_L.device)))
    return out[:B, :max_L]


def remote_positions(cu_seqlens_q, w_pretrained: int, cu_seqlens_k=None):
    """(pos [Tq], f [Tq], G [B]) int32 cuda tensors from the device kernel."""
    torch = _torch()
    _need_cuda(cu_seqlens_q, cu_seqlens_k)
    B = cu_seqlens_q.numel() - 1
    Tq = int(cu_seqlens_q[-1].item())
    dev = cu_seqlens_q.device
    pos = torch.empty(max(Tq, 1), dtype=torch.int32, device=dev)
    f = torch.empty(max(Tq, 1), dtype=torch.int32, device=dev)
    G = torch.empty(max(B, 1), dtype=torch.int32, device=dev)
    _check(lib().jl_bifocal_remote_positions(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Tq,
                                             int(w_pretrained), _ptr(pos), _ptr(f), _ptr(G), _stream(dev)))
    return pos[:Tq], f[:Tq], G[:B]


def tile_classes(Lq: int, L: int, w0: int, BM: int, BN: int, device="cuda"):
    """uint8 [ceil(Lq/BM), ceil(L/BN)] tile map from the device classifier."""
    torch = _torch()
    nqb, nkb = -(-Lq // BM), -(-L // BN)
    out = torch.empty(max(nqb * nkb, 1), dtype=torch.uint8, device=device)
    _check(lib().jl_bifocal_tile_classes(int(Lq), int(L), int(w0), int(BM), int(BN), _ptr(out),
                                         _stream(out.device)))
    return out[: nqb * nkb].view(nqb, nkb)


def prefill_tile_shape(dtype: int, Hq: int, Hkv: int, head_dim: int):
    bm, bn = ctypes.c_int(), ctypes.c_int()
    _check(lib().jl_bifocal_prefill_tile_shape(dtype, Hq, Hkv, head_dim, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value
