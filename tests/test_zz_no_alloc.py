"""jl_bifocal_decode_with_table_noalloc (no workspace, partial states in the
library's device scratch) against jl_bifocal_decode_with_table, through the C
ABI: two calls in a row on one stream, the second with a smaller batch and
cache (the scratch keeps the first call's contents), each compared bit for bit
with the entry point it varies and with the oracle within the bf16 / fp32
tolerance; sizes beyond the scratch are rejected before anything runs."""
import ctypes

import numpy as np
import pytest

import oracle
import zero_shot_rope_bifocal_amd as jl
from zero_shot_rope_bifocal_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _noalloc(q, k, v, seq, wp, w0, table, rows, out, lse, flags=0):
    import torch
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    B, Hq, d = q.shape
    _, S, Hkv, _ = k.shape
    sb, ss, sh, _ = k.stride()
    dt = jl.JL_BF16 if q.dtype == torch.bfloat16 else jl.JL_F32
    return jl.lib().jl_bifocal_decode_with_table_noalloc(
        vp(q), vp(k), vp(v), sb, ss, sh, vp(out), vp(lse), dt, vp(seq), B, S, Hq, Hkv, d, wp, w0, 0.0, vp(table),
        table.numel(), rows, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), flags)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_noalloc_decode_matches_decode_with_table(dt):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wp, theta = 512, 1e6
    table = jl.rope_table(6000, 128, theta)
    calls = [  # (B, S, seq_L, Hq, Hkv, w0, seed): the second call is smaller
        (16, 4000, [4000, 3999, 2500, 1] + [4000 - 37 * i for i in range(12)], 32, 8, 300, 91),
        (3, 1000, [1000, 517, 64], 16, 4, 100, 92),
    ]
    for B, S, seq_L, Hq, Hkv, w0, seed in calls:
        inp = W.decode_inputs(B, S, Hq, Hkv, 128, dt, seed, seq_L=seq_L)
        q, k, v = (W.to_device(inp[n], dt) for n in ("q", "k", "v"))
        seq = torch.from_numpy(inp["seq_L"]).cuda()
        ref, ref_lse = jl.decode_with_table(q, k, v, seq, wp, w0, table, 6000, return_lse=True)
        out = torch.full_like(q, 3.0)
        lse = torch.full((B, Hq), 3.0, dtype=torch.float32, device="cuda")
        rc = _noalloc(q, k, v, seq, wp, w0, table, 6000, out, lse)
        assert rc == 0, jl.lib().jl_last_error()
        torch.cuda.synchronize()
        print("[case] noalloc", dt, B, S, flush=True)
        if dt == "bf16":
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        else:
            assert torch.equal(out, ref)
        assert torch.equal(lse, ref_lse)
        o_ref, _ = oracle.bifocal_decode(W.as_f64(inp["q"], dt), W.as_f64(inp["k"], dt), W.as_f64(inp["v"], dt),
                                         inp["seq_L"], wp, w0, theta)
        assert np.max(np.abs(out.float().cpu().numpy() - o_ref)) <= TOL[dt]


def test_noalloc_rejects_sizes_beyond_the_scratch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = jl.lib()
    vp = ctypes.c_void_p
    # 4096 sequences x 64 heads over 128K keys: at least one partial state of
    # 130 floats per (sequence, head, wave) > 64 MiB
    need = jl.decode_with_table_workspace_size(jl.JL_BF16, 4096, 131072, 64, 8, 128)
    assert need > 64 << 20
    rc = L.jl_bifocal_decode_with_table_noalloc(vp(256), vp(256), vp(256), 131072 * 8 * 128, 8 * 128, 128, vp(256),
                                                None, jl.JL_BF16, vp(256), 4096, 131072, 64, 8, 128, 32768, 2048, 0.0,
                                                vp(256), 1 << 40, 131072, None, 0)
    assert rc == -2 and b"scratch" in L.jl_last_error()
