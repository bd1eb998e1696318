"""The slice generators of workloads.py (used by the benchmark's CPU
baseline workers) give exactly the elements of the full arrays."""
import numpy as np

from zero_shot_rope_bifocal_amd import workloads as W


def test_slices_equal_full_arrays(monkeypatch):
    wl = dict(W.WORKLOADS)
    wl["t_pre"] = dict(kind="prefill", dtype="bf16", lens=[3000], Hq=8, Hkv=2, d=128, w_pretrained=512, w0=64,
                       theta=1e4, seed=9, peaked_rows=5, peak_seed=3, peak_scale=4.0)
    wl["t_dec"] = dict(kind="decode", dtype="bf16", B=3, L=5000, Hq=8, Hkv=2, d=128, w_pretrained=512, w0=64,
                       theta=1e4, seed=10)
    monkeypatch.setattr(W, "WORKLOADS", wl)
    full = W.workload_inputs("t_pre")
    k, v = W.prefill_kv("t_pre")
    assert np.array_equal(k, full["k"]) and np.array_equal(v, full["v"])
    assert np.array_equal(W.prefill_q_rows("t_pre", 1000, 77), full["q"][1000:1077])
    assert np.array_equal(W.prefill_q_rows("t_pre", 0, 3000), full["q"])
    d = W.workload_inputs("t_dec")
    for b in range(3):
        q, k, v = W.decode_sequence("t_dec", b)
        assert np.array_equal(q[0], d["q"][b]) and np.array_equal(k[0], d["k"][b]) and np.array_equal(v[0], d["v"][b])


def test_normals_range_crosses_chunks():
    n = (1 << 22) + 1000
    full = W._normals(11, 1, (n,), False)
    a = (1 << 22) - 500
    assert np.array_equal(W.normals_range(11, 1, a, 1200, False), full[a:a + 1200])
