"""Host-side checks of the seeded synthetic workloads (no GPU, no oracle)."""

import numpy as np

import workloads as wl


def test_varlen_lengths_and_offsets():
    w = wl.CFG[4]
    assert w.lengths().tolist() == [12182, 15510, 14563, 8878, 15470, 16020, 15928, 2265]
    cu = w.cu_seqlens()
    assert cu[0] == 0 and cu[-1] == 100816 and cu.dtype == np.int32
    assert w.visible_pairs_per_head() == 717377301


def test_decode_lengths():
    L = wl.CFG[5].lengths()
    assert L.sum() == 1151702 and L.min() == 4125 and L.max() == 32745 and len(L) == 64


def test_algorithmic_work():
    assert abs(wl.CFG[1].flops() - 4 * 64 * 16 * (512 * 513 // 2)) < 1
    assert abs(wl.CFG[2].flops() - 68.72e9) < 0.01e9
    assert abs(wl.CFG[3].flops() - 549.8e9) < 0.1e9
    assert abs(wl.CFG[4].flops() - 4 * 128 * 32 * 717377301) < 1
    assert wl.CFG[5].bytes_moved() == 18869485568 + 1048576 + 8192


def test_draws_are_deterministic_and_chunked():
    a = wl.normal_f32(7, 1, wl.CHUNK + 1000)
    b = wl.normal_f32(7, 1, wl.CHUNK + 1000)
    np.testing.assert_array_equal(a, b)
    c = wl.normal_f32(7, 2, 1000)
    assert not np.array_equal(a[:1000], c)
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01


def test_dtype_rounding_and_scale():
    import torch
    w = wl.SMALL[4]
    q, k, v, cu = wl.varlen_inputs(w)
    assert q.dtype == torch.float16 and q.shape == (int(cu[-1]), w.H, w.D)
    x = wl.normal_f32(w.seed, 0, q.numel()) * np.float32(0.5)
    np.testing.assert_array_equal(q.reshape(-1).numpy(), torch.from_numpy(x).to(torch.float16).numpy())
    q2, k2, v2 = wl.prefill_inputs(wl.SMALL[3])
    assert q2.dtype == torch.bfloat16 and q2.shape == (2, 1000, 4, 64)
