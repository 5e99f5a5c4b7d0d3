"""The seeded generators produce the workloads' shapes and statistics."""

import numpy as np

import synth
from synth import WORKLOADS


def f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -1.5, 1 + 2.0 ** -8 + 2.0 ** -20], np.float32)
    assert synth.f32_to_bf16_bits(v).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xBFC0, 0x3F81]


def test_rows_regenerate_independently():
    wl = WORKLOADS["prefill_oproj"]
    rows = np.array([0, 17, 4095, 8190])
    a = synth.activation_rows(wl, rows)
    b = synth.activation_rows(wl, np.array([17]))
    assert np.array_equal(a[1], b[0])
    assert a.shape == (4, wl.K)


def test_outliers_and_zero_tokens():
    wl = WORKLOADS["prefill_oproj"]
    assert wl.n_outliers == 72 and wl.n_zero_tokens == 8
    z = wl.zero_tokens()
    assert len(np.unique(z)) == 8 and z.max() < wl.M
    x = f32(synth.activation_rows(wl, np.concatenate([z, np.arange(64)])))
    assert np.all(x[:8] == 0) and not np.any(np.signbit(x[:8]))
    body = x[8:][~np.isin(np.arange(64), z)]
    ch = wl.outlier_channels()
    other = np.setdiff1d(np.arange(wl.K), ch)
    assert abs(body[:, other].std() - 1.0) < 0.01
    assert abs(body[:, ch].std() / 20.0 - 1.0) < 0.05


def test_segment_sigmas_and_weight_sigma():
    wl = WORKLOADS["fusion_fc"]
    x = f32(synth.activation_rows(wl, np.arange(64)))
    for i, sig in enumerate((1.0, 2.0, 4.0)):
        seg = x[:, i * 7168:(i + 1) * 7168]
        assert abs(seg.std() / sig - 1.0) < 0.01
        assert abs(seg.mean()) < 0.01 * sig
    w = f32(synth.bf16_normal(256, wl.K, wl.w_sigma, wl.seed, wl.w_tid))
    assert abs(w.std() / 0.01 - 1.0) < 0.01


def test_workload_shapes_and_algorithmic_work():
    c = WORKLOADS["decode_qkv"]
    assert (c.M, c.K, c.N) == (1, 7168, 9216)
    assert c.gemm_bytes() == 66_102_240
    assert WORKLOADS["spec_mlp_gu"].gemm_bytes() == 117_790_464
    assert WORKLOADS["spec_mlp_down"].gemm_bytes() == 58_916_864
    assert WORKLOADS["prefill_oproj"].gemm_flops() == 2 * 8191 * 7168 * 7168
    assert WORKLOADS["tiny"].gemm_bytes() == 201_840


def test_w4a16_weights_bytes_and_scale():
    wl = synth.W4A16_WORKLOADS["w4a16_decode_down"]
    small = synth.W4A16Workload("probe", 1, wl.K, 64)
    p, s, g = synth.w4a16_weight(small)
    assert p.shape == (64, wl.K // 2) and s.shape == (64, wl.K // 16) and g.dtype == np.float32
    assert s.min() == 0x60 and s.max() == 0x77
    counts = np.bincount(np.concatenate([p & 15, p >> 4]).ravel(), minlength=16)
    assert counts.min() > 0.9 * counts.mean()
    # rows regenerate independently of the tensor's size
    p2, s2, _ = synth.w4a16_weight(synth.W4A16Workload("probe", 1, wl.K, 8))
    assert np.array_equal(p2, p[:8]) and np.array_equal(s2, s[:8])
    import oracle
    assert abs(oracle.dequant_nvfp4(p, s, g).std() / 0.02 - 1.0) < 0.05


def test_w4a16_workload_shapes():
    W = synth.W4A16_WORKLOADS
    assert (W["w4a16_decode_qkv"].M, W["w4a16_decode_qkv"].K, W["w4a16_decode_qkv"].N) == (1, 7168, 9216)
    assert W["w4a16_decode_qkv"].gemm_bytes() == 9216 * 3584 + 9216 * 448 + 2 * 7168 + 2 * 9216
    assert W["w4a16_prefill_chunk"].gemm_flops() == 2 * 2048 * 7168 * 7168
    x = synth.w4a16_activation_rows(W["w4a16_decode_qkv"], np.arange(4))
    assert x.shape == (4, 7168) and x.dtype == np.uint16
