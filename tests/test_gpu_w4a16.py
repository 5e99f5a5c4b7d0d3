"""GPU parity: the HIP NVFP4 weight-only linear against the float64 oracle.

Every element must satisfy |y - ref| <= 4e-3 |ref| + 1e-3 rms(ref).  Cases whose
result is exactly representable (one-hot activations with g = 1 read back single
dequantized weights) are compared bit for bit."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as fb
import oracle
import synth
from tests.gpu_util import assert_bits_equal, banner, dev_bf16, dev_u8, host_u16

pytestmark = pytest.mark.gpu

# E4M3 codes without the two NaN patterns.
E4M3_FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)


def bf16(x):
    x = np.asarray(x, dtype=np.float32)
    return synth.f32_to_bf16_bits(x).reshape(x.shape)


def random_case(M, N, K, seed, scale_codes=None):
    rng = np.random.default_rng(seed)
    x = bf16(rng.standard_normal((M, K)))
    w4 = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    if scale_codes is None:
        bs = rng.integers(0x30, 0x78, size=(N, K // 16), dtype=np.uint8)
    else:
        bs = rng.choice(scale_codes, size=(N, K // 16)).astype(np.uint8)
    return x, w4, bs


def gpu(x, w4, bs, g, workspace=None):
    y = fb.nvfp4_linear(dev_bf16(x), dev_u8(w4), dev_u8(bs), g, workspace=workspace)
    torch.cuda.synchronize()
    return host_u16(y)


def no_workspace():
    return torch.empty(0, dtype=torch.uint8, device="cuda")


def check(x, w4, bs, g, what, workspace=None):
    banner(f"nvfp4_linear {what} M={x.shape[0]} N={w4.shape[0]} K={x.shape[1]}")
    y = gpu(x, w4, bs, g, workspace)
    res = oracle.check_tolerance(y, oracle.linear_w4a16_ref(x, w4, bs, g))
    assert res["ok"], f"{what}: {res}"
    return y


SHAPES = [(M, N, K) for M in (1, 2, 5, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 128, 129, 300)
          for (N, K) in ((128, 128), (384, 512), (1024, 1152))]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_shapes(M, N, K):
    x, w4, bs = random_case(M, N, K, seed=M * 131 + N + K)
    check(x, w4, bs, np.float32(3.7e-3), "random")


@pytest.mark.parametrize("M", [1, 16, 40, 200])
def test_every_scale_code(M):
    """Scales drawn from every finite E4M3 code: zero, subnormal, negative, 448."""
    x, w4, bs = random_case(M, 512, 1024, seed=900 + M, scale_codes=E4M3_FINITE)
    check(x, w4, bs, np.float32(0.75), "every scale code")


def test_dequantized_weights_bitwise():
    """x = identity (128 tokens x 128 channels), g = 1: y = W^T exactly, for every
    code in every group position and every finite scale code."""
    N, K = 512, 128
    rng = np.random.default_rng(77)
    w4 = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    bs = np.resize(E4M3_FINITE, N * (K // 16)).reshape(N, K // 16)
    x = bf16(np.eye(K, dtype=np.float32))
    banner("nvfp4_linear identity activations bitwise")
    y = gpu(x, w4, bs, np.float32(1.0))
    want = oracle.dequant_nvfp4(w4, bs, np.float32(1.0)).T                  # exact in BF16
    want_bits = bf16(want.astype(np.float32))
    got = y.copy()
    got[(got & 0x7FFF) == 0] = 0                                           # +-0 both fine
    want_bits[(want_bits & 0x7FFF) == 0] = 0
    assert_bits_equal(got, want_bits, "identity readback")


@pytest.mark.parametrize("k", [0, 1, 15, 16, 31, 32, 63, 64, 127, 128, 255])
def test_one_hot_decode_row(k):
    """M = 1 with x one-hot at column k reads back column k of W (decode path)."""
    N, K = 256, 256
    rng = np.random.default_rng(k)
    w4 = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    bs = rng.choice(E4M3_FINITE, size=(N, K // 16)).astype(np.uint8)
    x = np.zeros((1, K), np.float32)
    x[0, k] = 1.0
    banner(f"nvfp4_linear one-hot k={k}")
    y = gpu(bf16(x), w4, bs, np.float32(1.0))
    want = bf16(oracle.dequant_nvfp4(w4, bs, np.float32(1.0))[:, k].astype(np.float32))[None, :]
    y[(y & 0x7FFF) == 0] = 0
    want[(want & 0x7FFF) == 0] = 0
    assert_bits_equal(y, want, f"one-hot column {k}")


DECODE_CASES = [
    # (M, K, N, env): token groups P = 4 / 8 / 16, whole and partial super blocks
    (1, 512, 384, None), (3, 2048, 1024, None), (4, 16384, 512, None), (2, 7168, 2048, None),
    (5, 1152, 384, None), (8, 7168, 1024, None), (6, 4096, 2048, None), (7, 32768, 256, None),
    (12, 1024, 1024, None), (16, 2048, 384, None), (16, 640, 2048, None), (9, 8576, 1024, None),
    (1, 8576, 2048, None), (1, 896, 384, None),
    # the streaming kernel at decode sizes
    (1, 7168, 2048, {"FP8BS_W4_DECODE": "0"}), (5, 1152, 1024, {"FP8BS_W4_DECODE": "0"}),
    # strips per workgroup, super blocks per load batch, waves (uneven splits)
    (1, 7168, 2048, {"FP8BS_W4_DECODE_NS": "1", "FP8BS_W4_DECODE_CH": "1"}),
    (2, 2048, 1152, {"FP8BS_W4_DECODE_NS": "4"}), (7, 1280, 384, {"FP8BS_W4_DECODE_NS": "4"}),
    (3, 1024, 1024, {"FP8BS_W4_DECODE_NS": "1", "FP8BS_W4_DECODE_CH": "2"}),
    (16, 512, 1024, {"FP8BS_W4_DECODE_WAVES": "3"}), (1, 896, 384, {"FP8BS_W4_DECODE_WAVES": "2"}),
    (4, 7168, 1024, {"FP8BS_W4_DECODE_WAVES": "5", "FP8BS_W4_DECODE_CH": "2"}),
    # every strip count with both batch sizes, partial last workgroups (40 strips of 16 in 3s)
    (1, 7168, 2048, {"FP8BS_W4_DECODE_NS": "3", "FP8BS_W4_DECODE_CH": "1"}),
    (1, 7168, 2048, {"FP8BS_W4_DECODE_NS": "3", "FP8BS_W4_DECODE_CH": "2"}),
    (6, 4096, 1152, {"FP8BS_W4_DECODE_NS": "3", "FP8BS_W4_DECODE_CH": "2"}),
    (12, 1024, 640, {"FP8BS_W4_DECODE_NS": "3"}),
    (2, 2048, 1152, {"FP8BS_W4_DECODE_NS": "4", "FP8BS_W4_DECODE_CH": "2"}),
    (9, 8576, 1024, {"FP8BS_W4_DECODE_NS": "4", "FP8BS_W4_DECODE_CH": "2"}),
    (16, 2048, 384, {"FP8BS_W4_DECODE_NS": "2", "FP8BS_W4_DECODE_CH": "2"}),
    (5, 1152, 384, {"FP8BS_W4_DECODE_NS": "2", "FP8BS_W4_DECODE_CH": "1"}),
    # rows past the decode kernel's bound (lowered from 2^27 by the test hook) stream
    (1, 2048, 384, {"FP8BS_DECODE_MAX_K": "1024"}),
    (7, 1152, 640, {"FP8BS_DECODE_MAX_K": "1024"}),
]


@pytest.mark.parametrize("M,K,N,env", DECODE_CASES)
def test_decode_schedules(M, K, N, env, monkeypatch):
    """Every decode schedule (K chunks folded into the MFMA, or streamed) and strip
    counts with ragged tails give the oracle's result."""
    for k, v in (env or {}).items():
        monkeypatch.setenv(k, v)
    x, w4, bs = random_case(M, N, K, seed=M + K + N)
    check(x, w4, bs, np.float32(2.0e-3), f"schedule {env}")


@pytest.mark.parametrize("tile", ["256256", "128256", "128128", "64128"])
@pytest.mark.parametrize("M,N,K", [(65, 384, 512), (300, 1024, 1152), (513, 384, 2048), (1000, 640, 256)])
def test_tile_configs(tile, M, N, K, monkeypatch):
    """Every LDS tile shape, with M and N tails that are not tile multiples."""
    monkeypatch.setenv("FP8BS_W4_TILE", tile)
    x, w4, bs = random_case(M, N, K, seed=M + N + K + int(tile))
    check(x, w4, bs, np.float32(1.5e-3), f"tile {tile}", workspace=no_workspace())


@pytest.mark.parametrize("M,N,K,split", [(65, 1024, 1152, None), (128, 2048, 2048, None), (200, 1024, 7168, None),
                                         (300, 1152, 1024, None), (128, 1024, 7168, "2"), (100, 512, 3072, "3"),
                                         (129, 768, 4096, "8"), (80, 256, 256, "4")])
def test_split_k(M, N, K, split, monkeypatch):
    """Split-K over workgroups (FP32 partials in the workspace, fixed-order sum)."""
    if split:
        monkeypatch.setenv("FP8BS_W4_KSPLIT", split)
    assert fb.nvfp4_workspace_size(M, N, K) > 0 or split
    x, w4, bs = random_case(M, N, K, seed=3 * M + N + K)
    ws = torch.empty(8 * M * N * 4, dtype=torch.uint8, device="cuda")
    y = check(x, w4, bs, np.float32(2.5e-3), f"split-K {split}", workspace=ws)
    assert_bits_equal(gpu(x, w4, bs, np.float32(2.5e-3), ws), y, "split-K repeat")


@pytest.mark.parametrize("M", [17, 25, 32, 33, 48, 63, 64])
@pytest.mark.parametrize("N,K", [(1024, 1152), (384, 2048)])
def test_streaming_kernel_without_workspace(M, N, K):
    """16 < M <= 64 without a workspace runs the streaming kernel (2 or 4 token groups)."""
    x, w4, bs = random_case(M, N, K, seed=17 * M + N + K)
    check(x, w4, bs, np.float32(1.0e-3), "streaming", workspace=no_workspace())


@pytest.mark.parametrize("M,N,K,strips", [(20, 1024, 1152, "4"), (32, 384, 2048, "4"), (30, 1024, 1152, "2"),
                                          (17, 9216, 512, None), (32, 16384, 256, None), (25, 7168, 384, None),
                                          (40, 9216, 256, None), (64, 1024, 1152, "2")])
def test_streaming_strips(M, N, K, strips, monkeypatch):
    """The streaming kernel with 1, 2 or 4 strips per workgroup (forced, or the host's own
    choice on wide N); M <= 32 streams even with a workspace."""
    if strips:
        monkeypatch.setenv("FP8BS_W4_STRIPS", strips)
    x, w4, bs = random_case(M, N, K, seed=29 * M + N + K)
    y = check(x, w4, bs, np.float32(1.0e-3), f"streaming strips={strips}", workspace=no_workspace())
    if M <= 32:
        ws = torch.empty(8 * M * N * 4, dtype=torch.uint8, device="cuda")
        assert_bits_equal(gpu(x, w4, bs, np.float32(1.0e-3), ws), y, "with a workspace: the same schedule")


def _random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 65)), int(rng.integers(65, 1200))]))
        N = 128 * int(rng.integers(1, 40))
        K = 128 * int(rng.integers(1, 12))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_shapes(2025, 24))
def test_random_shapes(M, N, K):
    """Seeded random shapes across every schedule the host can pick (decode, streaming
    strips, split-K, each tile shape), with the binding's default workspace and without."""
    x, w4, bs = random_case(M, N, K, seed=M + 5 * N + 11 * K)
    ref = oracle.linear_w4a16_ref(x, w4, bs, np.float32(1e-3))
    for ws in (None, no_workspace()):
        banner(f"nvfp4_linear random shape M={M} N={N} K={K} workspace={'default' if ws is None else 'none'}")
        res = oracle.check_tolerance(gpu(x, w4, bs, np.float32(1e-3), ws), ref)
        assert res["ok"], res


def test_split_k_workspace_sizes():
    """A smaller workspace selects a smaller split (or none); every result is in
    tolerance and the size query's workspace is enough for the default split."""
    M, N, K = 128, 2048, 4096
    x, w4, bs = random_case(M, N, K, seed=11)
    ref = oracle.linear_w4a16_ref(x, w4, bs, np.float32(1e-2))
    need = fb.nvfp4_workspace_size(M, N, K)
    assert need > 0
    for nbytes in (need, need // 2, 2 * M * N * 4, M * N * 4, 0):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        banner(f"nvfp4_linear split-K workspace {nbytes}")
        res = oracle.check_tolerance(gpu(x, w4, bs, np.float32(1e-2), ws), ref)
        assert res["ok"], (nbytes, res)


def test_global_scale_sign_and_zero():
    x, w4, bs = random_case(24, 384, 512, seed=5)
    y1 = gpu(x, w4, bs, np.float32(0.5))
    yn = gpu(x, w4, bs, np.float32(-0.5))
    assert_bits_equal(yn ^ np.uint16(0x8000), y1, "negated global scale")
    y0 = gpu(x, w4, bs, np.float32(0.0))
    assert not np.any(y0 & 0x7FFF)


@pytest.mark.parametrize("M", [1, 8, 50, 300])
def test_deterministic(M):
    x, w4, bs = random_case(M, 1024, 2048, seed=M + 3)
    banner(f"nvfp4_linear repeat M={M}")
    assert_bits_equal(gpu(x, w4, bs, np.float32(1e-2)), gpu(x, w4, bs, np.float32(1e-2)), "repeat")


@pytest.mark.parametrize("M", [1, 8, 40, 300])
def test_graph_replay_matches_eager(M):
    """nvfp4_linear captured in a HIP graph (as the bench runs it) reproduces the eager
    output on every replay, with eager work in between: decode, streaming and tiled
    schedules."""
    x, w4, bs = random_case(M, 1024, 2048, seed=70 + M)
    xd, wd, bd = dev_bf16(x), dev_u8(w4), dev_u8(bs)
    y = torch.empty((M, 1024), dtype=torch.bfloat16, device="cuda")
    banner(f"nvfp4_linear graph replay M={M}")
    fb.nvfp4_linear(xd, wd, bd, 0.01, out=y)
    torch.cuda.synchronize()
    ref = y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fb.nvfp4_linear(xd, wd, bd, 0.01, out=y)
    for i in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), i
        fb.nvfp4_linear(xd, wd, bd, 0.5)       # eager work between replays
        torch.cuda.synchronize()


def test_empty_and_errors():
    e = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    w4 = torch.zeros((128, 128), dtype=torch.uint8, device="cuda")
    bs = torch.zeros((128, 16), dtype=torch.uint8, device="cuda")
    assert fb.nvfp4_linear(e, w4, bs, 1.0).shape == (0, 128)
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fb.Fp8bsError):
        fb.nvfp4_linear(x, w4, bs, float("nan"))


@pytest.mark.parametrize("name", sorted(synth.W4A16_WORKLOADS))
def test_workload(name):
    wl = synth.W4A16_WORKLOADS[name]
    w4, bs, g = synth.w4a16_weight(wl)
    x = synth.w4a16_activation_rows(wl, np.arange(wl.M))
    banner(f"nvfp4_linear workload {name} M={wl.M} N={wl.N} K={wl.K}")
    y = gpu(x, w4, bs, g)
    rows = synth.sample_rows(wl.M, wl.sampled_rows, wl.seed) if wl.sampled_rows else np.arange(wl.M)
    ref = oracle.linear_w4a16_ref(x[rows], w4, bs, g)
    res = oracle.check_tolerance(y[rows], ref)
    assert res["ok"], f"{name}: {res}"
