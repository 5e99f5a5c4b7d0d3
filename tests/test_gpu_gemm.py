"""GPU parity: the HIP block-scaled GEMM against the float64 oracle.

Every element must satisfy |y - ref| <= 4e-3 |ref| + 1e-3 rms(ref).  Special cases
whose result is exact are compared bit for bit."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as fb
import oracle
import synth
from tests.gpu_util import assert_bits_equal, banner, dev_bf16, dev_f32, dev_u8, host_u16

pytestmark = pytest.mark.gpu


def bf16(x):
    x = np.asarray(x, dtype=np.float32)
    return synth.f32_to_bf16_bits(x).reshape(x.shape)


def inputs(M, N, K, seed, x_sigma=1.0, w_sigma=0.02):
    """Seeded BF16 activations [M, K] and weights [N, K] (host bit patterns)."""
    rng = np.random.default_rng(seed)
    return bf16(rng.standard_normal((M, K)) * x_sigma), bf16(rng.standard_normal((N, K)) * w_sigma)


def gpu_path(x, w, workspace=None, ws_mult=None):
    """The HIP path end to end: quantize both operands on the GPU, then the GEMM."""
    q, s = fb.quant_act(dev_bf16(x))
    qw, ws = fb.quant_weight(dev_bf16(w))
    if ws_mult is not None:
        ws = ws * ws_mult
    y = fb.block_linear(q, s, qw, ws, workspace=workspace)
    torch.cuda.synchronize()
    return host_u16(y)


def oracle_path(x, w):
    q, s = oracle.quant_act(x)
    qw, ws = oracle.quant_weight(w)
    return oracle.linear_ref(q, s, qw, ws)


def check_linear(x, w, what, workspace=None):
    banner(f"block_linear {what} M={x.shape[0]} N={w.shape[0]} K={x.shape[1]}")
    y = gpu_path(x, w, workspace)
    res = oracle.check_tolerance(y, oracle_path(x, w))
    assert res["ok"], f"{what}: {res}"
    return y


SHAPES = [(M, N, K) for M in (1, 2, 5, 8, 9, 16, 17, 32, 33, 64, 65, 100, 128, 129, 255, 256, 257, 300, 513)
          for (N, K) in ((128, 128), (384, 512), (1024, 1152))]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_linear_shapes(M, N, K):
    x, w = inputs(M, N, K, seed=M * 31 + N + K)
    check_linear(x, w, "random")


@pytest.mark.parametrize("M", [1, 8, 16, 40, 200])
def test_linear_without_workspace(M):
    x, w = inputs(M, 1152, 2048, seed=M)
    check_linear(x, w, "no workspace", workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("M", [3, 8, 16, 64, 200])
def test_identity_weights_bitwise(M):
    """s = 1 (every group holds 448) and identity weights: y = dec(q) exactly."""
    rng = np.random.default_rng(M)
    x = bf16(rng.standard_normal((M, 128)) * 60.0)
    x[:, 5] = bf16(np.float32(448.0))
    qg, sg = fb.quant_act(dev_bf16(x))
    qw = np.zeros((128, 128), np.uint8)
    np.fill_diagonal(qw, 0x38)                       # E4M3 1.0 on the diagonal
    y = fb.block_linear(qg, sg, dev_u8(qw), dev_f32(np.ones((1, 1), np.float32)))
    torch.cuda.synchronize()
    y = host_u16(y)
    q, s = oracle.quant_act(x)
    assert np.all(s == 1.0)
    want = bf16(oracle.decode(q).astype(np.float32))
    zero = (want & 0x7FFF) == 0
    assert_bits_equal(np.where(zero, 0, y), np.where(zero, 0, want), "identity")
    assert np.all((y[zero] & 0x7FFF) == 0)


@pytest.mark.parametrize("M", [4, 16, 129])
def test_zero_tokens_exact_zero(M):
    x, w = inputs(M, 384, 512, seed=5)
    x[1] = 0
    y = gpu_path(x, w)
    assert np.all(y[1] == 0)                 # +0.0 exactly
    assert np.all(np.any(y[[0, 2]] != 0, axis=1))


@pytest.mark.parametrize("M", [1, 8, 100])
def test_negation_symmetry(M):
    x, w = inputs(M, 1024, 1152, seed=9)
    y = gpu_path(x, w).astype(np.uint32)
    yn = gpu_path(x ^ np.uint16(0x8000), w).astype(np.uint32)
    f = lambda b: (b << 16).view(np.float32)
    assert np.array_equal(f(yn), -f(y))


@pytest.mark.parametrize("M", [1, 8, 64])
def test_power_of_two_weight_scale_doubles_output(M):
    x, w = inputs(M, 384, 1152, seed=10)
    y = gpu_path(x, w)
    y2 = gpu_path(x, w, ws_mult=2.0)
    f = lambda b: (b.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(f(y2), 2 * f(y))


@pytest.mark.parametrize("M", [1, 8, 16, 300])
def test_deterministic(M):
    x, w = inputs(M, 2048, 3072, seed=11)
    args = (*fb.quant_act(dev_bf16(x)), *fb.quant_weight(dev_bf16(w)))
    ref = fb.block_linear(*args).clone()
    for _ in range(5):
        assert torch.equal(fb.block_linear(*args), ref)


def test_workspace_argument_is_accepted():
    """A caller-provided workspace (the ABI's optional scratch) changes nothing."""
    wsp = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    for i, (M, N, K) in enumerate(((1, 9216, 7168), (8, 7168, 8192), (3, 384, 512))):
        x, w = inputs(M, N, K, seed=40 + i)
        a = check_linear(x, w, f"with workspace {i}", workspace=wsp)
        b = gpu_path(x, w)
        assert np.array_equal(a, b)


@pytest.mark.parametrize("M,K", [(16, 12288), (9, 20480)])
def test_decode_activations_beyond_lds(M, K):
    """M x K codes too large to stage in LDS: B fragments are read from global memory."""
    x, w = inputs(M, 256, K, seed=70 + M)
    check_linear(x, w, "decode, activations from global")


@pytest.mark.parametrize("interleave", [0, 1])
@pytest.mark.parametrize("batch", [1, 2])
@pytest.mark.parametrize("strips", [1, 2, 3, 4])
@pytest.mark.parametrize("M,N", [(1, 640), (5, 384), (8, 1152), (12, 640)])
def test_decode_strips_per_workgroup(strips, batch, interleave, M, N, monkeypatch):
    """Every strips-per-workgroup setting and load batch (super blocks whose loads
    are issued together), with contiguous and interleaved super blocks per wave,
    including a partial last workgroup, a partial last super block (K = 1408: 11 K
    blocks) and a partial last batch."""
    monkeypatch.setenv("FP8BS_DECODE_STRIPS", str(strips))
    monkeypatch.setenv("FP8BS_DECODE_BATCH", str(batch))
    monkeypatch.setenv("FP8BS_DECODE_INTERLEAVE", str(interleave))
    x, w = inputs(M, N, 1408, seed=80 + strips + M)
    check_linear(x, w, f"decode strips={strips} batch={batch}")


@pytest.mark.parametrize("M,K", [(1, 1152), (5, 2048), (16, 1408), (3, 1024)])
def test_decode_rows_past_the_decode_bound(M, K, monkeypatch):
    """Rows longer than the decode kernel's bound (2^27, lowered to 1024 by the test
    hook) take the mid-size kernel, also for M <= 16; K = 1024 stays on the decode
    kernel."""
    monkeypatch.setenv("FP8BS_DECODE_MAX_K", "1024")
    x, w = inputs(M, 384, K, seed=660 + M + K)
    check_linear(x, w, f"decode bound K={K}")


@pytest.mark.parametrize("M", [1, 3, 6, 8, 13])
@pytest.mark.parametrize("K", [128, 256, 384, 640, 896])
def test_decode_short_k(M, K):
    """K shorter than a super block of the natural row group (the plan widens the group so
    that one super block fits) and a last, partial super block whose weight scales are
    loaded from K block KB - G."""
    x, w = inputs(M, 384, K, seed=100 + M + K)
    check_linear(x, w, f"decode short K={K}")


@pytest.mark.parametrize("interleave", [0, 1])
@pytest.mark.parametrize("waves", [1, 2, 3, 5, 7, 8])
def test_decode_split_counts(waves, interleave, monkeypatch):
    """Every split-K degree of the decode schedule meets the tolerance, with
    contiguous and interleaved super blocks per wave."""
    monkeypatch.setenv("FP8BS_DECODE_WAVES", str(waves))
    monkeypatch.setenv("FP8BS_DECODE_INTERLEAVE", str(interleave))
    x, w = inputs(5, 384, 2048, seed=50 + waves)
    check_linear(x, w, f"decode waves={waves}")


@pytest.mark.parametrize("tile", ["256256", "256128", "128256", "128128"])
@pytest.mark.parametrize("M", [129, 300])
def test_prefill_tile_shapes(tile, M, monkeypatch):
    """Every prefill tile shape, ragged M in the clamped (M < 256) and the moved-back
    last-tile forms."""
    monkeypatch.setenv("FP8BS_PREFILL_TILE", tile)
    x, w = inputs(M, 1024, 1152, seed=90 + M)
    # no workspace: the tile shape is not replaced by a split-K schedule
    check_linear(x, w, f"prefill tile {tile}", workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))


@pytest.mark.parametrize("tile", ["256256", "256128", "128256", "128128"])
@pytest.mark.parametrize("M,K", [(100, 128), (257, 256), (130, 384), (300, 640), (200, 896)])
def test_prefill_stage_ring(tile, M, K, monkeypatch):
    """The K loop's ring of LDS stages (2 to 4 per tile shape) with fewer K blocks than
    stages (the prologue repeats the last block) and with counts that wrap the ring."""
    monkeypatch.setenv("FP8BS_PREFILL_TILE", tile)
    x, w = inputs(M, 512, K, seed=7 * M + K)
    check_linear(x, w, f"prefill tile {tile} K={K}", workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))


def test_prefill_default_mid_tile():
    """M = 1024 on the 7168-wide projection: the default schedule picks 128 x 256 tiles."""
    x, w = inputs(1024, 7168, 1024, seed=97)
    assert fb.workspace_size(1024, 7168, 1024) == 0          # enough tiles: no split
    check_linear(x, w, "prefill 128x256 default")


@pytest.mark.parametrize("M", [17, 32, 40, 64])
@pytest.mark.parametrize("strips,waves", [("1", "8"), ("2", "8"), ("4", "8"), ("1", "3"), ("2", "5"), ("4", "6")])
def test_mid_schedules(M, strips, waves, monkeypatch):
    """The mid-size kernel (16 < M <= 64) under every strip count (4 only up to 32 rows;
    the hook leaves larger M on its own choice) and several in-workgroup split-K degrees."""
    monkeypatch.setenv("FP8BS_MID_STRIPS", strips)
    monkeypatch.setenv("FP8BS_MID_WAVES", waves)
    x, w = inputs(M, 1024, 2176, seed=70 + M)
    check_linear(x, w, f"mid strips={strips} waves={waves}",
                 workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))    # no split-K: the mid kernel


@pytest.mark.parametrize("M,N,K", [(20, 9216, 512), (32, 16384, 256), (30, 7168, 384), (48, 9216, 256),
                                   (25, 1024, 1024)])
def test_mid_default_plans(M, N, K):
    """The mid-size kernel's own strip choice (4 strips per workgroup on wide N up to 32
    rows, 2 on N = 7168, 1 on narrow N), with and without a workspace: M <= 32 stays on
    this kernel even when a workspace is given."""
    x, w = inputs(M, N, K, seed=3 * M + N)
    y = check_linear(x, w, "mid default plan", workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    ws = torch.empty(8 * M * N * 4, dtype=torch.uint8, device="cuda")
    if M <= 32:
        assert np.array_equal(gpu_path(x, w, workspace=ws), y)
    else:
        check_linear(x, w, "mid-size M with a workspace", workspace=ws)


def _random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        M = int(rng.choice([int(rng.integers(1, 17)), int(rng.integers(17, 65)), int(rng.integers(65, 1200))]))
        N = 128 * int(rng.integers(1, 40))
        K = 128 * int(rng.integers(1, 12))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("M,N,K", _random_shapes(2024, 24))
def test_linear_random_shapes(M, N, K):
    """Seeded random shapes across every schedule the host can pick (decode, mid-size
    strips, split-K, each tile shape), with the binding's default workspace and without."""
    x, w = inputs(M, N, K, seed=M + 7 * N + 13 * K)
    ref = oracle_path(x, w)
    for ws in (None, torch.empty(0, dtype=torch.uint8, device="cuda")):
        banner(f"block_linear random shape M={M} N={N} K={K} workspace={'default' if ws is None else 'none'}")
        res = oracle.check_tolerance(gpu_path(x, w, workspace=ws), ref)
        assert res["ok"], res


def test_subnormal_codes_and_scales():
    """E4M3 subnormal codes and FP32-subnormal scales reach the MFMA and the promotion."""
    rng = np.random.default_rng(13)
    M, N, K = 8, 256, 256
    x = bf16(rng.standard_normal((M, K)) * 1e-3)
    x[:, ::2] = bf16(rng.standard_normal((M, K // 2)) * 1e-6)    # tiny -> subnormal codes
    x[0] = bf16(rng.standard_normal(K) * 1e-39)                   # subnormal scales
    w = bf16(rng.standard_normal((N, K)) * 0.02)
    q, s = oracle.quant_act(x)
    assert np.any((q & 0x78) == 0) and np.any(s < np.finfo(np.float32).tiny)
    check_linear(x, w, "subnormal codes")


@pytest.mark.parametrize("M,N,K,split", [(65, 1024, 2048, None), (128, 2048, 7168, None), (200, 1024, 4096, None),
                                         (300, 1152, 2048, None), (128, 1024, 7168, "2"), (100, 512, 3072, "3"),
                                         (129, 768, 4096, "8"), (80, 256, 512, "4"),
                                         # 128 x 256 split tiles (M > 128, N a multiple of 256)
                                         (300, 1024, 2048, None), (384, 2048, 4096, None), (129, 512, 3072, "5"),
                                         (257, 768, 1152, "2"), (500, 1280, 2048, "3")])
def test_split_k(M, N, K, split, monkeypatch):
    """Split-K over the workgroups of each tile (FP32 partials in the workspace, then a
    fixed-order reduce): within tolerance, and bitwise repeatable."""
    if split:
        monkeypatch.setenv("FP8BS_PREFILL_KSPLIT", split)
    assert fb.workspace_size(M, N, K) > 0 or split
    x, w = inputs(M, N, K, seed=5 * M + N + K)
    ws = torch.empty(8 * M * N * 4, dtype=torch.uint8, device="cuda")
    y = check_linear(x, w, f"split-K {split}", workspace=ws)
    assert np.array_equal(gpu_path(x, w, workspace=ws), y)


def test_default_workspace_per_stream():
    """The binding's default workspace is one buffer per (device, stream): split-K calls
    on two streams at once give the same bits as the same calls in sequence."""
    M, N, K = 128, 2048, 4096
    cases = [inputs(M, N, K, seed=40 + i) for i in range(2)]
    dev_in = []
    for x, w in cases:
        q, s = fb.quant_act(dev_bf16(x))
        qw, ws = fb.quant_weight(dev_bf16(w))
        dev_in.append((q, s, qw, ws))
    assert fb.workspace_size(M, N, K) > 0
    want = [host_u16(fb.block_linear(*a)) for a in dev_in]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    outs = []
    for _ in range(5):
        for st, a in zip(streams, dev_in):
            with torch.cuda.stream(st):
                outs.append(fb.block_linear(*a))
    torch.cuda.synchronize()
    for i, y in enumerate(outs):
        assert np.array_equal(host_u16(y), want[i % 2]), i
    with torch.cuda.stream(streams[0]):
        w0 = fb.get_workspace("cuda", 1)
    with torch.cuda.stream(streams[1]):
        w1 = fb.get_workspace("cuda", 1)
    assert w0.data_ptr() != w1.data_ptr()


def test_split_k_workspace_sizes():
    """A smaller workspace selects a smaller split or none; every result is in tolerance."""
    M, N, K = 128, 2048, 4096
    x, w = inputs(M, N, K, seed=12)
    ref = oracle_path(x, w)
    need = fb.workspace_size(M, N, K)
    assert need > 0
    for nbytes in (need, need // 2, 2 * M * N * 4, M * N * 4, 0):
        banner(f"block_linear split-K workspace {nbytes}")
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        res = oracle.check_tolerance(gpu_path(x, w, workspace=ws), ref)
        assert res["ok"], (nbytes, res)


def test_graph_replay_matches_eager():
    """The path captured in a HIP graph (as the bench runs it) reproduces the eager
    outputs on every replay, with eager work in between."""
    x, w = inputs(8, 2048, 3072, seed=60)
    xd, wd = dev_bf16(x), dev_bf16(w)
    qw, ws = fb.quant_weight(wd)
    q = torch.empty((8, 3072), dtype=torch.uint8, device="cuda")
    s = torch.empty((8, 24), dtype=torch.float32, device="cuda")
    y = torch.empty((8, 2048), dtype=torch.bfloat16, device="cuda")
    fb.quant_act(xd, q, s)
    fb.block_linear(q, s, qw, ws, out=y)
    torch.cuda.synchronize()
    ref_q, ref_s, ref_y = q.clone(), s.clone(), y.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fb.quant_act(xd, q, s)
        fb.block_linear(q, s, qw, ws, out=y)
    for i in range(4):
        q.zero_(); s.zero_(); y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(q, ref_q) and torch.equal(s, ref_s) and torch.equal(y, ref_y), i
        fb.block_linear(q, s, qw, ws)          # eager work between replays
        torch.cuda.synchronize()
