"""GPU parity: the HIP quantizers against the CPU oracle, bit for bit.

Codes and scales must match exactly (activations: per-token group-128; weights:
128x128 blocks; SiLU(gate)*up re-quantization)."""

import numpy as np
import pytest
import torch

import fp8_block_scaled_amd as fb
import oracle
import synth
from tests.gpu_util import assert_bits_equal, banner, dev_bf16, host_f32, host_u8

pytestmark = pytest.mark.gpu


def bf16(x):
    x = np.asarray(x, dtype=np.float32)
    return synth.f32_to_bf16_bits(x).reshape(x.shape)


def run_quant(bits):
    q, s = fb.quant_act(dev_bf16(bits))
    torch.cuda.synchronize()
    return host_u8(q), host_f32(s)


def check_quant(bits, what):
    banner(f"quant_act {what} shape={bits.shape}")
    q, s = run_quant(bits)
    qo, so = oracle.quant_act(bits)
    assert_bits_equal(s, so, f"{what} scales")
    assert_bits_equal(q, qo, f"{what} codes")


@pytest.mark.parametrize("M,K,sigma", [(1, 128, 1.0), (3, 384, 0.02), (4, 512, 1.0), (17, 1024, 7.0),
                                       (64, 7168, 1.0), (129, 2048, 1e-3), (1000, 256, 3e4)])
def test_quant_act_random(M, K, sigma):
    rng = np.random.default_rng(M * 1000 + K)
    check_quant(bf16(rng.standard_normal((M, K)) * sigma), f"random sigma={sigma}")


def test_quant_act_edge_groups():
    rng = np.random.default_rng(7)
    x = bf16(rng.standard_normal((12, 1024)))
    x[0, :128] = 0                         # +0 group
    x[1, :] = 0x8000                       # row of -0.0
    x[2, :128] = 0x0001                    # smallest subnormal everywhere
    x[2, 128:256] = 0x8001
    x[2, 256:384] = bf16(np.full(128, 3.0))        # constant group -> all 448
    x[3, :128] = 0x7F7F                    # largest finite BF16
    x[3, 128] = 0xFF7F
    x[4, :] = bf16(rng.standard_normal(1024) * 1e-38)   # subnormal scales
    x[5, 0] = bf16(np.float32(448.0))      # s = 1: x/s = x, codes hit E4M3 midpoints
    mids = []
    t = oracle.decode_table()[:0x7F]
    for c in range(0x7E):
        mids.append((t[c] + t[c + 1]) / 2)
    mids = np.array(mids, dtype=np.float32)          # the 126 midpoints between magnitudes
    x[5, 1:127] = bf16(mids)
    x[5, 128:256] = bf16(-np.float32(448.0) * np.ones(128))
    x[6, 1:128] = bf16(np.float32(1e-30))  # one non-zero in a group of tiny values
    x[6, 0] = bf16(np.float32(5.0))
    x[7, :] = bf16(np.linspace(-448, 448, 1024))
    x[8, ::2] = 0x8000
    check_quant(x, "edge groups")


def test_quant_act_every_bf16_amax():
    """One group per positive finite BF16 amax (32639 groups), the other 127 values
    spread over [-amax, amax] in BF16."""
    amax_bits = np.arange(1, 0x7F80, dtype=np.uint32)
    amax = (amax_bits << 16).view(np.float32)
    frac = np.linspace(-1.0, 1.0, 127, dtype=np.float64)
    body = (amax[:, None].astype(np.float64) * frac[None, :]).astype(np.float32)
    # |amax * frac| <= amax and amax is a BF16 value, so rounding never exceeds it.
    x = np.concatenate([amax_bits.astype(np.uint16)[:, None], bf16(body)], axis=1)
    check_quant(np.ascontiguousarray(x), "all BF16 amax values")


def test_quant_act_empty():
    q, s = fb.quant_act(torch.empty((0, 256), dtype=torch.bfloat16, device="cuda"))
    assert q.shape == (0, 256) and s.shape == (0, 2)


@pytest.mark.parametrize("N,K,sigma", [(128, 128, 0.02), (384, 512, 0.02), (256, 1152, 10.0), (1024, 256, 1e-5)])
def test_quant_weight_random(N, K, sigma):
    rng = np.random.default_rng(N + K)
    w = bf16(rng.standard_normal((N, K)) * sigma)
    w[:128, :128] = 0                      # an all-zero block
    banner(f"quant_weight N={N} K={K}")
    qw, ws = fb.quant_weight(dev_bf16(w))
    torch.cuda.synchronize()
    qo, so = oracle.quant_weight(w)
    assert_bits_equal(host_f32(ws), so, "weight scales")
    assert_bits_equal(host_u8(qw), qo, "weight codes")


@pytest.mark.parametrize("M,I,sigma", [(1, 128, 1.7), (8, 8192, 1.7), (37, 1024, 0.3), (5, 256, 40.0)])
def test_silu_mul_quant(M, I, sigma):
    rng = np.random.default_rng(M * 7 + I)
    gu = bf16(rng.standard_normal((M, 2 * I)) * sigma)
    gu[0, :8] = bf16(np.array([0, -0.0, 80, -80, 1e-30, -1e-30, 300, -300], np.float32))
    banner(f"silu_mul_quant M={M} I={I}")
    q, s = fb.silu_mul_quant(dev_bf16(gu))
    torch.cuda.synchronize()
    qo, so = oracle.silu_mul_quant(gu)
    assert_bits_equal(host_f32(s), so, "silu scales")
    assert_bits_equal(host_u8(q), qo, "silu codes")


@pytest.mark.parametrize("M,I", [(1023, 8192), (1024, 8192), (2048, 8192)])
def test_silu_mul_quant_both_sides_of_the_unrolled_form(M, I):
    """1023 x 8192 (65,472 groups) runs the one-group-per-row form, 1024 x 8192 (exactly
    65,536 groups) and 2048 x 8192 (the chunked-prefill size the bench times) the
    unrolled one; near-midpoint probes are planted in every row, 8 per row."""
    rng = np.random.default_rng(M + I)
    gu = bf16(rng.standard_normal((M, 2 * I)) * 1.7)
    g_near, u_near = _silu_probes(rng, 8 * M, 24)
    rows = np.repeat(np.arange(M), 8)
    cols = rng.integers(0, I, 8 * M)
    gu[rows, cols] = g_near
    gu[rows, I + cols] = u_near
    banner(f"silu_mul_quant M={M} I={I} ({M * I // 128} groups)")
    q, s = fb.silu_mul_quant(dev_bf16(gu))
    torch.cuda.synchronize()
    qo, so = oracle.silu_mul_quant(gu)
    assert_bits_equal(host_f32(s), so, "silu scales")
    assert_bits_equal(host_u8(q), qo, "silu codes")


@pytest.mark.parametrize("M,I", [(65537, 128), (65600, 256)])
def test_silu_mul_quant_rows_past_the_grid(M, I):
    """More rows than the grid's second dimension holds (65,535): blocks walk the rest with a
    stride; every row, the last ones included, bit-exact."""
    rng = np.random.default_rng(M + 3 * I)
    gu = bf16(rng.standard_normal((M, 2 * I)) * 1.7)
    gu[-1, :4] = bf16(np.array([3.0, -2.0, 0.5, 80.0], np.float32))
    banner(f"silu_mul_quant M={M} I={I} (rows past the grid)")
    q, s = fb.silu_mul_quant(dev_bf16(gu))
    torch.cuda.synchronize()
    qo, so = oracle.silu_mul_quant(gu)
    assert_bits_equal(host_f32(s), so, "silu scales")
    assert_bits_equal(host_u8(q), qo, "silu codes")


def test_quant_is_deterministic():
    rng = np.random.default_rng(99)
    x = dev_bf16(bf16(rng.standard_normal((257, 2048))))
    ref = [t.clone() for t in fb.quant_act(x)]
    for _ in range(3):
        q, s = fb.quant_act(x)
        assert torch.equal(q, ref[0]) and torch.equal(s.view(torch.int32), ref[1].view(torch.int32))


def every_x_groups(amax_bits):
    """Groups holding, for each amax, every BF16 magnitude in [0, amax] once (each
    group starts with amax itself, so that is its scale); odd groups negated."""
    rows = []
    for a in amax_bits:
        xs = np.arange(0, int(a) + 1, dtype=np.uint16)
        pad = (-len(xs)) % 127
        xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 127)
        g = np.concatenate([np.full((len(xs), 1), a, np.uint16), xs], axis=1)
        g[1::2] |= np.uint16(0x8000)
        rows.append(g)
    return np.concatenate(rows)


def test_quant_act_every_x_for_many_scales():
    """For amax across the whole BF16 exponent range (mantissas 0x00, 0x7F and
    random), every BF16 value up to amax, both signs: codes and scales bit-exact.
    Covers both quotient paths (group scales below and above 2^-60)."""
    rng = np.random.default_rng(17)
    amax = []
    for e in range(1, 255):                          # every biased BF16 exponent
        for m in (0x00, 0x7F, int(rng.integers(1, 0x7F))):
            amax.append((e << 7) | m)
    amax += [0x0001, 0x0040, 0x007F, 0x2640, 0x2641, 0x2660, 0x2680, 0x3F80, 0x43E0, 0x4270, 0x7F7F]
    amax = sorted(set(amax))
    bits = every_x_groups(np.array(amax, np.uint16))
    check_quant(bits, f"every x for {len(amax)} scales")


def _silu_probes(rng, count, window):
    """(g, u) BF16 pairs whose float64 g u / (1 + e^-g) lies within `window` float32
    ulps of a BF16 rounding midpoint (low 16 bits near 0x8000)."""
    found = []
    while sum(len(f[0]) for f in found) < count:
        g = bf16(rng.standard_normal(1 << 20) * 3.0)
        u = bf16(rng.standard_normal(1 << 20) * 3.0)
        gf = oracle.bf16_bits_to_f32(g).astype(np.float64)
        uf = oracle.bf16_bits_to_f32(u).astype(np.float64)
        h = gf * uf / (1.0 + np.exp(-gf))
        low = h.astype(np.float32).view(np.uint32) & 0xFFFF
        near = np.nonzero((np.abs(low.astype(np.int64) - 0x8000) <= window) & (np.abs(h) > 1e-30))[0]
        found.append((g[near], u[near]))
    g = np.concatenate([f[0] for f in found])[:count]
    u = np.concatenate([f[1] for f in found])[:count]
    return g, u


def test_silu_mul_quant_probes():
    """Each 128-group holds one probe element that dominates the group, so the group's
    scale fl32(amax / 448) reads back the probe's BF16 h exactly: probes within 24 float32
    ulps of a BF16 rounding midpoint (the float64 recomputation), extreme gates (float32
    exp overflow and underflow) and huge or tiny products, against the oracle."""
    rng = np.random.default_rng(99)
    I = 1024
    groups_per_row = I // 128
    g_near, u_near = _silu_probes(rng, 2048, 24)
    extreme_g = np.array([-200, -120, -100, -90, -88, -87, -80, -60, -20, 20, 60, 87, 88, 100, 200], np.float32)
    extreme_u = np.array([1e36, -1e36, 1e30, 1e-30, -1e-37, 5e-39], np.float32)   # |h| stays below BF16 max
    eg, eu = np.meshgrid(extreme_g, extreme_u)
    probes_g = np.concatenate([g_near, bf16(eg.ravel())])
    probes_u = np.concatenate([u_near, bf16(eu.ravel())])
    n = len(probes_g)
    M = (n + groups_per_row - 1) // groups_per_row
    gate = bf16(rng.standard_normal((M, I)) * 1e-3)       # background: tiny products
    up = bf16(rng.standard_normal((M, I)) * 1e-3)
    idx = np.arange(n)
    rows, cols = idx // groups_per_row, (idx % groups_per_row) * 128 + rng.integers(0, 128, n)
    gate[rows, cols] = probes_g
    up[rows, cols] = probes_u
    gu = np.concatenate([gate, up], axis=1)
    banner(f"silu_mul_quant probes: {len(g_near)} near midpoints, {eg.size} extreme")
    q, s = fb.silu_mul_quant(dev_bf16(gu))
    torch.cuda.synchronize()
    qo, so = oracle.silu_mul_quant(gu)
    assert_bits_equal(host_f32(s), so, "probe scales")
    assert_bits_equal(host_u8(q), qo, "probe codes")


def check_rmsnorm(x, g, eps, what):
    banner(f"rmsnorm_quant {what} shape={x.shape}")
    q, s = fb.rmsnorm_quant(dev_bf16(x), dev_bf16(g), eps)
    torch.cuda.synchronize()
    qo, so = oracle.rmsnorm_quant(x, g, eps)
    assert_bits_equal(host_f32(s), so, f"{what} scales")
    assert_bits_equal(host_u8(q), qo, f"{what} codes")


@pytest.mark.parametrize("M,K", [(1, 128), (1, 7168), (5, 384), (37, 2048), (300, 1024), (8, 21504), (2000, 1024),
                                 (3, 4096), (2, 8192), (2, 33024), (64, 1152), (65, 1152), (1, 66048)])
def test_rmsnorm_quant_random(M, K):
    # (64, 1152) and (65, 1152) sit on both sides of the switch to 1024-thread workgroups
    # for few rows; (1, 66048) takes the few-rows kernel's re-reading form (over 8 passes).
    rng = np.random.default_rng(M * 7 + K)
    x = bf16(rng.standard_normal((M, K)) * 10.0 ** rng.integers(-3, 4, (M, 1)))
    g = bf16(rng.standard_normal(K) * 0.3 + 1.0)
    check_rmsnorm(x, g, np.float32(1e-5), "random")


# Each shape reaches one form of the kernel (chunks per thread U, threads per row NT):
# 256 threads above 64 rows, 1024 up to 64 rows; U = groups per thread rounded up to
# 1, 2, 4, 8, 16 (256 threads only), else 0 (the form that re-reads x and gamma).
@pytest.mark.parametrize("M,K,form", [(70, 2048, "<1,256>"), (70, 4096, "<2,256>"), (65, 7168, "<4,256>"),
                                      (70, 16384, "<8,256>"), (66, 32768, "<16,256>"), (66, 33024, "<0,256>"),
                                      (4, 7168, "<1,1024>"), (4, 12288, "<2,1024>"), (2, 32768, "<4,1024>"),
                                      (2, 65536, "<8,1024>"), (1, 66048, "<0,1024>")])
def test_rmsnorm_quant_every_form(M, K, form):
    rng = np.random.default_rng(M * 13 + K)
    x = bf16(rng.standard_normal((M, K)) * 10.0 ** rng.integers(-3, 4, (M, 1)))
    x[0, :128] = 0                                      # a zero group
    g = bf16(rng.standard_normal(K) * 0.3 + 1.0)
    check_rmsnorm(x, g, np.float32(1e-5), f"form {form}")


def test_rmsnorm_quant_prefill_oproj_full_size():
    """The bench's prefill case, 8191 x 7168 (256-thread form, 4 chunks per thread), in
    one call; 256 seeded rows, the 8 zero tokens and the last row against the oracle
    (each row is independent of the others)."""
    wl = synth.WORKLOADS["prefill_oproj"]
    x = synth.make_activation(wl)
    g = bf16(oracle.bf16_bits_to_f32(synth.bf16_normal(1, wl.K, 0.1, wl.seed, synth.TID_GAMMA)[0]) + 1.0)
    banner(f"rmsnorm_quant prefill_oproj full M={wl.M} K={wl.K}")
    q, s = fb.rmsnorm_quant(dev_bf16(x), dev_bf16(g), 1e-5)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([synth.sample_rows(wl.M, 256, wl.seed), wl.zero_tokens(), [wl.M - 1]]))
    rows_t = torch.from_numpy(rows.astype(np.int64)).cuda()
    qh, sh = host_u8(q[rows_t]), host_f32(s[rows_t])
    qo, so = oracle.rmsnorm_quant(x[rows], g, np.float32(1e-5))
    assert_bits_equal(sh, so, "prefill_oproj rmsnorm scales")
    assert_bits_equal(qh, qo, "prefill_oproj rmsnorm codes")
    assert np.all(sh[np.isin(rows, wl.zero_tokens())] == 0)


def test_rmsnorm_quant_redo_path():
    """Inputs with many elements whose float32 product x r gamma lies within 8 ulps of a
    BF16 rounding midpoint, the case the kernel recomputes in float64: the count is
    taken on the host first, so the test is known to reach that path."""
    rng = np.random.default_rng(41)
    M, K = 512, 2048
    x = bf16(rng.standard_normal((M, K)))
    g = bf16(rng.standard_normal(K) * 0.3 + 1.0)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + 1e-5)
    h32 = (oracle.bf16_bits_to_f32(x) * r.astype(np.float32)) * oracle.bf16_bits_to_f32(g)
    low = h32.astype(np.float32).view(np.uint32) & 0xFFFF
    near = int(np.count_nonzero((low >= 0x7FF8) & (low < 0x8008)))
    assert near > 100, near
    check_rmsnorm(x, g, np.float32(1e-5), f"{near} near-midpoint elements")


def test_rmsnorm_quant_probes():
    """One element per 128-group dominates its group (the rest is a tiny background), so
    every group scale reads back that element's BF16 h exactly.  16384 rows x 8 probes
    put a few dozen probes within 8 float32 ulps of a BF16 rounding midpoint, where the
    kernel recomputes in float64, and many more just outside; the count is taken on the
    host first."""
    rng = np.random.default_rng(77)
    M, K = 16384, 1024
    x = bf16(rng.standard_normal((M, K)) * 1e-4)
    cols = np.arange(0, K, 128)[None, :] + rng.integers(0, 128, (M, K // 128))
    rows = np.repeat(np.arange(M)[:, None], K // 128, axis=1)
    x[rows, cols] = bf16(rng.standard_normal((M, K // 128)) * 4.0)
    g = bf16(rng.standard_normal(K) * 0.3 + 1.0)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(xf * xf, axis=1, keepdims=True) + 1e-5)
    h = (xf * r * oracle.bf16_bits_to_f32(g).astype(np.float64))[rows, cols]
    low = h.astype(np.float32).view(np.uint32).astype(np.int64) & 0xFFFF
    near = int(np.count_nonzero(np.abs(low - 0x8000) <= 8))
    assert near > 20, near
    check_rmsnorm(x, g, np.float32(1e-5), f"probes ({near} within 8 ulps of a midpoint)")


def test_rmsnorm_quant_edge_rows():
    rng = np.random.default_rng(3)
    K = 1024
    x = bf16(rng.standard_normal((8, K)))
    x[0] = 0                                   # zero row -> all scales 0
    x[1] = 0x8000                              # -0.0 row
    x[2, :] = 0x0001                           # smallest subnormal: eps dominates
    x[3, :] = bf16(np.float32(3e38))           # largest magnitudes (x^2 in float64)
    x[4, 5] = bf16(np.float32(1e4))            # one spike: other groups near zero
    x[5, 128:256] = 0                          # one zero group in a normal row
    g = bf16(rng.standard_normal(K))
    g[:128] = 0                                # zero weights -> zero group
    check_rmsnorm(x, g, np.float32(1e-5), "edge rows")
    check_rmsnorm(x, g, np.float32(1.0), "edge rows, eps 1")


def test_rmsnorm_quant_workload_rows():
    """The decode shape (one token, K = 7168) and 64 rows of the prefill shape."""
    wl = synth.WORKLOADS["decode_qkv"]
    x = synth.make_activation(wl)
    g = bf16(oracle.bf16_bits_to_f32(synth.bf16_normal(1, wl.K, 0.1, wl.seed, synth.TID_GAMMA)[0]) + 1.0)
    check_rmsnorm(x, g, np.float32(1e-5), "decode_qkv")
    wp = synth.WORKLOADS["prefill_oproj"]
    rows = synth.activation_rows(wp, np.arange(64) * 127)
    check_rmsnorm(rows, g, np.float32(1e-5), "prefill_oproj rows")
