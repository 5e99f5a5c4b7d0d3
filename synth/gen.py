"""Counter-based seeded BF16 draws (no method arithmetic lives here)."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Tensor ids: independent streams for each tensor of a workload.
TID_X = 0
TID_W = 1
TID_OUTLIER = 2
TID_ZERO = 3
TID_ROWS = 4
TID_GU = 5
TID_W_DOWN = 6
TID_GAMMA = 7          # RMSNorm weight vector
TID_W4 = 8             # packed 4-bit weight codes (two per byte)
TID_W4_SCALE = 9       # 8-bit per-group weight scale codes


def _rng(seed, tid, row):
    """Generator for row ``row`` of tensor ``tid`` under ``seed`` (Philox key)."""
    key = (int(seed) << 96) | (int(tid) << 64) | int(row)
    return np.random.Generator(np.random.Philox(key=key))


def f32_to_bf16_bits(x):
    """Round float32 to BF16 (nearest, ties to even) and return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def _threads():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, n or 1))


def normal_rows(rows, n_cols, seed, tid, col_scale=None):
    """float32 [len(rows), n_cols]: standard normal samples of the given rows.

    ``col_scale`` (float32 [n_cols]) multiplies each column after drawing.
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    out = np.empty((rows.size, n_cols), dtype=np.float32)

    def work(lo, hi):
        for i in range(lo, hi):
            out[i] = _rng(seed, tid, rows[i]).standard_normal(n_cols, dtype=np.float32)
            if col_scale is not None:
                out[i] *= col_scale

    n = rows.size
    nt = _threads() if n * n_cols >= (1 << 22) else 1
    step = (n + nt - 1) // nt if n else 1
    if nt == 1:
        work(0, n)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(lambda lo: work(lo, min(n, lo + step)), range(0, n, step)))
    return out


def bf16_normal(n_rows, n_cols, sigma, seed, tid, rows=None):
    """uint16 BF16 bits of N(0, sigma^2) samples, [n_rows, n_cols] (or the given rows)."""
    rows = np.arange(n_rows) if rows is None else rows
    scale = np.full(n_cols, np.float32(sigma), dtype=np.float32)
    return f32_to_bf16_bits(normal_rows(rows, n_cols, seed, tid, scale))


def uniform_bytes(n_rows, n_cols, lo, hi, seed, tid):
    """uint8 [n_rows, n_cols], each byte uniform on the integers [lo, hi], seeded per row."""
    out = np.empty((n_rows, n_cols), dtype=np.uint8)

    def work(a, b):
        for i in range(a, b):
            out[i] = _rng(seed, tid, i).integers(lo, hi + 1, size=n_cols, dtype=np.uint8)

    nt = _threads() if n_rows * n_cols >= (1 << 22) else 1
    step = (n_rows + nt - 1) // nt if n_rows else 1
    if nt == 1:
        work(0, n_rows)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(lambda a: work(a, min(n_rows, a + step)), range(0, n_rows, step)))
    return out


def choose(n_total, n_pick, seed, tid):
    """Sorted int64 array of ``n_pick`` distinct indices in [0, n_total), seeded."""
    perm = _rng(seed, tid, 0).permutation(n_total)
    return np.sort(perm[:n_pick]).astype(np.int64)


def sample_rows(n_total, n_pick, seed):
    """Seeded rows for sampled checks of large outputs."""
    return choose(n_total, min(n_pick, n_total), seed, TID_ROWS)
