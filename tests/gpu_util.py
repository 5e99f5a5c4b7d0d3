"""Helpers for the GPU parity tests: move seeded host arrays to the device and back.

Inputs always come from ``synth`` (host numpy); the oracle and the HIP path each
receive the same host arrays and never each other's outputs."""

import sys

import numpy as np
import torch


def banner(msg):
    """Name the case before a GPU step, flushed, so a failing run still says which."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).cuda()


def dev_f32(v):
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).cuda()


def host_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_u8(t):
    return t.contiguous().cpu().numpy()


def host_f32(t):
    return t.contiguous().cpu().numpy()


def assert_bits_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if got.dtype == np.float32:
        got, want = got.view(np.uint32), want.view(np.uint32)
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: got {got[i]!r} want {want[i]!r}")
