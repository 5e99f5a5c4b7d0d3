"""MI355X (gfx950) W8A8 FP8 block-scaled linear.

Thin torch-facing binding over libfp8bs.so (include/fp8bs.h).  Torch supplies
device memory and the current stream; every step of the computation runs in the
library's HIP kernels.  The wrappers only check dtypes/devices/contiguity, allocate
outputs and pass raw pointers.

    q, s = quant_act(x)                       # x: bf16 [M, K] on a gfx950 device
    qw, ws = quant_weight(w)                  # w: bf16 [N, K]
    y = block_linear(q, s, qw, ws)            # y: bf16 [M, N]
    q2, s2 = silu_mul_quant(gu)               # gu: bf16 [M, 2I] -> codes of BF16(silu(g)*u)
    q3, s3 = rmsnorm_quant(x, gamma, 1e-5)    # codes of BF16(RMSNorm(x) * gamma)
    y4 = nvfp4_linear(x, w4, bs, g)           # NVFP4 weights: w4 uint8 [N, K/2], bs [N, K/16]

Tensor dtypes: BF16 tensors are torch.bfloat16; E4M3 codes are torch.uint8 (view
them as torch.float8_e4m3fn if wanted); scales are torch.float32.
"""

import torch

from ._lib import Fp8bsError, check, lib  # noqa: F401

__all__ = [
    "quant_act",
    "quant_weight",
    "silu_mul_quant",
    "rmsnorm_quant",
    "block_linear",
    "nvfp4_linear",
    "nvfp4_workspace_size",
    "workspace_size",
    "get_workspace",
    "Fp8bsError",
]

_workspaces = {}


def _call(fn_name, device, *args):
    """Call a C entry point with the current stream of ``device`` appended."""
    fn = getattr(lib(), fn_name)
    if device.index is None or device.index == torch.cuda.current_device():
        check(fn_name, fn(*args, torch.cuda.current_stream().cuda_stream))
    else:
        with torch.cuda.device(device):
            check(fn_name, fn(*args, torch.cuda.current_stream().cuda_stream))


def _check_tensor(t, name, dtypes, ndim):
    """Type, dtype, number of dimensions and contiguity of one tensor (devices are
    checked by _check_tensors once every operand's shape is known)."""
    _check_tensors([(t, name, dtypes, ndim)], devices=False)


def _check_tensors(specs, devices=True):
    """Validate tensors before any pointer reaches the library.

    ``specs``: (tensor, name, dtypes, shape) with shape an int (the number of
    dimensions) or a tuple (the exact shape).  Every tensor is checked for type,
    dtype, shape and contiguity first, then all of them for being on one GPU: a
    wrong-sized output would otherwise let a kernel write past its allocation,
    which the C layer cannot detect.
    """
    for t, name, dtypes, shape in specs:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype not in dtypes:
            raise TypeError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
        if isinstance(shape, int):
            if t.dim() != shape:
                raise ValueError(f"{name} must be {shape}-D, got shape {tuple(t.shape)}")
        elif tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)}, got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not devices:
        return
    dev = None
    for t, name, _, _ in specs:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device (there is no CPU path)")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other operands on {dev}: all must be on one GPU")


_BF16 = (torch.bfloat16, torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.bfloat16, torch.int16)
_CODES = (torch.uint8, torch.float8_e4m3fn)


def _quant_outputs(x, q, s, M, K):
    """Allocate (or check) the codes [M, K] and scales [M, K/128] of a quantizer."""
    if K % 128:
        raise ValueError(f"K = {K} must be a multiple of 128")
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device) if q is None else q
    s = torch.empty((M, K // 128), dtype=torch.float32, device=x.device) if s is None else s
    _check_tensors([(x, "input", _BF16, 2), (q, "q", _CODES, (M, K)), (s, "s", (torch.float32,), (M, K // 128))])
    return q, s


def quant_act(x, q=None, s=None):
    """Per-token group-128 quantization of BF16 x [M, K] -> (q uint8 [M, K], s f32 [M, K/128])."""
    _check_tensor(x, "x", _BF16, 2)
    M, K = x.shape
    q, s = _quant_outputs(x, q, s, M, K)
    _call("fp8_quant_act", x.device, x.data_ptr(), q.data_ptr(), s.data_ptr(), M, K)
    return q, s


def quant_weight(w):
    """128x128 block quantization of BF16 w [N, K] -> (qw uint8 [N, K], ws f32 [N/128, K/128])."""
    _check_tensor(w, "w", _BF16, 2)
    N, K = w.shape
    if N % 128 or K % 128:
        raise ValueError(f"N = {N} and K = {K} must be multiples of 128")
    qw = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    _check_tensors([(w, "w", _BF16, 2), (qw, "qw", _CODES, (N, K)), (ws, "ws", (torch.float32,), (N // 128, K // 128))])
    _call("fp8_quant_weight", w.device, w.data_ptr(), qw.data_ptr(), ws.data_ptr(), N, K)
    return qw, ws


def silu_mul_quant(gu, q=None, s=None):
    """Codes and scales of BF16(silu(gate) * up) for gu = [gate | up], BF16 [M, 2I]."""
    _check_tensor(gu, "gu", _BF16, 2)
    M, two_i = gu.shape
    if two_i % 2:
        raise ValueError("gate/up width must be even")
    I = two_i // 2
    q, s = _quant_outputs(gu, q, s, M, I)
    _call("fp8_silu_mul_quant", gu.device, gu.data_ptr(), q.data_ptr(), s.data_ptr(), M, I)
    return q, s


def rmsnorm_quant(x, gamma, eps, q=None, s=None):
    """Codes and scales of BF16(x / sqrt(mean(x^2) + eps) * gamma) for BF16 x [M, K]
    and gamma [K] (FP64 evaluation, one BF16 rounding), quantized per token and group."""
    _check_tensor(x, "x", _BF16, 2)
    M, K = x.shape
    _check_tensor(gamma, "gamma", _BF16, 1)
    if gamma.shape[0] != K:
        raise ValueError(f"gamma must have shape ({K},), got shape {tuple(gamma.shape)}")
    q, s = _quant_outputs(x, q, s, M, K)
    _check_tensors([(x, "x", _BF16, 2), (gamma, "gamma", _BF16, (K,))])
    _call("fp8_rmsnorm_quant", x.device, x.data_ptr(), gamma.data_ptr(), float(eps), q.data_ptr(), s.data_ptr(), M, K)
    return q, s


def workspace_size(M, N, K):
    return int(lib().fp8_block_linear_workspace_size(M, N, K))


def get_workspace(device, nbytes):
    """A workspace of at least ``nbytes`` for ``device`` and its current stream, cached
    per (device, stream).

    No call reads workspace it has not written earlier in the same call, so the buffer
    is neither cleared nor initialized (no fill is enqueued, also under graph capture).
    Calls on one stream run in order, so they can share it; calls on different streams
    get different buffers, each allocated while its stream is current.
    """
    device = torch.device(device)
    index = device.index if device.index is not None else torch.cuda.current_device()
    key = (index, torch.cuda.current_stream(index).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(nbytes, 1 << 20)
        size = (size + 255) // 256 * 256
        ws = torch.empty(size, dtype=torch.uint8, device=torch.device("cuda", index))
        _workspaces[key] = ws
    return ws


def block_linear(q, s, qw, ws, out=None, workspace=None):
    """y [M, N] bf16 = (q * s) @ (qw * ws)^T with FP32 accumulation per 128-wide K block."""
    _check_tensor(q, "q", _CODES, 2)
    _check_tensor(qw, "qw", _CODES, 2)
    M, K = q.shape
    N = qw.shape[0]
    if qw.shape[1] != K:
        raise ValueError("q and qw disagree on K")
    if K % 128 or N % 128:
        raise ValueError(f"K = {K} and N = {N} must be multiples of 128")
    dev = q.device
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    specs = [(q, "q", _CODES, (M, K)), (s, "s", (torch.float32,), (M, K // 128)), (qw, "qw", _CODES, (N, K)),
             (ws, "ws", (torch.float32,), (N // 128, K // 128)), (y, "out", _BF16, (M, N))]
    if workspace is not None:
        specs.append((workspace, "workspace", (torch.uint8,), 1))
    _check_tensors(specs)
    if workspace is None:
        need = workspace_size(M, N, K) if K > 0 else 0
        workspace = get_workspace(dev, need) if need else None
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _call("fp8_block_linear", dev, q.data_ptr(), s.data_ptr(), qw.data_ptr(), ws.data_ptr(), y.data_ptr(),
          M, N, K, wptr, wbytes)
    return y


def nvfp4_workspace_size(M, N, K):
    """Bytes of workspace nvfp4_linear's fastest schedule can use for this shape."""
    return int(lib().nvfp4_w4a16_workspace_size(M, N, K))


def nvfp4_linear(x, w4, bs, g, out=None, workspace=None):
    """y [M, N] bf16 = x @ W^T, W[n, k] = e2m1(w4 codes) * e4m3(bs[n, k/16]) * g.

    x: bf16 [M, K]; w4: uint8 [N, K/2] packed codes (element 2j in the low nibble of
    byte j); bs: uint8 (or float8_e4m3fn) [N, K/16] group scales; g: float global scale.
    workspace: None (a cached per-device buffer of nvfp4_workspace_size bytes), or a
    uint8 tensor (an empty one selects the schedules that need none).
    """
    _check_tensor(x, "x", _BF16, 2)
    _check_tensor(w4, "w4", (torch.uint8,), 2)
    M, K = x.shape
    N = w4.shape[0]
    if w4.shape[1] * 2 != K:
        raise ValueError("w4 must be [N, K/2]")
    dev = x.device
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else out
    specs = [(x, "x", _BF16, (M, K)), (w4, "w4", (torch.uint8,), (N, K // 2)), (bs, "bs", _CODES, (N, K // 16)),
             (y, "out", _BF16, (M, N))]
    if workspace is not None:
        specs.append((workspace, "workspace", (torch.uint8,), 1))
    _check_tensors(specs)
    if workspace is None:
        need = nvfp4_workspace_size(M, N, K) if K > 0 and K % 128 == 0 and N % 128 == 0 else 0
        workspace = get_workspace(dev, need) if need else None
    wptr = workspace.data_ptr() if workspace is not None and workspace.numel() else None
    wbytes = workspace.numel() * workspace.element_size() if wptr is not None else 0
    _call("nvfp4_w4a16_linear", dev, x.data_ptr(), w4.data_ptr(), bs.data_ptr(), float(g), y.data_ptr(), M, N, K,
          wptr, wbytes)
    return y
