"""Python binding of libvq.so, the gfx950 quantized linear layer for video DiTs.

Argument marshalling only: every function takes torch tensors on the GPU, checks
their dtype/shape/contiguity, allocates missing outputs with torch (device memory
is PyTorch's), and calls the C entry point of the same name on torch's current
stream.  All arithmetic happens in the HIP kernels; if libvq.so is missing the
import of this module fails.
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvq.so")

VQ_OK, VQ_ERR_INVALID_ARG, VQ_ERR_SHAPE, VQ_ERR_UNSUPPORTED, VQ_ERR_HIP = range(5)
VQ_F16, VQ_BF16, VQ_F32 = 0, 1, 2
VQ_PER_TENSOR, VQ_PER_TOKEN, VQ_PER_TENSOR_STATIC = 0, 1, 2
VQ_MXFP6, VQ_MXFP4 = 2, 4
VQ_MXFP4_KBLOCK = VQ_MXFP4 | 0x100  # FP4 codes in 64-byte K pieces (weights)
VQ_K_ALIGN = 64
VQ_HAD_BLOCK = 128
VQ_MAX_OUTLIERS = 128
VQ_W_KBLOCK = 0x100  # weight layout flag: 64-byte K pieces, piece j of every row together

EXPORTS = (
    "vq_outlier_part_len", "vq_packed_k", "vq_weight_bytes", "vq_detect_workspace_elems", "vq_detect_outliers",
    "vq_pack_weights", "vq_quant_act", "vq_hadamard_block", "vq_qgemm_dequant", "vq_qgemm_workspace_bytes",
    "vq_qgemm_scratch_bytes", "vq_qgemm_dequant_noalloc",
    "vq_route_workspace_elems", "vq_route_rel_l1", "vq_quant_residual", "vq_residual_workspace_bytes",
    "vq_qgemm_dequant_residual", "vq_mx_code_bytes", "vq_mx_scale_bytes", "vq_mx_quant", "vq_mx_quant_rotated",
    "vq_mx_gemm",
    "vq_mx_gemm_workspace_bytes", "vq_gemm_dense",
    "vq_calib_hist_bins", "vq_calib_static_scale", "vq_control_workspace_elems", "vq_step_control",
    "vq_status_string", "vq_last_hip_error", "vq_version",
)
CALIB_GRID = (100.0, 99.999, 99.99, 99.9, 99.8, 99.5, 99.0, 98.0, 97.0, 95.0, 90.0)

_DT = {torch.float16: VQ_F16, torch.bfloat16: VQ_BF16, torch.float32: VQ_F32}
_GRAN = {"tensor": VQ_PER_TENSOR, "token": VQ_PER_TOKEN, "static": VQ_PER_TENSOR_STATIC}
_MX = {"fp4": VQ_MXFP4, "fp6": VQ_MXFP6}
_MX_BITS = {"fp4": 4, "fp6": 6}


class VQError(RuntimeError):
    def __init__(self, fn, status, text, hip):
        super().__init__(f"{fn} failed: status {status} ({text}); last HIP error {hip}")
        self.status = status
        self.hip_error = hip


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run python bit_quantized_linear_vq_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, I32, I, D, F = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int,
                            ctypes.c_double, ctypes.c_float)
    sig = {
        "vq_outlier_part_len": (I64, [I32]),
        "vq_packed_k": (I64, [I64, I32]),
        "vq_weight_bytes": (I64, [I64, I64, I]),
        "vq_detect_workspace_elems": (I64, [I64, I64]),
        "vq_detect_outliers": (I, [P, I, I64, I64, I64, D, D, D, P, P, P, P, P, P, P]),
        "vq_control_workspace_elems": (I64, []),
        "vq_step_control": (I, [P, P, I, I64, P, P, I, I64, P, I64, P, P, P, P, P, P, P, P]),
        "vq_pack_weights": (I, [P, I, I64, I64, I64, I, P, I32, I, P, P, P]),
        "vq_quant_act": (I, [P, I, I64, I64, I64, I, P, I, I, P, I32, P, P, P, P]),
        "vq_hadamard_block": (I, [P, I, I64, P, I, I64, I64, I64, I, I, P]),
        "vq_qgemm_dequant": (I, [P, P, I, P, I, P, I64, I64, I64, I64, P, I, I64, P, P, P]),
        "vq_qgemm_workspace_bytes": (I64, [I64, I64, I64]),
        "vq_qgemm_scratch_bytes": (I64, []),
        "vq_qgemm_dequant_noalloc": (I, [P, P, I, P, I, P, I64, I64, I64, I64, P, I, I64, P]),
        "vq_route_workspace_elems": (I64, [I64]),
        "vq_route_rel_l1": (I, [P, P, I, I64, D, I, I, P, P, P, P]),
        "vq_quant_residual": (I, [P, I, I64, I64, I64, I, I, P, I64, P, P, P]),
        "vq_residual_workspace_bytes": (I64, [I64, I64, I64]),
        "vq_qgemm_dequant_residual": (I, [P, P, P, I, P, I64, I64, I64, P, P, P, I64, P, I, I64, P, P]),
        "vq_mx_code_bytes": (I64, [I64, I64, I]),
        "vq_mx_scale_bytes": (I64, [I64, I64]),
        "vq_mx_quant": (I, [P, I, I64, I64, I64, I, P, P, P]),
        "vq_mx_quant_rotated": (I, [P, I, I64, I64, I64, I, I, P, P, P]),
        "vq_mx_gemm": (I, [P, P, I, P, P, I, I64, I64, I64, P, I, I64, P, P]),
        "vq_mx_gemm_workspace_bytes": (I64, [I64, I64, I64]),
        "vq_gemm_dense": (I, [P, P, I, I64, I64, I64, I64, I64, P, I, I64, P]),
        "vq_calib_hist_bins": (I64, []),
        "vq_calib_static_scale": (I, [P, I, I64, I64, I64, I, P, I32, P, P, P, P, P, P, P]),
        "vq_status_string": (ctypes.c_char_p, [I]),
        "vq_last_hip_error": (I, []),
        "vq_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def _check(fn, status):
    if status != VQ_OK:
        raise VQError(fn, status, _lib.vq_status_string(status).decode(), _lib.vq_last_hip_error())


def _stream(t: torch.Tensor):
    """torch's current stream on t's device, as the raw handle (an int: the signatures
    declare it a pointer).  The raw-handle accessor skips building a Stream object, which
    dominates the host cost of a call on small layers."""
    return torch._C._cuda_getCurrentRawStream(t.get_device())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev(t, name):
    """A device tensor whose last dimension is dense (the library takes a row pitch only)."""
    if not (isinstance(t, torch.Tensor) and t.is_cuda):
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dim() > 2 or (t.dim() >= 1 and t.size(-1) > 1 and t.stride(-1) != 1):
        raise ValueError(f"{name} must be 1-D or 2-D with unit stride along its last dimension")
    return t


def _buf(t, name, nbytes, device):
    """A caller-given output or scratch buffer: a contiguous device tensor of at least nbytes bytes."""
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.device == device):
        raise TypeError(f"{name} must be a CUDA (HIP) tensor on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, {nbytes} are needed")
    return t


def _in(t, name, dtypes, numel, device):
    """A caller-given device input read by a kernel: on `device`, one of `dtypes`,
    contiguous, with at least `numel` elements.  Checked before any launch, since a host
    tensor or a short buffer would be read out of bounds by the GPU."""
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.device == device):
        raise TypeError(f"{name} must be a CUDA (HIP) tensor on {device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} are needed")
    return t


_I32 = (torch.int32,)
_F32 = (torch.float32,)
_U8 = (torch.uint8,)


def _out2d(t, name, rows, cols, device):
    """A caller-given [rows x cols] output with unit stride along its rows (any row pitch >= cols)."""
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.device == device):
        raise TypeError(f"{name} must be a CUDA (HIP) tensor on {device}")
    if tuple(t.shape) != (rows, cols) or (cols > 1 and t.stride(1) != 1) or (rows > 1 and t.stride(0) < cols):
        raise ValueError(f"{name} must be [{rows} x {cols}] with unit stride along its rows")
    return t


def vq_outlier_part_len(n_out: int) -> int:
    return int(_lib.vq_outlier_part_len(n_out))


@functools.lru_cache(maxsize=1024)
def vq_packed_k(k: int, n_out: int) -> int:
    return int(_lib.vq_packed_k(k, n_out))


# Workspace sizes depend only on the shape (and the device's CU count, fixed per process).
@functools.lru_cache(maxsize=1024)
def _qgemm_ws_bytes(m: int, n: int, k0: int) -> int:
    return int(_lib.vq_qgemm_workspace_bytes(m, n, k0))


@functools.lru_cache(maxsize=1024)
def _mx_ws_bytes(m: int, n: int, k: int) -> int:
    return int(_lib.vq_mx_gemm_workspace_bytes(m, n, k))


def vq_detect_workspace_elems(rows: int, cols: int) -> int:
    """Float64 elements of the device workspace vq_detect_outliers needs for x [rows x cols]."""
    return int(_lib.vq_detect_workspace_elems(rows, cols))


def vq_detect_outliers(x: torch.Tensor, tau: float = 3.5, alpha: float = 2.0, kfac: float = 1.0, ws=None,
                       n_out_dev=None):
    """Outlier input channels (columns) of x.  Returns (mask uint8 [K], idx int32 [n_out], norms f64 [K]) on the host;
    n_out_dev (device int32 [1]), if given, receives the count for vq_step_control."""
    _dev(x, "x")
    rows, cols = x.shape
    need = vq_detect_workspace_elems(rows, cols)
    if ws is None:
        ws = torch.empty(need, dtype=torch.float64, device=x.device)
    _buf(ws, "ws", 8 * need, x.device)
    if n_out_dev is not None:
        _in(n_out_dev, "n_out_dev", _I32, 1, x.device)
    norms = torch.empty(cols, dtype=torch.float64)
    mask = torch.empty(cols, dtype=torch.uint8)
    idx = torch.empty(cols, dtype=torch.int32)
    n_out = ctypes.c_int32(0)
    _check("vq_detect_outliers", _lib.vq_detect_outliers(
        _ptr(x), _DT.get(x.dtype, -1), rows, cols, x.stride(0), tau, alpha, kfac, _ptr(ws),
        _ptr(norms), _ptr(mask), _ptr(idx), ctypes.byref(n_out), _ptr(n_out_dev), _stream(x)))
    return mask, idx[: n_out.value].clone(), norms


def vq_weight_bytes(n: int, kp: int, wfmt: int) -> int:
    return int(_lib.vq_weight_bytes(n, kp, wfmt))


def vq_pack_weights(w: torch.Tensor, bits: int, idx: torch.Tensor | None = None, had_block: int = 0,
                    codes=None, scales=None, kblock: bool = False):
    """Per-output-channel codes of W [N x K].  Returns (codes, scales).

    codes are int8 [N x kp] (8-bit) or uint8 [N x kp/2] (4-bit, two per byte); with
    kblock=True the same codes in 64-byte K pieces, [pieces x N x 64] (the GEMM calls take
    either form and tell them apart by the tensor's rank)."""
    _dev(w, "w")
    n, k = w.shape
    n_out = 0 if idx is None else int(idx.numel())
    if idx is not None:
        _in(idx, "idx", _I32, n_out, w.device)
    kp = vq_packed_k(k, n_out)
    wfmt = bits | (VQ_W_KBLOCK if kblock else 0)
    dt = torch.int8 if bits == 8 else torch.uint8
    row_bytes = kp if bits == 8 else kp // 2
    if codes is None:
        shape = ((row_bytes + 63) // 64, n, 64) if kblock else (n, row_bytes)
        codes = torch.empty(shape, dtype=dt, device=w.device)
    if scales is None:
        scales = torch.empty((n, 2) if n_out else (n,), dtype=torch.float32, device=w.device)
    _buf(codes, "codes", vq_weight_bytes(n, kp, wfmt) if bits in (4, 8) else 0, w.device)
    _buf(scales, "scales", 4 * n * (2 if n_out else 1), w.device)
    _check("vq_pack_weights", _lib.vq_pack_weights(
        _ptr(w), _DT.get(w.dtype, -1), n, k, w.stride(0), wfmt, _ptr(idx), n_out, had_block,
        _ptr(codes), _ptr(scales), _stream(w)))
    return codes, scales


def vq_kblock_to_rows(codes: torch.Tensor, n: int, row_bytes: int) -> torch.Tensor:
    """The row-major [N x row_bytes] view of weight codes in 64-byte K pieces (a copy)."""
    return codes.reshape(-1, n, 64).permute(1, 0, 2).reshape(n, -1)[:, :row_bytes].contiguous()


def vq_quant_act(x: torch.Tensor, bits: int, gran: str = "token", had_block: int = 0,
                 idx: torch.Tensor | None = None, static_scale: torch.Tensor | None = None,
                 bits_dev: torch.Tensor | None = None, codes=None, scales=None):
    """Online activation codes of X [M x K].  Returns (codes int8 [M x kp], scales)."""
    _dev(x, "x")
    m, k = x.shape
    n_out = 0 if idx is None else int(idx.numel())
    if idx is not None:
        _in(idx, "idx", _I32, n_out, x.device)
    if static_scale is not None:
        _in(static_scale, "static_scale", _F32, 2 if n_out else 1, x.device)
    if bits_dev is not None:
        _in(bits_dev, "bits_dev", _I32, 1, x.device)
    kp = vq_packed_k(k, n_out)
    g = _GRAN.get(gran, -1)
    if codes is None:
        codes = torch.empty((m, kp), dtype=torch.int8, device=x.device)
    if scales is None:
        parts = 2 if n_out else 1
        shape = ((m, 2) if n_out else (m,)) if g == VQ_PER_TOKEN else (parts,)
        scales = torch.empty(shape, dtype=torch.float32, device=x.device)
    _buf(codes, "codes", m * kp, x.device)
    _buf(scales, "scales", 4 * (m if g == VQ_PER_TOKEN else 1) * (2 if n_out else 1), x.device)
    _check("vq_quant_act", _lib.vq_quant_act(
        _ptr(x), _DT.get(x.dtype, -1), m, k, x.stride(0), bits, _ptr(bits_dev), g, had_block,
        _ptr(idx), n_out, _ptr(static_scale), _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def vq_hadamard_block(x: torch.Tensor, out_dtype=None, normalize: bool = True, block: int = 128, y=None):
    """Block Hadamard rotation of the rows of x (128-element blocks)."""
    _dev(x, "x")
    rows, cols = x.shape
    if y is None:
        y = torch.empty((rows, cols), dtype=out_dtype or x.dtype, device=x.device)
    _out2d(y, "y", rows, cols, x.device)
    _check("vq_hadamard_block", _lib.vq_hadamard_block(
        _ptr(x), _DT.get(x.dtype, -1), x.stride(0), _ptr(y), _DT.get(y.dtype, -1), y.stride(0), rows, cols,
        block, int(bool(normalize)), _stream(x)))
    return y


def vq_qgemm_dequant(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor, b_bits: int,
                     k0: int | None = None, out_dtype=torch.bfloat16, sa_per_token: bool = True,
                     acc_debug: bool = False, y=None, acc=None, ws=None):
    """Y = dequant(A_codes . B_codes^T).  Returns y, or (y, acc int32 [P x M x N]) with acc_debug.

    ws: None uses a zero-filled workspace kept per device and stream (the library leaves it
    zeroed after every call), a tensor of vq_qgemm_workspace_bytes() bytes is used as
    given, False runs without the remainder split."""
    _dev(a, "a")
    m, kp = a.shape
    k0 = kp if k0 is None else k0
    n, wfmt = _check_gemm_operands(a, sa, b, sb, b_bits, kp, k0, sa_per_token)
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=a.device)
    if acc_debug and acc is None:
        acc = torch.empty((2 if k0 < kp else 1, m, n), dtype=torch.int32, device=a.device)
    _out2d(y, "y", m, n, a.device)
    if acc_debug:
        _buf(acc, "acc", 4 * (2 if k0 < kp else 1) * m * n, a.device)
    ws = _gemm_workspace(m, n, k0, a.device) if ws is None else ws
    if ws is not False:
        _buf(ws, "ws", _qgemm_ws_bytes(m, n, k0), a.device)
    _check("vq_qgemm_dequant", _lib.vq_qgemm_dequant(
        _ptr(a), _ptr(sa), int(bool(sa_per_token)), _ptr(b), wfmt, _ptr(sb), m, n, kp, k0,
        _ptr(y), _DT.get(y.dtype, -1), y.stride(0), _ptr(acc if acc_debug else None),
        None if ws is False else _ptr(ws), _stream(a)))
    return (y, acc) if acc_debug else y


def _check_gemm_operands(a, sa, b, sb, b_bits, kp, k0, sa_per_token=True):
    """The GEMM's codes and scales as the kernels read them: A int8 [M x kp] dense; B int8
    [N x kp] (8-bit weights) or uint8 [N x kp/2] (4-bit), or those codes in 64-byte K
    pieces [pieces x N x 64] (vq_pack_weights(..., kblock=True)); scales float32 with one
    or two partitions (k0 < kp: two per row, column and tensor).  Returns (N, the weight
    format for the library: b_bits, with VQ_W_KBLOCK for the pieces)."""
    dev = a.device
    m = a.shape[0]
    parts = 2 if k0 < kp else 1
    _in(a, "a", (torch.int8,), m * kp, dev)
    if not (isinstance(b, torch.Tensor) and b.dim() in (2, 3)):
        raise TypeError("b must be a 2-D (row-major) or 3-D (K pieces) CUDA (HIP) tensor of packed weight codes")
    kblock = b.dim() == 3
    n = b.shape[1] if kblock else b.shape[0]
    if b_bits in (4, 8):
        row_bytes = kp if b_bits == 8 else kp // 2
        dts = (torch.int8,) if b_bits == 8 else _U8
        what = "int8 codes for 8-bit weights" if b_bits == 8 else "packed nibbles for 4-bit weights"
        _in(b, "b", dts, 0, dev)  # device, dtype and density first; then the shape fixes the size
        if kblock:
            pieces = (row_bytes + 63) // 64
            if tuple(b.shape) != (pieces, n, 64):
                raise ValueError(f"b in K pieces must be [{pieces} x N x 64] {what}")
        elif b.shape[1] != row_bytes:
            raise ValueError(f"b must be [N x {row_bytes}] {what}")
    _in(sa, "sa", _F32, (m if sa_per_token else 1) * parts, dev)
    _in(sb, "sb", _F32, n * parts, dev)
    return n, b_bits | (VQ_W_KBLOCK if kblock else 0)


def vq_qgemm_dequant_noalloc(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor, b_bits: int,
                             y: torch.Tensor, k0: int | None = None, sa_per_token: bool = True):
    """Y = dequant(A_codes . B_codes^T) into the caller's y, allocating nothing (the remainder
    split uses the library's static scratch; overlapping calls on one GPU race)."""
    _dev(a, "a")
    m, kp = a.shape
    k0 = kp if k0 is None else k0
    n, wfmt = _check_gemm_operands(a, sa, b, sb, b_bits, kp, k0, sa_per_token)
    _out2d(y, "y", m, n, a.device)
    _check("vq_qgemm_dequant_noalloc", _lib.vq_qgemm_dequant_noalloc(
        _ptr(a), _ptr(sa), int(bool(sa_per_token)), _ptr(b), wfmt, _ptr(sb), m, n, kp, k0,
        _ptr(y), _DT.get(y.dtype, -1), y.stride(0), _stream(a)))
    return y


_GEMM_WS = {}


def _gemm_workspace(m, n, k0, device):
    return _workspace(_qgemm_ws_bytes(m, n, k0), device)


def _workspace(need, device):
    """A remainder-split workspace of `need` bytes: one zero-filled buffer per device and
    stream, shared by both GEMMs and grown on demand (calls on one stream never overlap,
    and each leaves it zeroed)."""
    if need == 0:
        return False
    key = (device, torch._C._cuda_getCurrentRawStream(device.index))
    t = _GEMM_WS.get(key)
    if t is None or t.numel() < need:
        # Under graph capture a new buffer's zero fill would only be recorded, while the
        # buffer would be cached for eager calls that run before the first replay.
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(
                "the GEMM's remainder-split workspace must exist before graph capture: pass ws= (a zero-filled "
                "buffer of vq_qgemm_workspace_bytes / vq_mx_gemm_workspace_bytes bytes) or ws=False, or make one "
                "eager call on the capturing stream first")
        t = torch.zeros(need, dtype=torch.uint8, device=device)
        _GEMM_WS[key] = t
    return t


def vq_gemm_dense(x: torch.Tensor, w: torch.Tensor, out_dtype=None, y=None):
    """Unquantized FP16/BF16 layer Y = X . W^T (float32 accumulation), for the layers the
    precision override runs at 16 bits.  x [M x K] and w [N x K] share one 16-bit dtype;
    out_dtype defaults to it.  Returns y."""
    _dev(x, "x")
    _dev(w, "w")
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x and w must be 2-D")
    m, k = x.shape
    n = w.shape[0]
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise TypeError("x must be float16 or bfloat16")
    if w.dtype != x.dtype or w.device != x.device:
        raise TypeError(f"w must be a {x.dtype} tensor on {x.device}")
    if w.shape[1] != k:
        raise ValueError(f"w must be [N x {k}]")
    out_dtype = out_dtype or x.dtype
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _out2d(y, "y", m, n, x.device)
    _check("vq_gemm_dense", _lib.vq_gemm_dense(
        _ptr(x), _ptr(w), _DT[x.dtype], m, n, k, x.stride(0), w.stride(0), _ptr(y), _DT.get(y.dtype, -1),
        y.stride(0), _stream(x)))
    return y


def vq_route_rel_l1(x: torch.Tensor, y: torch.Tensor, threshold: float = 0.1, bits_hi: int = 8, bits_lo: int = 4,
                    ws=None, gamma=None, bits=None):
    """Device-side DMPQ route: returns (bits int32 [1], gamma float64 [1]) on the device."""
    _dev(x, "x")
    n = x.numel()
    _in(x, "x", (x.dtype,), n, x.device)
    _in(y, "y", (x.dtype,), n, x.device)
    if ws is None:
        ws = torch.empty(int(_lib.vq_route_workspace_elems(n)), dtype=torch.float64, device=x.device)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float64, device=x.device)
    if bits is None:
        bits = torch.empty(1, dtype=torch.int32, device=x.device)
    _buf(ws, "ws", 8 * int(_lib.vq_route_workspace_elems(n)), x.device)
    _buf(gamma, "gamma", 8, x.device)
    _buf(bits, "bits", 4, x.device)
    _check("vq_route_rel_l1", _lib.vq_route_rel_l1(
        _ptr(x), _ptr(y), _DT.get(x.dtype, -1), n, threshold, bits_hi, bits_lo, _ptr(ws), _ptr(gamma),
        _ptr(bits), _stream(x)))
    return bits, gamma


def vq_version() -> str:
    return _lib.vq_version().decode()


def vq_quant_residual(x: torch.Tensor, rows: torch.Tensor, bits1: int, bits2: int, codes=None, scales=None):
    """Decomposition operand of the listed rows.  Returns (codes int8 [2R x K], scales f32 [2R]):
    rows 0..R-1 hold the first quantizer's codes of the listed rows, rows R..2R-1 their residual codes."""
    _dev(x, "x")
    m, k = x.shape
    n_rows = int(rows.numel())
    if codes is None:
        codes = torch.empty((2 * n_rows, k), dtype=torch.int8, device=x.device)
    if scales is None:
        scales = torch.empty((2 * n_rows,), dtype=torch.float32, device=x.device)
    _in(rows, "rows", _I32, n_rows, x.device)
    _buf(codes, "codes", 2 * n_rows * k, x.device)
    _buf(scales, "scales", 8 * n_rows, x.device)
    _check("vq_quant_residual", _lib.vq_quant_residual(
        _ptr(x), _DT.get(x.dtype, -1), m, k, x.stride(0), bits1, bits2, _ptr(rows), n_rows,
        _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def vq_residual_workspace_bytes(m: int, n_rows: int, n: int) -> int:
    return int(_lib.vq_residual_workspace_bytes(m, n_rows, n))


def vq_qgemm_dequant_residual(a: torch.Tensor, sa: torch.Tensor, b: torch.Tensor, sb: torch.Tensor, b_bits: int,
                              a2: torch.Tensor, sa2: torch.Tensor, rows: torch.Tensor,
                              out_dtype=torch.bfloat16, y=None, ws=None):
    """Y = dequant(A . B^T); listed rows get both terms of the stacked operand (a2, sa2) added before rounding."""
    _dev(a, "a")
    m, kp = a.shape
    n, wfmt = _check_gemm_operands(a, sa, b, sb, b_bits, kp, kp)
    n_rows = int(rows.numel())
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=a.device)
    if ws is None and n_rows:
        ws = torch.empty(vq_residual_workspace_bytes(m, n_rows, n), dtype=torch.uint8, device=a.device)
    _out2d(y, "y", m, n, a.device)
    if n_rows:
        _in(rows, "rows", _I32, n_rows, a.device)
        _in(a2, "a2", (torch.int8,), 2 * n_rows * kp, a.device)
        _in(sa2, "sa2", _F32, 2 * n_rows, a.device)
        _buf(ws, "ws", vq_residual_workspace_bytes(m, n_rows, n), a.device)
    _check("vq_qgemm_dequant_residual", _lib.vq_qgemm_dequant_residual(
        _ptr(a), _ptr(sa), _ptr(b), wfmt, _ptr(sb), m, n, kp, _ptr(a2), _ptr(sa2), _ptr(rows), n_rows,
        _ptr(y), _DT.get(y.dtype, -1), y.stride(0), _ptr(ws), _stream(a)))
    return y


def vq_mx_code_bytes(rows: int, k: int, fmt: str) -> int:
    return int(_lib.vq_mx_code_bytes(rows, k, _MX[fmt]))


def vq_mx_scale_bytes(rows: int, k: int) -> int:
    return int(_lib.vq_mx_scale_bytes(rows, k))


def vq_mx_quant(x: torch.Tensor, fmt: str = "fp4", codes=None, scales=None, had_block: int = 0,
                exp_offset: int = 0, kblock: bool = False):
    """MX codes of X [rows x K].  Returns (codes uint8 [rows x K*w/8], scales uint8 E8M0 in step-major order).

    had_block=128 rotates each row by the unnormalized 128-point block Hadamard transform
    first (vq_mx_quant_rotated), scaled by 2^exp_offset (-7 for weights rotated offline).
    kblock=True (FP4 only, for weights): the codes in 64-byte K pieces, [pieces x rows x 64]
    (vq_mx_gemm tells the layouts apart by the tensor's rank)."""
    _dev(x, "x")
    rows, k = x.shape
    if kblock and fmt != "fp4":
        raise ValueError("K pieces hold FP4 codes only")
    code = (VQ_MXFP4_KBLOCK if kblock else _MX[fmt]) if fmt in _MX else -1
    if codes is None:
        row_bytes = k * _MX_BITS.get(fmt, 8) // 8
        shape = ((row_bytes + 63) // 64, rows, 64) if kblock else (rows, row_bytes)
        codes = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(max(vq_mx_scale_bytes(rows, k), 1), dtype=torch.uint8, device=x.device)
    if fmt in _MX:
        _buf(codes, "codes", int(_lib.vq_mx_code_bytes(rows, k, code)), x.device)
        _buf(scales, "scales", vq_mx_scale_bytes(rows, k), x.device)
    if had_block:
        if had_block != VQ_HAD_BLOCK:
            raise ValueError(f"had_block must be 0 or {VQ_HAD_BLOCK}")
        _check("vq_mx_quant_rotated", _lib.vq_mx_quant_rotated(
            _ptr(x), _DT.get(x.dtype, -1), rows, k, x.stride(0), code, exp_offset, _ptr(codes),
            _ptr(scales), _stream(x)))
        return codes, scales
    _check("vq_mx_quant", _lib.vq_mx_quant(
        _ptr(x), _DT.get(x.dtype, -1), rows, k, x.stride(0), code, _ptr(codes), _ptr(scales), _stream(x)))
    return codes, scales


def vq_mx_gemm(a: torch.Tensor, sa: torch.Tensor, fa: str, b: torch.Tensor, sb: torch.Tensor, fb: str = "fp4",
               out_dtype=torch.bfloat16, y=None, ws=None):
    """Y = dec(A) . dec(B)^T on the scaled MFMA; a, b are the MX code buffers of vq_mx_quant
    (b row-major [N x K/2], or in 64-byte K pieces [pieces x N x 64]).

    ws: None uses the zero-filled workspace kept per device and stream, a tensor of
    vq_mx_gemm_workspace_bytes() bytes is used as given, False runs without the split."""
    _dev(a, "a")
    m = a.shape[0]
    if not (isinstance(b, torch.Tensor) and b.dim() in (2, 3)):
        raise TypeError("b must be a 2-D (row-major) or 3-D (K pieces) CUDA (HIP) tensor of MX codes")
    kblock = b.dim() == 3
    n = b.shape[1] if kblock else b.shape[0]
    k = a.shape[1] * 8 // _MX_BITS[fa]
    if kblock and fb != "fp4":
        raise ValueError("K pieces hold FP4 codes only")
    fb_code = (VQ_MXFP4_KBLOCK if kblock else _MX[fb]) if fb in _MX else -1
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=a.device)
    _out2d(y, "y", m, n, a.device)
    if fa in _MX and fb in _MX:
        _in(a, "a", _U8, vq_mx_code_bytes(m, k, fa), a.device)
        _in(sa, "sa", _U8, vq_mx_scale_bytes(m, k), a.device)
        _in(b, "b", _U8, int(_lib.vq_mx_code_bytes(n, k, fb_code)), a.device)
        if kblock and tuple(b.shape) != ((k // 2 + 63) // 64, n, 64):
            raise ValueError(f"b in K pieces must be [{(k // 2 + 63) // 64} x N x 64] FP4 codes")
        _in(sb, "sb", _U8, vq_mx_scale_bytes(n, k), a.device)
    need = _mx_ws_bytes(m, n, k)
    ws = _workspace(need, a.device) if ws is None else ws
    if ws is not False:
        _buf(ws, "ws", need, a.device)
    _check("vq_mx_gemm", _lib.vq_mx_gemm(
        _ptr(a), _ptr(sa), _MX.get(fa, -1), _ptr(b), _ptr(sb), fb_code, m, n, k,
        _ptr(y), _DT.get(y.dtype, -1), y.stride(0), None if ws is False else _ptr(ws), _stream(a)))
    return y


def vq_calib_static_scale(x: torch.Tensor, bits: int, percentiles=CALIB_GRID, scale=None, hist=None):
    """Clipping-percentile search of a static per-tensor scale for x (asynchronous).

    Returns dict of device tensors: clips, scales (float32 [n]), mse (float64 [n]), best
    (int32 [1]), scale (float32 [1], ready for vq_quant_act(..., "static",
    static_scale=...)) and hist (the |x| histogram).
    """
    _dev(x, "x")
    rows, cols = x.shape
    n = len(percentiles)
    pct = (ctypes.c_double * n)(*percentiles)
    kw = dict(device=x.device)
    clips = torch.empty(n, dtype=torch.float32, **kw)
    scales = torch.empty(n, dtype=torch.float32, **kw)
    mse = torch.empty(n, dtype=torch.float64, **kw)
    best = torch.empty(1, dtype=torch.int32, **kw)
    if hist is None:
        hist = torch.empty(int(_lib.vq_calib_hist_bins()), dtype=torch.int32, **kw)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, **kw)
    _buf(hist, "hist", 4 * int(_lib.vq_calib_hist_bins()), x.device)
    _buf(scale, "scale", 4, x.device)
    _check("vq_calib_static_scale", _lib.vq_calib_static_scale(
        _ptr(x), _DT.get(x.dtype, -1), rows, cols, x.stride(0), bits, pct, n, _ptr(hist),
        _ptr(clips), _ptr(scales), _ptr(mse), _ptr(best), _ptr(scale), _stream(x)))
    return {"clips": clips, "scales": scales, "mse": mse, "best": best, "scale": scale, "hist": hist}


class ControlParams(ctypes.Structure):
    """vq_control_params: TDC skip and drift thresholds, skip limit, DMPQ widths and
    threshold, PDR outlier-ratio limit."""
    _fields_ = [("skip_threshold", ctypes.c_double), ("drift_threshold", ctypes.c_double),
                ("max_skips", ctypes.c_int32), ("bits_hi", ctypes.c_int32), ("bits_lo", ctypes.c_int32),
                ("route_threshold", ctypes.c_double), ("outlier_ratio_max", ctypes.c_double)]


CONTROL_STATE_BYTES = 16


def vq_control_state(device) -> torch.Tensor:
    """Zeroed per-block control state (consecutive skips, accumulated error)."""
    return torch.zeros(CONTROL_STATE_BYTES // 8, dtype=torch.float64, device=device)


def vq_step_control(state: torch.Tensor, params: ControlParams, delta_new=None, delta_old=None, x_prev=None,
                    y_prev=None, n_out_dev=None, channels: int = 0, ws=None, skip=None, bits=None, e=None,
                    gamma=None):
    """One block's decision at a step, on the device.  Returns (skip int32 [1], bits int32 [1],
    E float64 [1], Gamma float64 [1]); the state tensor is updated in place."""
    _buf(state, "state", CONTROL_STATE_BYTES, state.device)
    dev = state.device
    for t, name in ((delta_new, "delta_new"), (delta_old, "delta_old"), (x_prev, "x_prev"), (y_prev, "y_prev")):
        if t is not None:
            _dev(t, name)
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
    if (delta_new is None) != (delta_old is None) or (x_prev is None) != (y_prev is None):
        raise ValueError("deltas and the previous input/output come in pairs")
    for a, b, what in ((delta_new, delta_old, "deltas"), (x_prev, y_prev, "previous input/output")):
        if a is not None and (a.numel() != b.numel() or a.dtype != b.dtype):
            raise ValueError(f"the {what} must have the same size and dtype")
    nw = int(_lib.vq_control_workspace_elems())
    ws = torch.empty(nw, dtype=torch.float64, device=dev) if ws is None else ws
    _buf(ws, "ws", 8 * nw, dev)
    skip = torch.empty(1, dtype=torch.int32, device=dev) if skip is None else skip
    bits = torch.empty(1, dtype=torch.int32, device=dev) if bits is None else bits
    e = torch.empty(1, dtype=torch.float64, device=dev) if e is None else e
    gamma = torch.empty(1, dtype=torch.float64, device=dev) if gamma is None else gamma
    for t, name, nb in ((skip, "skip", 4), (bits, "bits", 4), (e, "e", 8), (gamma, "gamma", 8)):
        _buf(t, name, nb, dev)
    if n_out_dev is not None:
        _in(n_out_dev, "n_out_dev", _I32, 1, dev)
    dnew_dt = _DT.get(delta_new.dtype, -1) if delta_new is not None else 0
    xy_dt = _DT.get(x_prev.dtype, -1) if x_prev is not None else 0
    _check("vq_step_control", _lib.vq_step_control(
        _ptr(delta_new), _ptr(delta_old), dnew_dt, delta_new.numel() if delta_new is not None else 0,
        _ptr(x_prev), _ptr(y_prev), xy_dt, x_prev.numel() if x_prev is not None else 0,
        _ptr(n_out_dev), channels, ctypes.byref(params), _ptr(state), _ptr(ws), _ptr(skip), _ptr(bits), _ptr(e),
        _ptr(gamma), _stream(state)))
    return skip, bits, e, gamma


# ------------------------------------------------------------------ prepared calls

# Entry points that only enqueue work on a stream (their last argument).
_LAUNCHES = frozenset((
    "vq_pack_weights", "vq_quant_act", "vq_hadamard_block", "vq_qgemm_dequant", "vq_qgemm_dequant_noalloc",
    "vq_route_rel_l1", "vq_quant_residual", "vq_qgemm_dequant_residual", "vq_mx_quant", "vq_mx_quant_rotated",
    "vq_mx_gemm", "vq_gemm_dense", "vq_calib_static_scale", "vq_step_control",
))


class _Recorder:
    """Stands in for the library while a binding function runs under prepare(): the
    launch entry points are recorded instead of called; everything else passes through."""

    def __init__(self, lib):
        self._lib = lib
        self.calls = []

    def __getattr__(self, name):
        f = getattr(self._lib, name)
        if name not in _LAUNCHES:
            return f

        def record(*args):
            self.calls.append((name, f, args))
            return VQ_OK
        return record


def prepare(fn, *args, **kwargs):
    """Validate and marshal a binding call once, for loops that repeat it on the same
    tensors (the binding's checks cost more host time than the kernels of a small layer).

    Runs fn(*args, **kwargs) with the library's launches recorded instead of enqueued, and
    returns (launch, result): result is what fn returned (its outputs, allocated now if
    not given), and launch() enqueues the recorded launches again, unchanged, on torch's
    current stream of the device at that time (the device of fn's first device-tensor
    argument, else the current device).  fn may also be a caller's function that makes
    binding calls: all their launches are recorded, in order.  The tensors involved must stay alive and
    keep their storage and shape (launch() holds references to them; it reads their data
    anew at each call).  fn must be one of the binding's asynchronous entry points;
    prepare() is not thread-safe (it swaps the library handle for the duration of fn).
    """
    global _lib
    real = _lib
    rec = _Recorder(real)
    _lib = rec
    try:
        result = fn(*args, **kwargs)
    finally:
        _lib = real
    if not rec.calls:
        raise ValueError(f"{getattr(fn, '__name__', fn)} enqueues nothing through the library")
    tensors = [a for a in list(args) + list(kwargs.values()) if isinstance(a, torch.Tensor) and a.is_cuda]
    device = tensors[0].get_device() if tensors else torch.cuda.current_device()
    calls = rec.calls
    keep = (args, kwargs, result)

    def launch():
        st = torch._C._cuda_getCurrentRawStream(device)
        for name, f, a in calls:
            _check(name, f(*a[:-1], st))
    launch.keep = keep
    return launch, result
