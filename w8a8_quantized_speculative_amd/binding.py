"""Thin Python binding over libquasar.so (include/quasar.h).

Argument marshalling only: torch tensors are checked for dtype, shape and
device, their device pointers and torch's current HIP stream are handed to the
C ABI, and a non-OK status becomes an exception.  Every step of the verify path
runs in the library's HIP kernels; there is no Python or CPU fallback -- if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first; libquasar binds to the same one

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libquasar.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "quasar.h")

QUASAR_OK = 0
QUASAR_ERR_INVALID_ARG = 1
QUASAR_ERR_UNSUPPORTED = 2
QUASAR_ERR_WORKSPACE = 3
QUASAR_ERR_HIP = 4
QUASAR_ERR_INCOMPLETE = 5
QUASAR_WAIT_LDS = 1
QUASAR_WAIT_ROWS = 2
QUASAR_WAIT_PARTIALS = 4
QUASAR_WAIT_CHAIN = 8
QUASAR_MAX_M = 128
QUASAR_MAX_K = 65536
QUASAR_MAX_DRAFT = 63

_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_SIGNATURES = {
    "quasar_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "quasar_abi_version": (ctypes.c_int, []),
    "quasar_device_check": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32)]),
    "quasar_debug_force_wait_expiry": (None, [ctypes.c_int]),
    "quasar_workspace_header_bytes": (_SZ, []),
    "quasar_workspace_init": (ctypes.c_int, [_P, _SZ, _P]),
    "quasar_quantize_weights": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P]),
    "quasar_quantize_weights_gated": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P]),
    "quasar_w8a8_linear_swiglu_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "quasar_w8a8_linear_swiglu": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _SZ,
                                                 _P]),
    "quasar_quantize_activations": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P, _P]),
    "quasar_packed_weight_bytes": (_SZ, [_I64, _I64]),
    "quasar_w8a8_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "quasar_w8a8_linear": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _SZ, _P]),
    "quasar_w8a8_linear_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P]),
    "quasar_accept_workspace_bytes": (_SZ, [_I64, _I64, _I64]),
    "quasar_verify_accept": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, ctypes.c_float, _P, _P, _P,
                                            _P, _P, _P, _SZ, _P]),
    "quasar_lm_head_verify_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64]),
    "quasar_lm_head_verify": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P,
                                             ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                             _P]),
    "quasar_w8a8_kernel_name": (ctypes.c_char_p, [_I64, _I64, _I64]),
    "quasar_packed_weight_bytes_w4": (_SZ, [_I64, _I64]),
    "quasar_quantize_weights_w4": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _P, _P]),
    "quasar_w4a8_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "quasar_w4a8_linear": (ctypes.c_int, [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "quasar_w4a8_kernel_name": (ctypes.c_char_p, [_I64, _I64, _I64]),
    "quasar_stream_copy": (ctypes.c_int, [_P, _P, _SZ, _P]),
    "quasar_stream_read": (ctypes.c_int, [_P, _SZ, _P, _P]),
    "quasar_embed": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _P, _P]),
    "quasar_rmsnorm": (ctypes.c_int, [_P, _P, _P, _I64, _I64, ctypes.c_float, _P, _P]),
    "quasar_qk_rope_cache": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                            ctypes.c_float, ctypes.c_float, _P, _P, _P, _P]),
    "quasar_attention_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64]),
    "quasar_attention": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _P,
                                        _P, _SZ, _P]),
    "quasar_silu_mul": (ctypes.c_int, [_P, _I64, _I64, _P, _P]),
    "quasar_w8a8_chain_workspace_bytes": (_SZ, [_P, _I64, _I64]),
    "quasar_w8a8_chain": (ctypes.c_int, [_P, _P, _I64, _I64, _P, _SZ, _P]),
    "quasar_chain_verify_workspace_bytes": (_SZ, [_P, _I64, _I64, _I64]),
    "quasar_chain_verify": (ctypes.c_int, [_P, _P, _I64, _I64, _I64, _P, ctypes.c_float, _P, _P,
                                           _P, _P, _P, _P, _SZ, _P]),
    "quasar_w8a8_chain_kernel_name": (ctypes.c_char_p, [_I64]),
}

QUASAR_LINK_SWIGLU = 1


class ChainLink(ctypes.Structure):
    """struct quasar_chain_link (include/quasar.h)."""
    _fields_ = [("x", _P), ("s", _P), ("wq", _P), ("w_scale", _P), ("y", _P), ("acc_out", _P),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64), ("ldx", ctypes.c_int64),
                ("dep", ctypes.c_int32), ("flags", ctypes.c_uint32)]


assert ctypes.sizeof(ChainLink) == 80


class QuasarError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib().quasar_status_string(status).decode()}")


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m w8a8_quantized_speculative_amd.build)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(fn: str, status: int) -> None:
    if status != QUASAR_OK:
        raise QuasarError(fn, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, dtype, shape, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_bytes_linear(M: int, N: int, K: int) -> int:
    return int(lib().quasar_w8a8_workspace_bytes(M, N, K))


def workspace_bytes_accept(B: int, k: int, V: int) -> int:
    return int(lib().quasar_accept_workspace_bytes(B, k, V))


def new_workspace(nbytes: int, device=None) -> torch.Tensor:
    """A zero-filled device byte buffer for the *_workspace_bytes sizes (256-byte
    aligned): the flag header at its start must be zero before first use."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8,
                       device=device if device is not None else "cuda")


def workspace_init(workspace: torch.Tensor) -> None:
    """Zero a workspace's flag header with the library's kernel (graph-safe)."""
    _check("quasar_workspace_init", lib().quasar_workspace_init(
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))


def device_check():
    """Wait for the device, read and clear its status word: (status, detail bits)."""
    bits = ctypes.c_uint32(0)
    st = lib().quasar_device_check(ctypes.byref(bits))
    return int(st), int(bits.value)


def force_wait_expiry(on: bool) -> None:
    """Test hook: every bounded wait of kernels launched while on gives up."""
    lib().quasar_debug_force_wait_expiry(1 if on else 0)


def w8a8_kernel_name(M: int, N: int, K: int) -> str:
    """Profiler name of the kernel(s) quasar_w8a8_linear launches for M x N x K."""
    return lib().quasar_w8a8_kernel_name(M, N, K).decode()


def quasar_stream_read(src: torch.Tensor, sink: torch.Tensor) -> None:
    """Diagnostic read-only stream of src's bytes (sink: 1024 int32 words)."""
    _check("quasar_stream_read", lib().quasar_stream_read(
        _ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream()))


def quasar_stream_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    """Diagnostic plain device copy of src's bytes into dst (same byte size)."""
    nbytes = src.numel() * src.element_size()
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous GPU tensors")
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must hold the same number of bytes")
    _check("quasar_stream_copy", lib().quasar_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream()))


# ------------------------------------------------------------------ calls
def packed_weight_bytes(N: int, K: int) -> int:
    return int(lib().quasar_packed_weight_bytes(N, K))


class PackedWeights:
    """Tile-packed INT8 (bits = 8) or 4-bit (bits = 4) codes of an N x K linear
    (layouts in include/quasar.h)."""

    def __init__(self, codes: torch.Tensor, N: int, K: int, bits: int = 8):
        self.codes, self.N, self.K, self.bits = codes, N, K, bits

    def data_ptr(self):
        return self.codes.data_ptr()


def quasar_quantize_weights(w: torch.Tensor, s: torch.Tensor):
    """W [N, K] bf16, s [K] f32 -> (PackedWeights, w_scale f32 [N])."""
    N, K = w.shape
    _need(w, torch.bfloat16, (N, K), "w")
    _need(s, torch.float32, (K,), "s")
    nbytes = packed_weight_bytes(N, K) if N > 0 else 0
    codes = torch.empty((max(nbytes, 16),), dtype=torch.int8, device=w.device)
    wq = PackedWeights(codes, N, K)
    sw = torch.empty((N,), dtype=torch.float32, device=w.device)
    _check("quasar_quantize_weights", lib().quasar_quantize_weights(
        _ptr(w), _ptr(s), N, K, _ptr(wq), _ptr(sw), _stream()))
    return wq, sw


def quasar_quantize_weights_gated(w: torch.Tensor, s: torch.Tensor):
    """[W_gate; W_up] [2I, K] bf16, s [K] f32 -> (PackedWeights in the gated row
    order, w_scale f32 [2I] in that order), for quasar_w8a8_linear_swiglu."""
    N, K = w.shape
    _need(w, torch.bfloat16, (N, K), "w")
    _need(s, torch.float32, (K,), "s")
    nbytes = packed_weight_bytes(N, K) if N > 0 else 0
    codes = torch.empty((max(nbytes, 16),), dtype=torch.int8, device=w.device)
    wq = PackedWeights(codes, N, K)
    sw = torch.empty((N,), dtype=torch.float32, device=w.device)
    _check("quasar_quantize_weights_gated", lib().quasar_quantize_weights_gated(
        _ptr(w), _ptr(s), N, K, _ptr(wq), _ptr(sw), _stream()))
    return wq, sw


def quasar_quantize_activations(x: torch.Tensor, s: torch.Tensor, want_xs: bool = False):
    """X [M, K] bf16 -> (qx int8 [M, K], x_scale f32 [M], xs f32 [M, K] or None)."""
    M, K = x.shape
    _need(x, torch.bfloat16, (M, K), "x")
    _need(s, torch.float32, (K,), "s")
    qx = torch.empty((M, K), dtype=torch.int8, device=x.device)
    sx = torch.empty((M,), dtype=torch.float32, device=x.device)
    xs = torch.empty((M, K), dtype=torch.float32, device=x.device) if want_xs else None
    _check("quasar_quantize_activations", lib().quasar_quantize_activations(
        _ptr(x), _ptr(s), M, K, _ptr(qx), _ptr(sx), _ptr(xs), _stream()))
    return qx, sx, xs


def quasar_w8a8_linear(x: torch.Tensor, s: torch.Tensor, wq: PackedWeights, w_scale: torch.Tensor,
                       out: torch.Tensor | None = None, acc_out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y [M, N] bf16 = dequant(quant(X diag(s)) @ W8^T) for X [M, K] bf16."""
    M, K = x.shape
    N = wq.N
    if not isinstance(wq, PackedWeights) or wq.K != K or wq.bits != 8:
        raise ValueError("wq must be the INT8 PackedWeights of a linear with the same K")
    _need(x, torch.bfloat16, (M, K), "x")
    _need(s, torch.float32, (K,), "s")
    _need(w_scale, torch.float32, (N,), "w_scale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, (M, N), "out")
    if acc_out is not None:
        _need(acc_out, torch.int32, (M, N), "acc_out")
    need = workspace_bytes_linear(M, N, K)
    if workspace is None and need > 0:
        workspace = new_workspace(need, x.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("quasar_w8a8_linear", lib().quasar_w8a8_linear(
        _ptr(x), _ptr(s), _ptr(wq), _ptr(w_scale), M, N, K, _ptr(out), _ptr(acc_out),
        _ptr(workspace), nbytes, _stream()))
    return out


def quasar_w8a8_linear_noalloc(x: torch.Tensor, s: torch.Tensor, wq: PackedWeights,
                               w_scale: torch.Tensor, out: torch.Tensor | None = None,
                               acc_out: torch.Tensor | None = None) -> torch.Tensor:
    """quasar_w8a8_linear without a workspace (the library's own scratch)."""
    M, K = x.shape
    N = wq.N
    _need(x, torch.bfloat16, (M, K), "x")
    _need(s, torch.float32, (K,), "s")
    _need(w_scale, torch.float32, (N,), "w_scale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, (M, N), "out")
    if acc_out is not None:
        _need(acc_out, torch.int32, (M, N), "acc_out")
    _check("quasar_w8a8_linear_noalloc", lib().quasar_w8a8_linear_noalloc(
        _ptr(x), _ptr(s), _ptr(wq), _ptr(w_scale), M, N, K, _ptr(out), _ptr(acc_out), _stream()))
    return out


def workspace_bytes_linear_swiglu(M: int, N: int, K: int) -> int:
    return int(lib().quasar_w8a8_linear_swiglu_workspace_bytes(M, N, K))


def quasar_w8a8_linear_swiglu(x: torch.Tensor, s: torch.Tensor, wq: PackedWeights,
                              w_scale: torch.Tensor, out: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """act [M, N/2] bf16 = silu(gate) * up of the gate_up linear, for weights from
    quasar_quantize_weights_gated."""
    M, K = x.shape
    N = wq.N
    if not isinstance(wq, PackedWeights) or wq.K != K or wq.bits != 8:
        raise ValueError("wq must be the INT8 PackedWeights of a linear with the same K")
    _need(x, torch.bfloat16, (M, K), "x")
    _need(s, torch.float32, (K,), "s")
    _need(w_scale, torch.float32, (N,), "w_scale")
    if out is None:
        out = torch.empty((M, N // 2), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, (M, N // 2), "out")
    need = workspace_bytes_linear_swiglu(M, N, K)
    if workspace is None and need > 0:
        workspace = new_workspace(need, x.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("quasar_w8a8_linear_swiglu", lib().quasar_w8a8_linear_swiglu(
        _ptr(x), _ptr(s), _ptr(wq), _ptr(w_scale), M, N, K, _ptr(out), _ptr(workspace), nbytes,
        _stream()))
    return out


def quasar_verify_accept(logits: torch.Tensor, draft: torch.Tensor | None, temperature: float = 0.0,
                         uniforms: torch.Tensor | None = None, want_argmax: bool = False,
                         want_p_draft: bool = False, workspace: torch.Tensor | None = None):
    """logits [B, k+1, V] bf16, draft [B, k] int32 ->
    (accept_len int32 [B], next_token int32 [B], argmax [B, k+1] or None, p_draft [B, k] or None)."""
    B, kp1, V = logits.shape
    k = kp1 - 1
    _need(logits, torch.bfloat16, (B, kp1, V), "logits")
    if k > 0 or draft is not None:
        _need(draft, torch.int32, (B, k), "draft")
    if uniforms is not None:
        _need(uniforms, torch.float32, (B, kp1), "uniforms")
    dev = logits.device
    acc_len = torch.empty((B,), dtype=torch.int32, device=dev)
    nxt = torch.empty((B,), dtype=torch.int32, device=dev)
    g = torch.empty((B, kp1), dtype=torch.int32, device=dev) if want_argmax else None
    pd = torch.empty((B, k), dtype=torch.float32, device=dev) if want_p_draft else None
    if workspace is None:
        workspace = new_workspace(workspace_bytes_accept(B, k, V), dev)
    nbytes = workspace.numel() * workspace.element_size()
    _check("quasar_verify_accept", lib().quasar_verify_accept(
        _ptr(logits), _ptr(draft), B, k, V, float(temperature), _ptr(uniforms), _ptr(acc_len),
        _ptr(nxt), _ptr(g), _ptr(pd), _ptr(workspace), nbytes, _stream()))
    return acc_len, nxt, g, pd


def workspace_bytes_lm_head_verify(B: int, k: int, V: int, K: int) -> int:
    return int(lib().quasar_lm_head_verify_workspace_bytes(B, k, V, K))


def quasar_lm_head_verify(x: torch.Tensor, s: torch.Tensor, wq: PackedWeights,
                          w_scale: torch.Tensor, B: int, draft: torch.Tensor | None,
                          temperature: float = 0.0, uniforms: torch.Tensor | None = None,
                          want_argmax: bool = False, want_p_draft: bool = False,
                          logits: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None,
                          accept_len: torch.Tensor | None = None,
                          next_token: torch.Tensor | None = None):
    """LM head over x [B*(k+1), K] bf16, then the accept step on its logits ->
    (logits [B, k+1, V] bf16, accept_len [B], next_token [B], argmax or None,
    p_draft or None)."""
    M, K = x.shape
    if B <= 0 or M % B:
        raise ValueError("x must hold B * (k+1) rows")
    kp1 = M // B
    k = kp1 - 1
    V = wq.N
    if not isinstance(wq, PackedWeights) or wq.K != K or wq.bits != 8:
        raise ValueError("wq must be the INT8 PackedWeights of a linear with the same K")
    _need(x, torch.bfloat16, (M, K), "x")
    _need(s, torch.float32, (K,), "s")
    _need(w_scale, torch.float32, (V,), "w_scale")
    if k > 0 or draft is not None:
        _need(draft, torch.int32, (B, k), "draft")
    if uniforms is not None:
        _need(uniforms, torch.float32, (B, kp1), "uniforms")
    dev = x.device
    if logits is None:
        logits = torch.empty((B, kp1, V), dtype=torch.bfloat16, device=dev)
    _need(logits, torch.bfloat16, (B, kp1, V), "logits")
    acc_len = torch.empty((B,), dtype=torch.int32, device=dev) if accept_len is None else accept_len
    nxt = torch.empty((B,), dtype=torch.int32, device=dev) if next_token is None else next_token
    _need(acc_len, torch.int32, (B,), "accept_len")
    _need(nxt, torch.int32, (B,), "next_token")
    g = torch.empty((B, kp1), dtype=torch.int32, device=dev) if want_argmax else None
    pd = torch.empty((B, k), dtype=torch.float32, device=dev) if want_p_draft else None
    if workspace is None:
        workspace = new_workspace(workspace_bytes_lm_head_verify(B, k, V, K), dev)
    nbytes = workspace.numel() * workspace.element_size()
    _check("quasar_lm_head_verify", lib().quasar_lm_head_verify(
        _ptr(x), _ptr(s), _ptr(wq), _ptr(w_scale), B, k, V, K, _ptr(draft), float(temperature),
        _ptr(uniforms), _ptr(logits), _ptr(acc_len), _ptr(nxt), _ptr(g), _ptr(pd),
        _ptr(workspace), nbytes, _stream()))
    return logits, acc_len, nxt, g, pd


# ------------------------------------------------------- 4-bit weight variant
def packed_weight_bytes_w4(N: int, K: int) -> int:
    return int(lib().quasar_packed_weight_bytes_w4(N, K))


def w4a8_kernel_name(M: int, N: int, K: int) -> str:
    return lib().quasar_w4a8_kernel_name(M, N, K).decode()


def quasar_quantize_weights_w4(w: torch.Tensor, s: torch.Tensor):
    """W [N, K] bf16, s [K] f32 (K % 128 == 0) -> (4-bit PackedWeights, w_scale f32 [N])."""
    N, K = w.shape
    _need(w, torch.bfloat16, (N, K), "w")
    _need(s, torch.float32, (K,), "s")
    nbytes = packed_weight_bytes_w4(N, K) if N > 0 else 0
    codes = torch.empty((max(nbytes, 16),), dtype=torch.int8, device=w.device)
    wq = PackedWeights(codes, N, K, bits=4)
    sw = torch.empty((N,), dtype=torch.float32, device=w.device)
    _check("quasar_quantize_weights_w4", lib().quasar_quantize_weights_w4(
        _ptr(w), _ptr(s), N, K, _ptr(wq), _ptr(sw), _stream()))
    return wq, sw


def workspace_bytes_w4(M: int, N: int, K: int) -> int:
    return int(lib().quasar_w4a8_workspace_bytes(M, N, K))


def quasar_w4a8_linear(x: torch.Tensor, s: torch.Tensor, wq: PackedWeights, w_scale: torch.Tensor,
                       out: torch.Tensor | None = None, acc_out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Y [M, N] bf16 = dequant(quant(X diag(s)) @ W4^T) for X [M, K] bf16, M <= 96."""
    M, K = x.shape
    N = wq.N
    if not isinstance(wq, PackedWeights) or wq.K != K or wq.bits != 4:
        raise ValueError("wq must be the 4-bit PackedWeights of a linear with the same K")
    _need(x, torch.bfloat16, (M, K), "x")
    _need(s, torch.float32, (K,), "s")
    _need(w_scale, torch.float32, (N,), "w_scale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, (M, N), "out")
    if acc_out is not None:
        _need(acc_out, torch.int32, (M, N), "acc_out")
    need = workspace_bytes_w4(M, N, K)
    if workspace is None and need > 0:
        workspace = new_workspace(need, x.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("quasar_w4a8_linear", lib().quasar_w4a8_linear(
        _ptr(x), _ptr(s), _ptr(wq), _ptr(w_scale), M, N, K, _ptr(out), _ptr(acc_out),
        _ptr(workspace), nbytes, _stream()))
    return out


# ------------------------------------------------- decoder steps around the linears
def quasar_embed(tokens: torch.Tensor, table: torch.Tensor, out: torch.Tensor | None = None):
    """tokens int32 [M], table bf16 [V, H] -> h f32 [M, H]."""
    M = tokens.numel()
    V, H = table.shape
    _need(tokens, torch.int32, (M,), "tokens")
    _need(table, torch.bfloat16, (V, H), "table")
    if out is None:
        out = torch.empty((M, H), dtype=torch.float32, device=table.device)
    _need(out, torch.float32, (M, H), "out")
    _check("quasar_embed", lib().quasar_embed(_ptr(tokens), _ptr(table), M, V, H, _ptr(out),
                                              _stream()))
    return out


def quasar_rmsnorm(h: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
                   delta: torch.Tensor | None = None, out: torch.Tensor | None = None):
    """h f32 [M, H] (updated in place by += delta when given) -> bf16 [M, H]."""
    M, H = h.shape
    _need(h, torch.float32, (M, H), "h")
    _need(gamma, torch.float32, (H,), "gamma")
    if delta is not None:
        _need(delta, torch.bfloat16, (M, H), "delta")
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=h.device)
    _need(out, torch.bfloat16, (M, H), "out")
    _check("quasar_rmsnorm", lib().quasar_rmsnorm(_ptr(h), _ptr(delta), _ptr(gamma), M, H, eps,
                                                  _ptr(out), _stream()))
    return out


def quasar_qk_rope_cache(qkv: torch.Tensor, q_gamma: torch.Tensor, k_gamma: torch.Tensor,
                         k_cache: torch.Tensor, v_cache: torch.Tensor, B: int, Hq: int, pos0: int,
                         rope_base: float = 1e6, eps: float = 1e-6,
                         q_out: torch.Tensor | None = None):
    """qkv bf16 [B*T, (Hq + 2 Hkv) D]; caches bf16 [B, Hkv, Lmax, D] -> q bf16 [B*T, Hq D]."""
    Bc, Hkv, Lmax, D = k_cache.shape
    M = qkv.shape[0]
    T = M // max(B, 1)
    if Bc != B or T * B != M:
        raise ValueError("qkv rows must be B*T and the caches' first dimension B")
    _need(qkv, torch.bfloat16, (M, (Hq + 2 * Hkv) * D), "qkv")
    _need(q_gamma, torch.float32, (D,), "q_gamma")
    _need(k_gamma, torch.float32, (D,), "k_gamma")
    _need(k_cache, torch.bfloat16, (B, Hkv, Lmax, D), "k_cache")
    _need(v_cache, torch.bfloat16, (B, Hkv, Lmax, D), "v_cache")
    if q_out is None:
        q_out = torch.empty((M, Hq * D), dtype=torch.bfloat16, device=qkv.device)
    _need(q_out, torch.bfloat16, (M, Hq * D), "q_out")
    _check("quasar_qk_rope_cache", lib().quasar_qk_rope_cache(
        _ptr(qkv), _ptr(q_gamma), _ptr(k_gamma), B, T, Hq, Hkv, D, pos0, Lmax, rope_base, eps,
        _ptr(q_out), _ptr(k_cache), _ptr(v_cache), _stream()))
    return q_out


def workspace_bytes_attention(B: int, T: int, Hq: int, Hkv: int, pos0: int) -> int:
    return int(lib().quasar_attention_workspace_bytes(B, T, Hq, Hkv, pos0))


def quasar_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, Hq: int,
                     pos0: int, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None):
    """q bf16 [B*T, Hq D], caches bf16 [B, Hkv, Lmax, D] -> bf16 [B*T, Hq D]."""
    B, Hkv, Lmax, D = k_cache.shape
    M = q.shape[0]
    T = M // max(B, 1)
    if T * B != M:
        raise ValueError("q rows must be B*T")
    _need(q, torch.bfloat16, (M, Hq * D), "q")
    _need(k_cache, torch.bfloat16, (B, Hkv, Lmax, D), "k_cache")
    _need(v_cache, torch.bfloat16, (B, Hkv, Lmax, D), "v_cache")
    if out is None:
        out = torch.empty((M, Hq * D), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, (M, Hq * D), "out")
    need = workspace_bytes_attention(B, T, Hq, Hkv, pos0)
    if workspace is None:
        workspace = new_workspace(need, q.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check("quasar_attention", lib().quasar_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), B, T, Hq, Hkv, D, pos0, Lmax, _ptr(out),
        _ptr(workspace), nbytes, _stream()))
    return out


def quasar_silu_mul(gate_up: torch.Tensor, out: torch.Tensor | None = None):
    """gate_up bf16 [M, 2I] -> bf16 [M, I] = silu(gate) * up."""
    M, I2 = gate_up.shape
    if I2 % 2:
        raise ValueError("gate_up must have an even number of columns")
    _need(gate_up, torch.bfloat16, (M, I2), "gate_up")
    if out is None:
        out = torch.empty((M, I2 // 2), dtype=torch.bfloat16, device=gate_up.device)
    _need(out, torch.bfloat16, (M, I2 // 2), "out")
    _check("quasar_silu_mul", lib().quasar_silu_mul(_ptr(gate_up), M, I2 // 2, _ptr(out), _stream()))
    return out


class Chain:
    """A list of W8A8 linears over one M-token window, run as one launch
    (quasar_w8a8_chain), or with the accept step after its last link, the LM
    head (quasar_chain_verify).  Links are added once; finalize() makes the
    host array and its device copy, which later runs reuse (the tensors passed
    to add() are kept alive by this object)."""

    def __init__(self, M: int, device=None):
        self.M = int(M)
        self.device = device if device is not None else "cuda"
        self.links = []
        self._keep = []
        self.host = None
        self.dev = None
        self.workspace = None

    def add(self, x: torch.Tensor, s: torch.Tensor, wq, w_scale: torch.Tensor, y: torch.Tensor,
            dep: int = -1, swiglu: bool = False, acc_out: torch.Tensor | None = None) -> int:
        """Append a link; returns its index.  x is [M, K] bf16 with unit column
        stride (a column slice of an earlier link's y is fine: its row stride is
        passed as ldx); y is [M, N] bf16 ([M, N/2] with swiglu), contiguous."""
        if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[0] != self.M or x.stride(1) != 1:
            raise ValueError("x must be a [M, K] bf16 matrix with unit column stride")
        K = x.shape[1]
        N = wq.N
        _need(s, torch.float32, (K,), "s")
        _need(w_scale, torch.float32, (N,), "w_scale")
        _need(y, torch.bfloat16, (self.M, N // 2 if swiglu else N), "y")
        if acc_out is not None:
            _need(acc_out, torch.int32, (self.M, N), "acc_out")
        lk = ChainLink(x.data_ptr(), s.data_ptr(), wq.data_ptr(), w_scale.data_ptr(), y.data_ptr(),
                       None if acc_out is None else acc_out.data_ptr(), N, K, x.stride(0),
                       int(dep), QUASAR_LINK_SWIGLU if swiglu else 0)
        self.links.append(lk)
        self._keep.append((x, s, wq, w_scale, y, acc_out))
        self.host = None
        return len(self.links) - 1

    def finalize(self):
        n = len(self.links)
        self.host = (ChainLink * max(n, 1))(*self.links)
        raw = torch.frombuffer(bytearray(bytes(self.host)), dtype=torch.uint8)
        self.dev = raw.to(self.device)
        need = int(lib().quasar_w8a8_chain_workspace_bytes(ctypes.cast(self.host, _P), n, self.M))
        if n and need == 0:
            raise QuasarError("quasar_w8a8_chain_workspace_bytes", QUASAR_ERR_INVALID_ARG)
        # a zero-filled workspace of this chain's own (its exchange areas depend on the links)
        self.workspace = new_workspace(need, self.device)
        return self

    def run(self, workspace: torch.Tensor | None = None) -> None:
        if self.host is None:
            self.finalize()
        ws = self.workspace if workspace is None else workspace
        _check("quasar_w8a8_chain", lib().quasar_w8a8_chain(
            ctypes.cast(self.host, _P), _ptr(self.dev), len(self.links), self.M, _ptr(ws),
            ws.numel() * ws.element_size(), _stream()))

    def verify_workspace(self, B: int, k: int) -> torch.Tensor:
        if self.host is None:
            self.finalize()
        need = int(lib().quasar_chain_verify_workspace_bytes(ctypes.cast(self.host, _P),
                                                              len(self.links), B, k))
        if need == 0:
            raise QuasarError("quasar_chain_verify_workspace_bytes", QUASAR_ERR_INVALID_ARG)
        return new_workspace(need, self.device)

    def run_verify(self, B: int, k: int, draft: torch.Tensor | None, temperature: float = 0.0,
                   uniforms: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                   want_argmax: bool = False, want_p_draft: bool = False, out=None):
        """The chain, then the accept step on its last link's logits.  Returns
        (accept_len [B], next_token [B], argmax [B, k+1] or None, p_draft [B, k] or None)."""
        if self.host is None:
            self.finalize()
        if workspace is None:
            if getattr(self, "_verify_ws", None) is None or self._verify_key != (B, k):
                self._verify_ws, self._verify_key = self.verify_workspace(B, k), (B, k)
            workspace = self._verify_ws
        dev = self.device
        if out is None:
            acc = torch.empty((B,), dtype=torch.int32, device=dev)
            nxt = torch.empty((B,), dtype=torch.int32, device=dev)
            g = torch.empty((B, k + 1), dtype=torch.int32, device=dev) if want_argmax else None
            pd = torch.empty((B, k), dtype=torch.float32, device=dev) if want_p_draft else None
        else:
            acc, nxt, g, pd = out
        if draft is not None:
            _need(draft, torch.int32, (B, k), "draft")
        if uniforms is not None:
            _need(uniforms, torch.float32, (B, k + 1), "uniforms")
        _check("quasar_chain_verify", lib().quasar_chain_verify(
            ctypes.cast(self.host, _P), _ptr(self.dev), len(self.links), B, k, _ptr(draft),
            float(temperature), _ptr(uniforms), _ptr(acc), _ptr(nxt), _ptr(g), _ptr(pd),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream()))
        return acc, nxt, g, pd


def chain_kernel_name(M: int) -> str:
    return lib().quasar_w8a8_chain_kernel_name(M).decode()
