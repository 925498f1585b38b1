"""Thin Python binding of libmbq (include/mbq.h) for PyTorch tensors.

Every function marshals tensor pointers, sizes and the current HIP stream into
the C ABI of the same name; all arithmetic runs in the library's HIP kernels.
If libmbq.so has not been built, importing works but every call raises
RuntimeError: there is no fallback implementation.

Build the library with ``python -m memory_bound_quantised_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmbq.so")

STATUS = {0: "MBQ_OK", -1: "MBQ_ERR_NULL", -2: "MBQ_ERR_SHAPE", -3: "MBQ_ERR_BITS",
          -4: "MBQ_ERR_ALIGN", -5: "MBQ_ERR_WORKSPACE", -6: "MBQ_ERR_PROGRAM",
          -7: "MBQ_ERR_HIP", -8: "MBQ_ERR_DEVICE", -9: "MBQ_ERR_TIMEOUT"}

EXPORTS = ["mbq_status_string", "mbq_last_hip_error", "mbq_version", "mbq_packed_bytes",
           "mbq_pack_weights", "mbq_unpack_weights", "mbq_pack_weights_inplace",
           "mbq_relayout_interleave_host", "mbq_quantize_act",
           "mbq_rmsnorm_quantize_act", "mbq_wrmsnorm_quantize_act", "mbq_swiglu_quantize_act",
           "mbq_linear_workspace_bytes", "mbq_w4a8_linear",
           "mbq_w6a8_linear", "mbq_linear_group_acc", "mbq_sequence_workspace_bytes",
           "mbq_sequence_prepare", "mbq_sequence_run", "mbq_sequence_check", "mbq_layer_sequence",
           "mbq_layer_sequence_unfused", "mbq_attention_workspace_bytes", "mbq_decode_attention",
           "mbq_stream_read", "mbq_linear_noalloc", "mbq_linear_prologue_workspace_bytes",
           "mbq_linear_prologue"]


class MbqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = f"{fn} failed: {STATUS.get(status, status)}"
        if status == -7 and _lib_handle is not None:
            msg += f" (hipError {_lib_handle.mbq_last_hip_error()})"
        super().__init__(msg)


class MbqOp(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("prologue", ctypes.c_int32), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("packed", ctypes.c_void_p), ("in_buf", ctypes.c_int32),
                ("out_buf", ctypes.c_int32), ("in_buf2", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("norm_w", ctypes.c_void_p)]


PRO_QUANT, PRO_RMSNORM_QUANT, PRO_WRMSNORM_QUANT, PRO_SWIGLU_QUANT = 0, 1, 2, 3


class MbqSequenceInfo(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint64), ("bits", ctypes.c_int32), ("M", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("lds_bytes", ctypes.c_int32), ("ws_bytes", ctypes.c_int64),
                ("plan_offset", ctypes.c_int64), ("full", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded libmbq; raises RuntimeError if it has not been built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m memory_bound_quantised_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.mbq_status_string.argtypes = [ctypes.c_int]
        L.mbq_status_string.restype = ctypes.c_char_p
        L.mbq_last_hip_error.restype = ctypes.c_int
        L.mbq_version.restype = ctypes.c_char_p
        L.mbq_packed_bytes.argtypes = [ctypes.c_int, I64, I64]
        L.mbq_packed_bytes.restype = I64
        L.mbq_pack_weights.argtypes = [ctypes.c_int, I64, I64, P, P, P, P]
        L.mbq_unpack_weights.argtypes = [ctypes.c_int, I64, I64, P, P, P, P]
        L.mbq_pack_weights_inplace.argtypes = [ctypes.c_int, I64, I64, P, I64, P]
        L.mbq_attention_workspace_bytes.argtypes = [I64, I64, I64, I64, I64]
        L.mbq_attention_workspace_bytes.restype = I64
        L.mbq_decode_attention.argtypes = [I64, I64, I64, I64, I64, I64, P, P, P, P, P, I64, P]
        L.mbq_relayout_interleave_host.argtypes = [ctypes.c_int, I64, I64, P, I64]
        L.mbq_quantize_act.argtypes = [I64, I64, P, P, P, P]
        L.mbq_rmsnorm_quantize_act.argtypes = [I64, I64, P, P, P, P]
        L.mbq_wrmsnorm_quantize_act.argtypes = [I64, I64, P, P, P, P, P]
        L.mbq_swiglu_quantize_act.argtypes = [I64, I64, P, P, P, P, P, P]
        L.mbq_linear_workspace_bytes.argtypes = [ctypes.c_int, I64, I64, I64]
        L.mbq_linear_workspace_bytes.restype = I64
        for fn in (L.mbq_w4a8_linear, L.mbq_w6a8_linear):
            fn.argtypes = [I64, I64, I64, P, P, P, P, P, I64, P]
        L.mbq_linear_group_acc.argtypes = [ctypes.c_int, ctypes.c_int, I64, I64, I64, P, P, P, P]
        L.mbq_sequence_workspace_bytes.argtypes = [P, I32, P, I32, I64]
        L.mbq_sequence_workspace_bytes.restype = I64
        L.mbq_layer_sequence.argtypes = [P, I32, P, P, I32, I64, P, I64, P]
        L.mbq_layer_sequence_unfused.argtypes = [P, I32, P, P, I32, I64, P, I64, P]
        L.mbq_sequence_prepare.argtypes = [P, I32, P, P, I32, I64, P, I64, P, P]
        L.mbq_sequence_run.argtypes = [P, P, P]
        L.mbq_sequence_check.argtypes = [P, P]
        L.mbq_stream_read.argtypes = [P, I64, P, P]
        L.mbq_linear_noalloc.argtypes = [ctypes.c_int, I64, I64, I64, P, P, P, P, P]
        L.mbq_linear_prologue_workspace_bytes.argtypes = [ctypes.c_int, I64, I64, I64]
        L.mbq_linear_prologue_workspace_bytes.restype = I64
        L.mbq_linear_prologue.argtypes = [ctypes.c_int, ctypes.c_int, I64, I64, I64, P, P, P, P, P, P, I64, P]
        for name in EXPORTS:
            if name not in ("mbq_status_string", "mbq_last_hip_error", "mbq_version",
                            "mbq_packed_bytes", "mbq_linear_workspace_bytes",
                            "mbq_sequence_workspace_bytes", "mbq_attention_workspace_bytes",
                            "mbq_linear_prologue_workspace_bytes"):
                getattr(L, name).restype = ctypes.c_int
        _lib_handle = L
    return _lib_handle


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise MbqError(fn, rc)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# ---------------------------------------------------------------- sizes

def packed_bytes(bits: int, N: int, K: int) -> int:
    v = lib().mbq_packed_bytes(bits, N, K)
    if v < 0:
        raise MbqError("mbq_packed_bytes", v)
    return v


def linear_workspace_bytes(bits: int, M: int, N: int, K: int) -> int:
    v = lib().mbq_linear_workspace_bytes(bits, M, N, K)
    if v < 0:
        raise MbqError("mbq_linear_workspace_bytes", v)
    return v


# ---------------------------------------------------------------- calls on torch tensors

def _empty(nbytes: int, device):
    import torch
    # 256-byte aligned by the caching allocator; at least one element
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _zeros(nbytes: int, device):
    import torch
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


def pack_weights(bits: int, w_canon, scales_f16, N: int, K: int, out=None):
    """Canonical codes (uint8 [N][K*bits/8]) + fp16 scales [N][K/128] -> packed uint8 tensor."""
    if out is None:
        out = _empty(packed_bytes(bits, N, K), w_canon.device)
    _check("mbq_pack_weights", lib().mbq_pack_weights(bits, N, K, _ptr(w_canon), _ptr(scales_f16),
                                                      _ptr(out), _stream()))
    return out


def pack_weights_inplace(bits: int, buf, N: int, K: int):
    """Re-lay in place: buf (uint8 device tensor of at least packed_bytes(bits, N, K)
    bytes) holds the canonical codes of the N rows followed by their fp16 scales;
    afterwards it holds the packed tiles.  Waits for the stream."""
    if buf.numel() * buf.element_size() < packed_bytes(bits, N, K):
        raise ValueError("buffer smaller than packed_bytes(bits, N, K)")
    _check("mbq_pack_weights_inplace", lib().mbq_pack_weights_inplace(
        bits, N, K, _ptr(buf), buf.numel() * buf.element_size(), _stream()))
    return buf


def relayout_interleave_host(bits: int, buf, N: int, K: int):
    """Test helper: the padding and row-block interleave steps of the in-place
    re-layout on a host numpy uint8 array (modified in place)."""
    import numpy as np
    assert isinstance(buf, np.ndarray) and buf.dtype == np.uint8 and buf.flags.c_contiguous
    _check("mbq_relayout_interleave_host", lib().mbq_relayout_interleave_host(
        bits, N, K, buf.ctypes.data, buf.nbytes))
    return buf


def attention_workspace_bytes(M: int, n_q: int, n_kv: int, D: int, P: int) -> int:
    v = lib().mbq_attention_workspace_bytes(M, n_q, n_kv, D, P)
    if v < 0:
        raise MbqError("mbq_attention_workspace_bytes", v)
    return v


def decode_attention(q, k_cache, v_cache, P: int, out=None, ws=None):
    """Split-prefix decode attention: q bf16 [M][n_q][D]; caches bf16 [n_kv][L][D]
    holding the M new tokens' keys and values at positions P .. P+M-1.  Token i
    attends to positions 0 .. P+i.  ws: a uint8 device tensor of at least
    attention_workspace_bytes(...) bytes (any contents, unless MBQ_ATTN_COMBINE=inline
    selects the in-launch combine: then zero-filled before its first use, and every
    call leaves its counters at zero); allocated here, zero-filled, when omitted."""
    import torch
    M, n_q, D = q.shape
    n_kv, L, D2 = k_cache.shape
    assert D2 == D and v_cache.shape == k_cache.shape
    if out is None:
        out = torch.empty((M, n_q, D), dtype=torch.bfloat16, device=q.device)
    need = attention_workspace_bytes(M, n_q, n_kv, D, P)
    if ws is None:
        ws = _zeros(need, q.device)
    _check("mbq_decode_attention", lib().mbq_decode_attention(
        M, n_q, n_kv, D, P, L, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(ws),
        ws.numel() * ws.element_size(), _stream()))
    return out


def unpack_weights(bits: int, packed, N: int, K: int):
    import torch
    canon = torch.empty((N, K * bits // 8), dtype=torch.uint8, device=packed.device)
    scales = torch.empty((N, K // 128), dtype=torch.float16, device=packed.device)
    _check("mbq_unpack_weights", lib().mbq_unpack_weights(bits, N, K, _ptr(packed), _ptr(canon),
                                                          _ptr(scales), _stream()))
    return canon, scales


def quantize_act(x_bf16, rmsnorm: bool = False, norm_w=None, up=None, h_out=None):
    """bf16 [M][K] -> (q int8 [M][K], s fp32 [M]) after the optional prologue:
    rmsnorm (weightless), norm_w (bf16 [K]: weighted RMSNorm), or up (bf16
    [M][K]: SwiGLU of x_bf16 as the gate; h_out receives the gated values)."""
    import torch
    M, K = x_bf16.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x_bf16.device)
    s = torch.empty((M,), dtype=torch.float32, device=x_bf16.device)
    L = lib()
    if up is not None:
        _check("mbq_swiglu_quantize_act", L.mbq_swiglu_quantize_act(
            M, K, _ptr(x_bf16), _ptr(up), _ptr(h_out) if h_out is not None else None, _ptr(q), _ptr(s),
            _stream()))
    elif norm_w is not None:
        _check("mbq_wrmsnorm_quantize_act", L.mbq_wrmsnorm_quantize_act(
            M, K, _ptr(x_bf16), _ptr(norm_w), _ptr(q), _ptr(s), _stream()))
    else:
        fn = L.mbq_rmsnorm_quantize_act if rmsnorm else L.mbq_quantize_act
        _check("mbq_quantize_act", fn(M, K, _ptr(x_bf16), _ptr(q), _ptr(s), _stream()))
    return q, s


def linear(bits: int, q, s, packed, N: int, ws=None, out=None):
    """y bf16 [M][N] = rescale(q x W^T); ws is a zero-initialised uint8 workspace (made if None)."""
    import torch
    M, K = q.shape
    need = linear_workspace_bytes(bits, M, N, K)
    if ws is None:
        ws = _zeros(need, q.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=q.device)
    fn = lib().mbq_w4a8_linear if bits == 4 else lib().mbq_w6a8_linear
    _check("mbq_w%da8_linear" % bits, fn(M, N, K, _ptr(q), _ptr(s), _ptr(packed), _ptr(out),
                                         _ptr(ws), ws.numel(), _stream()))
    return out


def linear_noalloc(bits: int, q, s, packed, N: int, out):
    """The linear on the library's own device scratch (mbq_linear_noalloc): no
    workspace; out is a caller-provided bf16 [M][N] tensor."""
    M, K = q.shape
    _check("mbq_linear_noalloc", lib().mbq_linear_noalloc(bits, M, N, K, _ptr(q), _ptr(s), _ptr(packed),
                                                          _ptr(out), _stream()))
    return out


def linear_prologue_workspace_bytes(bits: int, M: int, N: int, K: int) -> int:
    n = lib().mbq_linear_prologue_workspace_bytes(bits, M, N, K)
    if n < 0:
        raise MbqError("mbq_linear_prologue_workspace_bytes", n)
    return n


def linear_prologue(bits: int, x_bf16, packed, N: int, prologue: int = PRO_QUANT, up=None, norm_w=None,
                    ws=None, out=None):
    """The linear with the quantisation and its prologue inside it
    (mbq_linear_prologue): bf16 rows x [M][K] (the gate rows for SwiGLU, with
    up [M][K]; norm_w [K] for the weighted RMSNorm) -> bf16 y [M][N]."""
    import torch
    M, K = x_bf16.shape
    if ws is None:
        ws = _zeros(linear_prologue_workspace_bytes(bits, M, N, K), x_bf16.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x_bf16.device)
    _check("mbq_linear_prologue", lib().mbq_linear_prologue(
        bits, prologue, M, N, K, _ptr(x_bf16), _ptr(up) if up is not None else None,
        _ptr(norm_w) if norm_w is not None else None, _ptr(packed), _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def w4a8_linear(q, s, packed, N, ws=None, out=None):
    return linear(4, q, s, packed, N, ws, out)


def w6a8_linear(q, s, packed, N, ws=None, out=None):
    return linear(6, q, s, packed, N, ws, out)


FORM_DOT4, FORM_MFMA, FORM_ROWSET = 0, 1, 2


def linear_group_acc(bits: int, q, packed, N: int, form: int = FORM_MFMA):
    """Exact int32 group sums [M][N][K/128] through the product's tile code:
    form=FORM_MFMA (the whole-tile code of the linears and the walk), FORM_ROWSET (the
    linear's row-set form) or FORM_DOT4 (the v_dot4 tile, off the product's path)."""
    import torch
    M, K = q.shape
    acc = torch.empty((M, N, K // 128), dtype=torch.int32, device=q.device)
    _check("mbq_linear_group_acc", lib().mbq_linear_group_acc(bits, form, M, N, K, _ptr(q), _ptr(packed),
                                                              _ptr(acc), _stream()))
    return acc


def stream_read(buf, sink=None):
    """One pass of the HBM stream-read ceiling kernel over the uint8 device tensor
    buf (a multiple of 1 KiB); sink: a uint32/int32 device scalar (made if None)."""
    import torch
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    _check("mbq_stream_read", lib().mbq_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                                    _stream()))
    return sink


class LayerSequence:
    """A decode-step walk: an op list over bf16 buffers.

    ops: iterable of dicts with bits, prologue, N, K, packed (uint8 tensor),
    in_buf, out_buf, and in_buf2 (SwiGLU's up buffer) or norm_w (bf16 tensor
    [K], weighted RMSNorm) where the prologue needs them.  bufs: list of bf16
    tensors [M][width].  The workspace is allocated (zero-filled) once here
    unless ws (a zero-filled uint8 device tensor, possibly shared with another
    LayerSequence over the same op list) is given.  fused=True prepares the persistent
    kernel's plan once (mbq_sequence_prepare) and run() is one launch
    (mbq_sequence_run); fused=False runs mbq_layer_sequence_unfused.
    """

    def __init__(self, ops, bufs, M: int, fused: bool = True, ws=None):
        self.M = M
        self.fused = fused
        self.bufs = list(bufs)
        self._keep = [o["packed"] for o in ops] + [o["norm_w"] for o in ops if o.get("norm_w") is not None]
        arr = (MbqOp * len(ops))()
        for i, o in enumerate(ops):
            nw = o.get("norm_w")
            arr[i] = MbqOp(o["bits"], o["prologue"], o["N"], o["K"], o["packed"].data_ptr(),
                           o["in_buf"], o["out_buf"], o.get("in_buf2", -1), 0,
                           nw.data_ptr() if nw is not None else None)
        self._ops = arr
        self._n_ops = len(ops)
        self._widths = (ctypes.c_int64 * len(bufs))(*[b.shape[1] for b in bufs])
        self._ptrs = (ctypes.c_void_p * len(bufs))(*[b.data_ptr() for b in bufs])
        need = lib().mbq_sequence_workspace_bytes(arr, self._n_ops, self._widths, len(bufs), M)
        if need < 0:
            raise MbqError("mbq_sequence_workspace_bytes", need)
        if ws is not None and ws.numel() * ws.element_size() < need:
            raise ValueError(f"workspace of {ws.numel()} bytes, {need} needed")
        self.ws = _zeros(need, bufs[0].device) if ws is None else ws
        self.info = MbqSequenceInfo()
        if fused:
            _check("mbq_sequence_prepare",
                   lib().mbq_sequence_prepare(self._ops, self._n_ops, self._ptrs, self._widths,
                                              len(self.bufs), M, _ptr(self.ws), self.ws.numel(),
                                              _stream(), ctypes.byref(self.info)))

    def run(self):
        if self.fused:
            _check("mbq_sequence_run", lib().mbq_sequence_run(ctypes.byref(self.info), _ptr(self.ws),
                                                              _stream()))
        else:
            _check("mbq_layer_sequence_unfused",
                   lib().mbq_layer_sequence_unfused(self._ops, self._n_ops, self._ptrs, self._widths,
                                                    len(self.bufs), self.M, _ptr(self.ws),
                                                    self.ws.numel(), _stream()))

    def check(self):
        """Synchronise and raise if a bounded wait inside the fused walk gave up."""
        _check("mbq_sequence_check", lib().mbq_sequence_check(_ptr(self.ws), _stream()))
