"""ctypes binding of libbsb.so (the gfx950 HIP kernels behind include/bsb.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library. PyTorch provides device memory and the current HIP
stream; tensors are passed as raw device pointers. There is no fallback: if
the library is not built, importing this module's functions raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbsb.so")

BSB_OUT_BF16, BSB_OUT_FP32 = 0, 1
BSB_FP8_OCP, BSB_FP8_FNUZ = 0, 1
STATUS = {0: "BSB_OK", 1: "BSB_ERR_INVALID_ARG", 2: "BSB_ERR_UNSUPPORTED_DEVICE",
          3: "BSB_ERR_MISALIGNED", 4: "BSB_ERR_LAUNCH"}

_c_p = ctypes.c_void_p
_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int

_SIGNATURES = {
    "bsb_quantize_act": [_c_p, _c_i64, _c_i64, _c_p, _c_p, _c_p],
    "bsb_gemm_w8a8_g128": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_int, _c_p],
    "bsb_repack_weights_mfma": [_c_p, _c_i64, _c_i64, _c_p, _c_p],
    "bsb_grouped_gemm_w8a8_g128_packed": [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                          _c_i64, _c_p, _c_int, _c_p],
    "bsb_gemm_w8a8_g128_packed": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_int,
                                  _c_p],
    "bsb_gemm_w8a8_channel": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_int,
                              _c_p],
    "bsb_grouped_gemm_w8a8_g128": [_c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64,
                                   _c_p, _c_int, _c_p],
    "bsb_grouped_gemm_w8a8_g128_gather": [_c_p, _c_p, _c_p, _c_i64, _c_p, _c_p, _c_p, _c_i64,
                                          _c_i64, _c_i64, _c_i64, _c_p, _c_int, _c_p],
    "bsb_decode_fp8_block": [_c_p, _c_p, _c_i64, _c_i64, _c_int, _c_p, _c_p, _c_p],
    "bsb_dequant_fp8_block_bf16": [_c_p, _c_p, _c_i64, _c_i64, _c_int, _c_p, _c_p],
    "bsb_decode_fp8_block_packed": [_c_p, _c_p, _c_i64, _c_i64, _c_int, _c_p, _c_p, _c_p],
    "bsb_gemm_w8a16_g128": [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_int, _c_p],
    "bsb_gemm_bf16": [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_int, _c_p],
    "bsb_decode_mxfp4": [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p],
    "bsb_decode_mxfp4_packed": [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p],
    "bsb_gemm_w8a8_g128_partials": [_c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p],
    "bsb_gather_rows": [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_p, _c_p, _c_p],
    "bsb_moe_combine": [_c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_p],
    "bsb_kv_cache_write": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_p,
                           _c_p, _c_p, _c_p, _c_p],
    "bsb_attention_decode_int8kv": [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                    _c_i64, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_int, _c_p],
    "bsb_attention_chunk_int8kv": [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64,
                                   _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_int,
                                   _c_p],
    "bsb_attention_decode_int8kv_noalloc": [_c_p, _c_p, _c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64,
                                            _c_i64, _c_i64, _c_i64, _c_i64, _c_p, _c_int, _c_p],
    "bsb_probe_mfma_i8": [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p],
    "bsb_probe_mfma_i8_epilogue": [_c_p, _c_p, _c_i64, _c_i64, _c_p, _c_p],
    "bsb_probe_hbm_read": [_c_p, _c_i64, _c_p, _c_p],
    "bsb_probe_hbm_copy": [_c_p, _c_p, _c_i64, _c_p],
    "bsb_kv_cache_write_bf16": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                _c_p, _c_p, _c_p],
    "bsb_attention_decode_bf16kv": [_c_p, _c_p, _c_p, _c_p, _c_i64, _c_i64, _c_i64, _c_i64,
                                    _c_i64, _c_i64, _c_p, _c_i64, _c_p, _c_int, _c_p],
}
EXPORTED = tuple(_SIGNATURES) + ("bsb_status_string", "bsb_abi_version",
                                 "bsb_attention_workspace_bytes")

_lib = None


def lib() -> ctypes.CDLL:
    """Load libbsb.so once (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_scaled_bit_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = _c_int
        L.bsb_status_string.argtypes = [_c_int]
        L.bsb_status_string.restype = ctypes.c_char_p
        L.bsb_abi_version.argtypes = []
        L.bsb_abi_version.restype = _c_int
        L.bsb_attention_workspace_bytes.argtypes = [_c_i64, _c_i64, _c_i64]
        L.bsb_attention_workspace_bytes.restype = _c_i64
        _lib = L
    return _lib


class BsbError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {lib().bsb_status_string(status).decode()}")


def _check(status: int, fn: str) -> None:
    if status != 0:
        raise BsbError(status, fn)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: torch.Tensor, name: str, dtypes, shape=None, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF16_BITS = (torch.bfloat16, torch.int16, torch.uint16)


def quantize_act(x: torch.Tensor, q: Optional[torch.Tensor] = None,
                 sa: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """BF16 activations [M,K] -> (q int8 [M,K], sa float32 [M])."""
    _need(x, "x", _BF16_BITS)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    dev = x.device
    q = torch.empty((M, K), dtype=torch.int8, device=dev) if q is None else q
    sa = torch.empty((M,), dtype=torch.float32, device=dev) if sa is None else sa
    _need(q, "q", (torch.int8,), (M, K), dev)
    _need(sa, "sa", (torch.float32,), (M,), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_quantize_act(_ptr(x), M, K, _ptr(q), _ptr(sa), _stream(dev)),
               "bsb_quantize_act")
    return q, sa


def _out_code(dtype) -> int:
    if dtype == torch.bfloat16:
        return BSB_OUT_BF16
    if dtype == torch.float32:
        return BSB_OUT_FP32
    raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")


def gemm_w8a8_g128(q: torch.Tensor, sa: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
                   out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [M,N] = W8A8 per-group-128 GEMM of q [M,K] (scales sa [M]) with qw [N,K] (scales sw [N,K/128])."""
    _need(q, "q", (torch.int8,))
    if q.dim() != 2 or qw.dim() != 2:
        raise ValueError("q [M,K] and qw [N,K] required")
    M, K = q.shape
    N = qw.shape[0]
    dev = q.device
    _need(qw, "qw", (torch.int8,), (N, K), dev)
    _need(sa, "sa", (torch.float32,), (M,), dev)
    _need(sw, "sw", (torch.float32,), (N, K // 128), dev)
    code = _out_code(out_dtype)
    out = torch.empty((M, N), dtype=out_dtype, device=dev) if out is None else out
    _need(out, "out", (out_dtype,), (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_gemm_w8a8_g128(_ptr(q), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K,
                                        _ptr(out), code, _stream(dev)), "bsb_gemm_w8a8_g128")
    return out


def repack_weights_mfma(qw: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """packed [N*K] int8: qw [N,K] rearranged into the matrix cores' operand order (1 KB per
    16-row x 64-column block), the weight form gemm_w8a8_g128_packed reads."""
    _need(qw, "qw", (torch.int8,))
    if qw.dim() != 2:
        raise ValueError("qw [N,K] required")
    N, K = qw.shape
    dev = qw.device
    out = torch.empty((N * K,), dtype=torch.int8, device=dev) if out is None else out
    _need(out, "out", (torch.int8,), (N * K,), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_repack_weights_mfma(_ptr(qw), N, K, _ptr(out), _stream(dev)),
               "bsb_repack_weights_mfma")
    return out


def gemm_w8a8_g128_packed(q: torch.Tensor, sa: torch.Tensor, packed: torch.Tensor,
                          sw: torch.Tensor, out_dtype=torch.bfloat16,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gemm_w8a8_g128 (M <= 64) on weights from repack_weights_mfma; sw [N,K/128] unchanged.
    Bit-identical to gemm_w8a8_g128 on the unpacked weights."""
    _need(q, "q", (torch.int8,))
    if q.dim() != 2 or sw.dim() != 2:
        raise ValueError("q [M,K] and sw [N,K/128] required")
    M, K = q.shape
    N = sw.shape[0]
    dev = q.device
    _need(packed, "packed", (torch.int8,), (N * K,), dev)
    _need(sa, "sa", (torch.float32,), (M,), dev)
    _need(sw, "sw", (torch.float32,), (N, K // 128), dev)
    code = _out_code(out_dtype)
    out = torch.empty((M, N), dtype=out_dtype, device=dev) if out is None else out
    _need(out, "out", (out_dtype,), (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_gemm_w8a8_g128_packed(_ptr(q), _ptr(sa), _ptr(packed), _ptr(sw), M, N,
                                               K, _ptr(out), code, _stream(dev)),
               "bsb_gemm_w8a8_g128_packed")
    return out


def gemm_w8a8_channel(q: torch.Tensor, sa: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
                      out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [M,N] = W8A8 GEMM of q [M,K] (scales sa [M]) with qw [N,K] and one weight scale per
    row (sw [N], per-channel) or one for all rows (sw [1], per-tensor)."""
    _need(q, "q", (torch.int8,))
    if q.dim() != 2 or qw.dim() != 2:
        raise ValueError("q [M,K] and qw [N,K] required")
    M, K = q.shape
    N = qw.shape[0]
    dev = q.device
    _need(qw, "qw", (torch.int8,), (N, K), dev)
    _need(sa, "sa", (torch.float32,), (M,), dev)
    _need(sw, "sw", (torch.float32,), None, dev)
    if sw.dim() != 1 or sw.shape[0] not in (1, N):
        raise ValueError("sw must be [N] (per-channel) or [1] (per-tensor)")
    stride = 1 if sw.shape[0] == N and N > 1 else 0
    code = _out_code(out_dtype)
    out = torch.empty((M, N), dtype=out_dtype, device=dev) if out is None else out
    _need(out, "out", (out_dtype,), (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_gemm_w8a8_channel(_ptr(q), _ptr(sa), _ptr(qw), _ptr(sw), stride, M, N, K,
                                           _ptr(out), code, _stream(dev)), "bsb_gemm_w8a8_channel")
    return out


def gemm_w8a8_g128_partials(q: torch.Tensor, qw: torch.Tensor,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """INT32 group partials P [M,N,K/128] from the GEMM's own main loop."""
    _need(q, "q", (torch.int8,))
    M, K = q.shape
    N = qw.shape[0]
    dev = q.device
    _need(qw, "qw", (torch.int8,), (N, K), dev)
    out = torch.empty((M, N, K // 128), dtype=torch.int32, device=dev) if out is None else out
    _need(out, "out", (torch.int32,), (M, N, K // 128), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_gemm_w8a8_g128_partials(_ptr(q), _ptr(qw), M, N, K, _ptr(out),
                                                 _stream(dev)), "bsb_gemm_w8a8_g128_partials")
    return out


def grouped_gemm_w8a8_g128(q: torch.Tensor, sa: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
                           offsets: torch.Tensor, out_dtype=torch.bfloat16,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MoE form: rows [offsets[e], offsets[e+1]) of q run against expert e's qw [E,N,K] / sw [E,N,K/128].

    R is taken from q's first dimension; offsets must satisfy offsets[0] = 0,
    non-decreasing, offsets[E] = R (device tensor, not read on the host).
    """
    _need(q, "q", (torch.int8,))
    if q.dim() != 2 or qw.dim() != 3:
        raise ValueError("q [R,K] and qw [E,N,K] required")
    R, K = q.shape
    E, N, _ = qw.shape
    dev = q.device
    _need(qw, "qw", (torch.int8,), (E, N, K), dev)
    _need(sa, "sa", (torch.float32,), (R,), dev)
    _need(sw, "sw", (torch.float32,), (E, N, K // 128), dev)
    _need(offsets, "offsets", (torch.int32,), (E + 1,), dev)
    code = _out_code(out_dtype)
    out = torch.empty((R, N), dtype=out_dtype, device=dev) if out is None else out
    _need(out, "out", (out_dtype,), (R, N), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_grouped_gemm_w8a8_g128(_ptr(q), _ptr(sa), _ptr(qw), _ptr(sw),
                                                _ptr(offsets), E, R, N, K, _ptr(out), code,
                                                _stream(dev)), "bsb_grouped_gemm_w8a8_g128")
    return out


def grouped_gemm_w8a8_g128_gather(q: torch.Tensor, sa: torch.Tensor, index: torch.Tensor,
                                  qw: torch.Tensor, sw: torch.Tensor, offsets: torch.Tensor,
                                  out_dtype=torch.bfloat16,
                                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """grouped_gemm_w8a8_g128 on rows gathered by the kernel: q [T,K] / sa [T] are the
    quantised tokens and row r is token index[r] (index [R] int32, device); bit-identical
    to gather_rows followed by grouped_gemm_w8a8_g128."""
    _need(q, "q", (torch.int8,))
    if q.dim() != 2 or qw.dim() != 3:
        raise ValueError("q [T,K] and qw [E,N,K] required")
    T, K = q.shape
    E, N, _ = qw.shape
    dev = q.device
    _need(index, "index", (torch.int32,), None, dev)
    if index.dim() != 1:
        raise ValueError("index must be [R]")
    R = index.shape[0]
    _need(qw, "qw", (torch.int8,), (E, N, K), dev)
    _need(sa, "sa", (torch.float32,), (T,), dev)
    _need(sw, "sw", (torch.float32,), (E, N, K // 128), dev)
    _need(offsets, "offsets", (torch.int32,), (E + 1,), dev)
    code = _out_code(out_dtype)
    out = torch.empty((R, N), dtype=out_dtype, device=dev) if out is None else out
    _need(out, "out", (out_dtype,), (R, N), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_grouped_gemm_w8a8_g128_gather(
            _ptr(q), _ptr(sa), _ptr(index), T, _ptr(qw), _ptr(sw), _ptr(offsets), E, R, N, K,
            _ptr(out), code, _stream(dev)), "bsb_grouped_gemm_w8a8_g128_gather")
    return out


def grouped_gemm_w8a8_g128_packed(q: torch.Tensor, sa: torch.Tensor, packed: torch.Tensor,
                                  sw: torch.Tensor, offsets: torch.Tensor,
                                  out_dtype=torch.bfloat16,
                                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """grouped_gemm_w8a8_g128 on packed expert weights: packed [E*N*K] is
    repack_weights_mfma(qw.view(E*N, K)); sw [E,N,K/128]. Bit-identical results."""
    _need(q, "q", (torch.int8,))
    if q.dim() != 2 or sw.dim() != 3:
        raise ValueError("q [R,K] and sw [E,N,K/128] required")
    R, K = q.shape
    E, N, _ = sw.shape
    dev = q.device
    _need(packed, "packed", (torch.int8,), (E * N * K,), dev)
    _need(sa, "sa", (torch.float32,), (R,), dev)
    _need(sw, "sw", (torch.float32,), (E, N, K // 128), dev)
    _need(offsets, "offsets", (torch.int32,), (E + 1,), dev)
    code = _out_code(out_dtype)
    out = torch.empty((R, N), dtype=out_dtype, device=dev) if out is None else out
    _need(out, "out", (out_dtype,), (R, N), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_grouped_gemm_w8a8_g128_packed(_ptr(q), _ptr(sa), _ptr(packed),
                                                       _ptr(sw), _ptr(offsets), E, R, N, K,
                                                       _ptr(out), code, _stream(dev)),
               "bsb_grouped_gemm_w8a8_g128_packed")
    return out


def decode_fp8_block(w: torch.Tensor, bs: torch.Tensor, dialect: int,
                     qw: Optional[torch.Tensor] = None,
                     sw: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """FP8 e4m3 bytes [N,K] + UE8M0 block exponents [N/128,K/128] -> (qw int8 [N,K], sw [N,K/128])."""
    _need(w, "w", (torch.uint8,))
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    N, K = w.shape
    dev = w.device
    _need(bs, "bs", (torch.uint8,), (N // 128, K // 128), dev)
    if dialect not in (BSB_FP8_OCP, BSB_FP8_FNUZ):
        raise ValueError("dialect must be BSB_FP8_OCP or BSB_FP8_FNUZ")
    qw = torch.empty((N, K), dtype=torch.int8, device=dev) if qw is None else qw
    sw = torch.empty((N, K // 128), dtype=torch.float32, device=dev) if sw is None else sw
    _need(qw, "qw", (torch.int8,), (N, K), dev)
    _need(sw, "sw", (torch.float32,), (N, K // 128), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_decode_fp8_block(_ptr(w), _ptr(bs), N, K, dialect, _ptr(qw), _ptr(sw),
                                          _stream(dev)), "bsb_decode_fp8_block")
    return qw, sw


def decode_fp8_block_packed(w: torch.Tensor, bs: torch.Tensor, dialect: int,
                            packed: Optional[torch.Tensor] = None,
                            sw: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """decode_fp8_block with the INT8 weight written in the matrix cores' operand order
    (packed [N*K], as repack_weights_mfma would leave it) and sw [N,K/128]."""
    _need(w, "w", (torch.uint8,))
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    N, K = w.shape
    dev = w.device
    _need(bs, "bs", (torch.uint8,), (N // 128, K // 128), dev)
    if dialect not in (BSB_FP8_OCP, BSB_FP8_FNUZ):
        raise ValueError("dialect must be BSB_FP8_OCP or BSB_FP8_FNUZ")
    packed = torch.empty((N * K,), dtype=torch.int8, device=dev) if packed is None else packed
    sw = torch.empty((N, K // 128), dtype=torch.float32, device=dev) if sw is None else sw
    _need(packed, "packed", (torch.int8,), (N * K,), dev)
    _need(sw, "sw", (torch.float32,), (N, K // 128), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_decode_fp8_block_packed(_ptr(w), _ptr(bs), N, K, dialect, _ptr(packed),
                                                 _ptr(sw), _stream(dev)),
               "bsb_decode_fp8_block_packed")
    return packed, sw


def dequant_fp8_block_bf16(w: torch.Tensor, bs: torch.Tensor, dialect: int,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """FP8 e4m3 bytes [N,K] + UE8M0 block exponents [N/128,K/128] -> BF16 weights [N,K]."""
    _need(w, "w", (torch.uint8,))
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    N, K = w.shape
    dev = w.device
    _need(bs, "bs", (torch.uint8,), (N // 128, K // 128), dev)
    if dialect not in (BSB_FP8_OCP, BSB_FP8_FNUZ):
        raise ValueError("dialect must be BSB_FP8_OCP or BSB_FP8_FNUZ")
    out = torch.empty((N, K), dtype=torch.bfloat16, device=dev) if out is None else out
    _need(out, "out", _BF16_BITS, (N, K), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_dequant_fp8_block_bf16(_ptr(w), _ptr(bs), N, K, dialect, _ptr(out),
                                                _stream(dev)), "bsb_dequant_fp8_block_bf16")
    return out


def gemm_w8a16_g128(x: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
                    out_dtype=torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [M,N] = weight-only INT8 GEMM of BF16 activations x [M,K] (M <= 64) with qw [N,K]
    and per-group scales sw [N,K/128]."""
    _need(x, "x", _BF16_BITS)
    if x.dim() != 2 or qw.dim() != 2:
        raise ValueError("x [M,K] and qw [N,K] required")
    M, K = x.shape
    N = qw.shape[0]
    dev = x.device
    _need(qw, "qw", (torch.int8,), (N, K), dev)
    _need(sw, "sw", (torch.float32,), (N, K // 128), dev)
    code = _out_code(out_dtype)
    out = torch.empty((M, N), dtype=out_dtype, device=dev) if out is None else out
    _need(out, "out", (out_dtype,), (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_gemm_w8a16_g128(_ptr(x), _ptr(qw), _ptr(sw), M, N, K, _ptr(out), code,
                                         _stream(dev)), "bsb_gemm_w8a16_g128")
    return out


def gemm_bf16(x: torch.Tensor, w: torch.Tensor, out_dtype=torch.bfloat16,
              out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y [M,N] = BF16 GEMM of x [M,K] (M <= 64) with w [N,K] (BF16)."""
    _need(x, "x", _BF16_BITS)
    if x.dim() != 2 or w.dim() != 2:
        raise ValueError("x [M,K] and w [N,K] required")
    M, K = x.shape
    N = w.shape[0]
    dev = x.device
    _need(w, "w", _BF16_BITS, (N, K), dev)
    code = _out_code(out_dtype)
    out = torch.empty((M, N), dtype=out_dtype, device=dev) if out is None else out
    _need(out, "out", (out_dtype,), (M, N), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_gemm_bf16(_ptr(x), _ptr(w), M, N, K, _ptr(out), code, _stream(dev)),
               "bsb_gemm_bf16")
    return out


def decode_mxfp4(packed: torch.Tensor, scale: torch.Tensor,
                 qw: Optional[torch.Tensor] = None,
                 sw: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """MXFP4 packed [E,N,K/2] + UE8M0 [E,N,K/32] -> (qw int8 [E,N,K], sw [E,N,K/128])."""
    _need(packed, "packed", (torch.uint8,))
    if packed.dim() != 3:
        raise ValueError("packed must be [E, N, K/2]")
    E, N, Kh = packed.shape
    K = 2 * Kh
    dev = packed.device
    _need(scale, "scale", (torch.uint8,), (E, N, K // 32), dev)
    qw = torch.empty((E, N, K), dtype=torch.int8, device=dev) if qw is None else qw
    sw = torch.empty((E, N, K // 128), dtype=torch.float32, device=dev) if sw is None else sw
    _need(qw, "qw", (torch.int8,), (E, N, K), dev)
    _need(sw, "sw", (torch.float32,), (E, N, K // 128), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_decode_mxfp4(_ptr(packed), _ptr(scale), E, N, K, _ptr(qw), _ptr(sw),
                                      _stream(dev)), "bsb_decode_mxfp4")
    return qw, sw


def decode_mxfp4_packed(packed: torch.Tensor, scale: torch.Tensor,
                        packed_qw: Optional[torch.Tensor] = None,
                        sw: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """decode_mxfp4 with the INT8 weight written in the matrix cores' operand order: packed_qw
    [E*N*K] as repack_weights_mfma leaves the stacked [E*N, K] weights, and sw [E,N,K/128]."""
    _need(packed, "packed", (torch.uint8,))
    if packed.dim() != 3:
        raise ValueError("packed must be [E, N, K/2]")
    E, N, Kh = packed.shape
    K = 2 * Kh
    dev = packed.device
    _need(scale, "scale", (torch.uint8,), (E, N, K // 32), dev)
    packed_qw = (torch.empty((E * N * K,), dtype=torch.int8, device=dev) if packed_qw is None
                 else packed_qw)
    sw = torch.empty((E, N, K // 128), dtype=torch.float32, device=dev) if sw is None else sw
    _need(packed_qw, "packed_qw", (torch.int8,), (E * N * K,), dev)
    _need(sw, "sw", (torch.float32,), (E, N, K // 128), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_decode_mxfp4_packed(_ptr(packed), _ptr(scale), E, N, K, _ptr(packed_qw),
                                             _ptr(sw), _stream(dev)), "bsb_decode_mxfp4_packed")
    return packed_qw, sw


def gather_rows(q: torch.Tensor, sa: torch.Tensor, index: torch.Tensor,
                q_out: Optional[torch.Tensor] = None,
                sa_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Quantised tokens q [T,K] / sa [T] -> rows in expert order q[index], sa[index] ([R,K], [R])."""
    _need(q, "q", (torch.int8,))
    if q.dim() != 2:
        raise ValueError("q must be [T, K]")
    T, K = q.shape
    dev = q.device
    _need(sa, "sa", (torch.float32,), (T,), dev)
    _need(index, "index", (torch.int32,), None, dev)
    if index.dim() != 1:
        raise ValueError("index must be [R]")
    R = index.shape[0]
    q_out = torch.empty((R, K), dtype=torch.int8, device=dev) if q_out is None else q_out
    sa_out = torch.empty((R,), dtype=torch.float32, device=dev) if sa_out is None else sa_out
    _need(q_out, "q_out", (torch.int8,), (R, K), dev)
    _need(sa_out, "sa_out", (torch.float32,), (R,), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_gather_rows(_ptr(q), _ptr(sa), _ptr(index), R, T, K, _ptr(q_out),
                                     _ptr(sa_out), _stream(dev)), "bsb_gather_rows")
    return q_out, sa_out


def moe_combine(y: torch.Tensor, row_of_pair: torch.Tensor, gate: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Expert outputs y [R,N] (BF16) -> per-token sum_k gate[t,k] * y[row_of_pair[t,k]] [T,N] BF16."""
    _need(y, "y", _BF16_BITS)
    if y.dim() != 2:
        raise ValueError("y must be [R, N]")
    R, N = y.shape
    dev = y.device
    _need(row_of_pair, "row_of_pair", (torch.int32,), None, dev)
    if row_of_pair.dim() != 2:
        raise ValueError("row_of_pair must be [T, topk]")
    T, topk = row_of_pair.shape
    _need(gate, "gate", (torch.float32,), (T, topk), dev)
    out = torch.empty((T, N), dtype=y.dtype, device=dev) if out is None else out
    _need(out, "out", _BF16_BITS, (T, N), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_moe_combine(_ptr(y), _ptr(row_of_pair), _ptr(gate), T, topk, R, N,
                                     _ptr(out), _stream(dev)), "bsb_moe_combine")
    return out


KV_HEAD_DIM = 128
KV_CHUNK = 64          # tokens per cache row: caches are [T/64, B, Hkv, 64 * 128]


def kv_cache_empty(B: int, Hkv: int, T: int, device) -> Tuple[torch.Tensor, ...]:
    """Allocate (k_cache, k_scale, v_cache, v_scale) for B sequences of T token
    slots (T a multiple of 64) over Hkv heads of dimension 128, in the layout of
    bsb_kv_cache_write (contents undefined until written)."""
    dev = torch.device(device)
    rows = (T // KV_CHUNK, B, Hkv, KV_CHUNK * KV_HEAD_DIM)
    return (torch.empty(rows, dtype=torch.int8, device=dev),
            torch.empty((B, Hkv, T), dtype=torch.float32, device=dev),
            torch.empty(rows, dtype=torch.int8, device=dev),
            torch.empty((B, Hkv, T), dtype=torch.float32, device=dev))


def _kv_shapes(k_cache, k_scale, v_cache, v_scale):
    _need(k_cache, "k_cache", (torch.int8,))
    if k_cache.dim() != 4 or k_cache.shape[3] != KV_CHUNK * KV_HEAD_DIM:
        raise ValueError("k_cache must be [T/64, B, Hkv, 8192]")
    nc, B, Hkv, _ = k_cache.shape
    T = nc * KV_CHUNK
    dev = k_cache.device
    _need(k_scale, "k_scale", (torch.float32,), (B, Hkv, T), dev)
    _need(v_cache, "v_cache", (torch.int8,), tuple(k_cache.shape), dev)
    _need(v_scale, "v_scale", (torch.float32,), (B, Hkv, T), dev)
    return B, Hkv, T, dev


def kv_cache_write(k: torch.Tensor, v: torch.Tensor, seq: torch.Tensor, pos: torch.Tensor,
                   k_cache: torch.Tensor, k_scale: torch.Tensor, v_cache: torch.Tensor,
                   v_scale: torch.Tensor) -> None:
    """Quantise n new tokens' keys and values k, v [n, Hkv, 128] (BF16) per vector and
    write them to slot pos[i] of sequence seq[i] (int32 [n])."""
    B, Hkv, T, dev = _kv_shapes(k_cache, k_scale, v_cache, v_scale)
    _need(k, "k", _BF16_BITS, None, dev)
    if k.dim() != 3 or k.shape[1:] != (Hkv, KV_HEAD_DIM):
        raise ValueError("k must be [n, Hkv, 128]")
    n = k.shape[0]
    _need(v, "v", _BF16_BITS, (n, Hkv, KV_HEAD_DIM), dev)
    _need(seq, "seq", (torch.int32,), (n,), dev)
    _need(pos, "pos", (torch.int32,), (n,), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_kv_cache_write(_ptr(k), _ptr(v), _ptr(seq), _ptr(pos), n, B, Hkv, T,
                                        KV_HEAD_DIM, _ptr(k_cache), _ptr(k_scale), _ptr(v_cache),
                                        _ptr(v_scale), _stream(dev)), "bsb_kv_cache_write")


def attention_workspace_bytes(B: int, Hq: int, max_len: int) -> int:
    n = lib().bsb_attention_workspace_bytes(B, Hq, max_len)
    if n < 0:
        raise ValueError("invalid attention sizes")
    return n


ATTENTION_NOALLOC_MAX_BYTES = 32 << 20   # BSB_ATTENTION_NOALLOC_MAX_BYTES


def attention_decode_int8kv_noalloc(q: torch.Tensor, k_cache: torch.Tensor,
                                    k_scale: torch.Tensor, v_cache: torch.Tensor,
                                    v_scale: torch.Tensor, lens: torch.Tensor, max_len: int,
                                    out: torch.Tensor) -> torch.Tensor:
    """attention_decode_int8kv with the library's static per-device workspace instead of a
    caller's (bsb_attention_decode_int8kv_noalloc): allocates nothing, so `out` [B, Hq, 128]
    (BF16 or float32) is required. Calls that overlap on one device race."""
    B, Hkv, T, dev = _kv_shapes(k_cache, k_scale, v_cache, v_scale)
    _need(q, "q", _BF16_BITS, None, dev)
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != KV_HEAD_DIM:
        raise ValueError("q must be [B, Hq, 128]")
    Hq = q.shape[1]
    _need(lens, "lens", (torch.int32,), (B,), dev)
    code = _out_code(out.dtype)
    _need(out, "out", (out.dtype,), (B, Hq, KV_HEAD_DIM), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_attention_decode_int8kv_noalloc(
            _ptr(q), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale), _ptr(lens),
            B, Hq, Hkv, T, KV_HEAD_DIM, max_len, _ptr(out), code, _stream(dev)),
            "bsb_attention_decode_int8kv_noalloc")
    return out


def attention_decode_int8kv(q: torch.Tensor, k_cache: torch.Tensor, k_scale: torch.Tensor,
                            v_cache: torch.Tensor, v_scale: torch.Tensor, lens: torch.Tensor,
                            max_len: int, out_dtype=torch.bfloat16,
                            out: Optional[torch.Tensor] = None,
                            work: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention of q [B, Hq, 128] (BF16) over the INT8 cache, lens int32 [B]
    cached tokens per sequence (<= max_len); returns out [B, Hq, 128]."""
    B, Hkv, T, dev = _kv_shapes(k_cache, k_scale, v_cache, v_scale)
    _need(q, "q", _BF16_BITS, None, dev)
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != KV_HEAD_DIM:
        raise ValueError("q must be [B, Hq, 128]")
    Hq = q.shape[1]
    _need(lens, "lens", (torch.int32,), (B,), dev)
    code = _out_code(out_dtype)
    out = torch.empty((B, Hq, KV_HEAD_DIM), dtype=out_dtype, device=dev) if out is None else out
    _need(out, "out", (out_dtype,), (B, Hq, KV_HEAD_DIM), dev)
    nbytes = attention_workspace_bytes(B, Hq, max_len)
    if work is None:
        work = torch.empty((max(nbytes, 4) // 4,), dtype=torch.float32, device=dev)
    _need(work, "work", (torch.float32,), None, dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_attention_decode_int8kv(
            _ptr(q), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale), _ptr(lens),
            B, Hq, Hkv, T, KV_HEAD_DIM, max_len, _ptr(work), work.numel() * 4, _ptr(out), code,
            _stream(dev)), "bsb_attention_decode_int8kv")
    return out


def attention_chunk_int8kv(q: torch.Tensor, k_cache: torch.Tensor, k_scale: torch.Tensor,
                           v_cache: torch.Tensor, v_scale: torch.Tensor, lens: torch.Tensor,
                           max_len: int, out_dtype=torch.bfloat16,
                           out: Optional[torch.Tensor] = None,
                           work: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal attention of the newest Qn tokens of each sequence, q [B, Qn, Hq, 128] (BF16),
    over the INT8 cache (their keys and values already written; lens counts them);
    returns out [B, Qn, Hq, 128]."""
    B, Hkv, T, dev = _kv_shapes(k_cache, k_scale, v_cache, v_scale)
    _need(q, "q", _BF16_BITS, None, dev)
    if q.dim() != 4 or q.shape[0] != B or q.shape[3] != KV_HEAD_DIM:
        raise ValueError("q must be [B, Qn, Hq, 128]")
    Qn, Hq = q.shape[1], q.shape[2]
    _need(lens, "lens", (torch.int32,), (B,), dev)
    code = _out_code(out_dtype)
    out = (torch.empty((B, Qn, Hq, KV_HEAD_DIM), dtype=out_dtype, device=dev) if out is None
           else out)
    _need(out, "out", (out_dtype,), (B, Qn, Hq, KV_HEAD_DIM), dev)
    nbytes = attention_workspace_bytes(B, Qn * Hq, max_len)
    if work is None:
        work = torch.empty((max(nbytes, 4) // 4,), dtype=torch.float32, device=dev)
    _need(work, "work", (torch.float32,), None, dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_attention_chunk_int8kv(
            _ptr(q), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale), _ptr(lens),
            B, Qn, Hq, Hkv, T, KV_HEAD_DIM, max_len, _ptr(work), work.numel() * 4, _ptr(out), code,
            _stream(dev)), "bsb_attention_chunk_int8kv")
    return out


def kv_cache_empty_bf16(B: int, Hkv: int, T: int, device) -> Tuple[torch.Tensor, torch.Tensor]:
    """Allocate the BF16 comparison cache (k_cache, v_cache) in the layout of
    bsb_kv_cache_write_bf16 (contents undefined until written)."""
    dev = torch.device(device)
    rows = (T // KV_CHUNK, B, Hkv, KV_CHUNK * KV_HEAD_DIM)
    return (torch.empty(rows, dtype=torch.bfloat16, device=dev),
            torch.empty(rows, dtype=torch.bfloat16, device=dev))


def _kv16_shapes(k_cache, v_cache):
    _need(k_cache, "k_cache", _BF16_BITS)
    if k_cache.dim() != 4 or k_cache.shape[3] != KV_CHUNK * KV_HEAD_DIM:
        raise ValueError("k_cache must be [T/64, B, Hkv, 8192]")
    nc, B, Hkv, _ = k_cache.shape
    T = nc * KV_CHUNK
    dev = k_cache.device
    _need(v_cache, "v_cache", _BF16_BITS, tuple(k_cache.shape), dev)
    return B, Hkv, T, dev


def kv_cache_write_bf16(k: torch.Tensor, v: torch.Tensor, seq: torch.Tensor, pos: torch.Tensor,
                        k_cache: torch.Tensor, v_cache: torch.Tensor) -> None:
    """Copy n new tokens' keys and values k, v [n, Hkv, 128] (BF16) into slot pos[i] of
    sequence seq[i] of the BF16 cache."""
    B, Hkv, T, dev = _kv16_shapes(k_cache, v_cache)
    _need(k, "k", _BF16_BITS, None, dev)
    if k.dim() != 3 or k.shape[1:] != (Hkv, KV_HEAD_DIM):
        raise ValueError("k must be [n, Hkv, 128]")
    n = k.shape[0]
    _need(v, "v", _BF16_BITS, (n, Hkv, KV_HEAD_DIM), dev)
    _need(seq, "seq", (torch.int32,), (n,), dev)
    _need(pos, "pos", (torch.int32,), (n,), dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_kv_cache_write_bf16(_ptr(k), _ptr(v), _ptr(seq), _ptr(pos), n, B, Hkv, T,
                                             KV_HEAD_DIM, _ptr(k_cache), _ptr(v_cache),
                                             _stream(dev)), "bsb_kv_cache_write_bf16")


def attention_decode_bf16kv(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            lens: torch.Tensor, max_len: int, out_dtype=torch.bfloat16,
                            out: Optional[torch.Tensor] = None,
                            work: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention of q [B, Hq, 128] (BF16) over the BF16 cache."""
    B, Hkv, T, dev = _kv16_shapes(k_cache, v_cache)
    _need(q, "q", _BF16_BITS, None, dev)
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != KV_HEAD_DIM:
        raise ValueError("q must be [B, Hq, 128]")
    Hq = q.shape[1]
    _need(lens, "lens", (torch.int32,), (B,), dev)
    code = _out_code(out_dtype)
    out = torch.empty((B, Hq, KV_HEAD_DIM), dtype=out_dtype, device=dev) if out is None else out
    _need(out, "out", (out_dtype,), (B, Hq, KV_HEAD_DIM), dev)
    nbytes = attention_workspace_bytes(B, Hq, max_len)
    if work is None:
        work = torch.empty((max(nbytes, 4) // 4,), dtype=torch.float32, device=dev)
    _need(work, "work", (torch.float32,), None, dev)
    with torch.cuda.device(dev):
        _check(lib().bsb_attention_decode_bf16kv(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(lens), B, Hq, Hkv, T, KV_HEAD_DIM, max_len,
            _ptr(work), work.numel() * 4, _ptr(out), code, _stream(dev)),
            "bsb_attention_decode_bf16kv")
    return out
