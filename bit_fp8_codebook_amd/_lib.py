"""ctypes binding of libq3.so: argument marshalling only.

Every function here forwards to the C entry point of the same name (declared in
include/q3.h); all arithmetic runs in the library's HIP kernels.  torch is used
for device memory and for the current HIP stream.  If the library is missing
the import fails loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq3.so")

c_i64 = ctypes.c_int64
c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p


class Q3LayoutInfo(ctypes.Structure):
    _fields_ = [(f, c_i64) for f in ("n", "k", "groups", "padded_groups", "tiles", "code_tile_bytes",
                                     "scale_tile_bytes", "code_plane_bytes", "scale_plane_bytes", "codebook_bytes",
                                     "payload_bytes")]


class Q3Matrix(ctypes.Structure):
    _fields_ = [("n", c_i64), ("k", c_i64), ("code_plane", c_vp), ("scale_plane", c_vp), ("codebook", c_vp)]


class Q3ExpertStack(ctypes.Structure):
    _fields_ = [("num_experts", c_i64), ("n", c_i64), ("k", c_i64),
                ("code_plane", c_vp), ("code_expert_stride", c_i64),
                ("scale_plane", c_vp), ("scale_expert_stride", c_i64),
                ("codebook", c_vp), ("codebook_expert_stride", c_i64)]


# name -> (restype, argtypes); the same list include/q3.h declares.
SIGNATURES = {
    "q3_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "q3_layout": (ctypes.c_int, [c_i64, c_i64, ctypes.POINTER(Q3LayoutInfo)]),
    "q3_pack": (ctypes.c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "q3_unpack": (ctypes.c_int, [ctypes.POINTER(Q3Matrix), c_vp, c_vp, c_vp]),
    "q3_gemv": (ctypes.c_int, [ctypes.POINTER(Q3Matrix), c_vp, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "q3_gemm_small_m": (ctypes.c_int, [ctypes.POINTER(Q3Matrix), c_vp, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "q3_moe_topk": (ctypes.c_int, [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "q3_grouped_expert_gemv": (ctypes.c_int, [ctypes.POINTER(Q3ExpertStack), c_vp, c_i64, c_i32, c_vp, c_i32,
                                              c_i32, c_vp, c_i64, c_vp]),
}

STATUS = {0: "Q3_OK", 1: "Q3_ERR_INVALID_ARG", 2: "Q3_ERR_UNSUPPORTED_SHAPE", 3: "Q3_ERR_MISALIGNED",
          4: "Q3_ERR_UNSUPPORTED_DEVICE", 5: "Q3_ERR_HIP"}

_lib = None


class Q3Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = _lib.q3_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({msg})")


def lib():
    """Load libq3.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bit_fp8_codebook_amd.build` "
                              "(the q3 ops have no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn, status):
    if status != 0:
        raise Q3Error(fn, status)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t


# ------------------------------------------------------------------ layout

def q3_layout(n: int, k: int) -> dict:
    info = Q3LayoutInfo()
    _check("q3_layout", lib().q3_layout(n, k, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in Q3LayoutInfo._fields_}


@dataclass
class PackedMatrix:
    """Device-resident packed weights of an n x k layer (planes as uint8 tensors)."""
    n: int
    k: int
    code_plane: torch.Tensor    # uint8 [code_plane_bytes], tile-major
    scale_plane: torch.Tensor   # uint8 [scale_plane_bytes], tile-major
    codebook: torch.Tensor      # uint8 [n][8] E4M3FN

    def desc(self) -> Q3Matrix:
        return Q3Matrix(self.n, self.k, self.code_plane.data_ptr(), self.scale_plane.data_ptr(),
                        self.codebook.data_ptr())

    @property
    def payload_bytes(self) -> int:
        return self.n * self.k * 13 // 32

    def clone(self) -> "PackedMatrix":
        return PackedMatrix(self.n, self.k, self.code_plane.clone(), self.scale_plane.clone(),
                            self.codebook.clone())


def empty_packed(n: int, k: int, device) -> PackedMatrix:
    L = q3_layout(n, k)
    return PackedMatrix(n, k, torch.empty(L["code_plane_bytes"], dtype=torch.uint8, device=device),
                        torch.empty(L["scale_plane_bytes"], dtype=torch.uint8, device=device),
                        torch.empty((n, 8), dtype=torch.uint8, device=device))


def q3_pack(codes: torch.Tensor, scales: torch.Tensor, codebook: torch.Tensor, out: PackedMatrix = None):
    """codes uint8 [n][k] (0..7), scales uint8 [n][k/32] (E8M0), codebook uint8 [n][8] -> PackedMatrix."""
    _dev(codes, "codes"), _dev(scales, "scales"), _dev(codebook, "codebook")
    n, k = codes.shape
    if codes.stride(1) != 1 or scales.stride(1) != 1:
        raise ValueError("codes and scales rows must be contiguous")
    w = out if out is not None else empty_packed(n, k, codes.device)
    w.codebook.copy_(codebook)
    _check("q3_pack", lib().q3_pack(codes.data_ptr(), codes.stride(0), scales.data_ptr(), scales.stride(0), n, k,
                                    w.code_plane.data_ptr(), w.scale_plane.data_ptr(), _stream(codes)))
    return w


def q3_unpack(w: PackedMatrix):
    codes = torch.empty((w.n, w.k), dtype=torch.uint8, device=w.code_plane.device)
    scales = torch.empty((w.n, w.k // 32), dtype=torch.uint8, device=w.code_plane.device)
    d = w.desc()
    _check("q3_unpack", lib().q3_unpack(ctypes.byref(d), codes.data_ptr(), scales.data_ptr(),
                                        _stream(w.code_plane)))
    return codes, scales


def _tokens(x: torch.Tensor, w_k: int):
    _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != w_k or x.stride(1) != 1:
        raise ValueError("x must be [m][k] with contiguous rows")
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("x must hold bf16 values (bfloat16 or 16-bit bit patterns)")
    return x


def _out(y, m, n, device):
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=device)
    if y.dtype != torch.float32 or y.stride(1) != 1:
        raise ValueError("y must be float32 with contiguous rows")
    return y


def q3_gemv(w: PackedMatrix, x: torch.Tensor, y: torch.Tensor = None) -> torch.Tensor:
    """y[m][n] = x[m] . w[n] for m <= 8 on the vector ALUs."""
    x = _tokens(x, w.k)
    m = x.shape[0]
    y = _out(y, m, w.n, x.device)
    d = w.desc()
    _check("q3_gemv", lib().q3_gemv(ctypes.byref(d), x.data_ptr(), m, x.stride(0), y.data_ptr(), y.stride(0),
                                    _stream(x)))
    return y


def q3_gemm_small_m(w: PackedMatrix, x: torch.Tensor, y: torch.Tensor = None) -> torch.Tensor:
    """y[m][n] = x[m] . w[n] for m <= 64 on the matrix cores."""
    x = _tokens(x, w.k)
    m = x.shape[0]
    y = _out(y, m, w.n, x.device)
    d = w.desc()
    _check("q3_gemm_small_m", lib().q3_gemm_small_m(ctypes.byref(d), x.data_ptr(), m, x.stride(0), y.data_ptr(),
                                                    y.stride(0), _stream(x)))
    return y


def q3_moe_topk(logits: torch.Tensor, topk: int, ids: torch.Tensor = None) -> torch.Tensor:
    _dev(logits, "logits")
    if logits.dtype != torch.float32 or not logits.is_contiguous():
        raise ValueError("logits must be contiguous float32 [t][E]")
    t, E = logits.shape
    if ids is None:
        ids = torch.empty((t, topk), dtype=torch.int32, device=logits.device)
    _check("q3_moe_topk", lib().q3_moe_topk(logits.data_ptr(), t, E, topk, ids.data_ptr(), _stream(logits)))
    return ids


@dataclass
class ExpertStack:
    """E packed experts of one shape, stored back to back."""
    num_experts: int
    n: int
    k: int
    code_plane: torch.Tensor    # uint8 [E][code_plane_bytes]
    scale_plane: torch.Tensor   # uint8 [E][scale_plane_bytes]
    codebook: torch.Tensor      # uint8 [E][n][8]

    def desc(self) -> Q3ExpertStack:
        return Q3ExpertStack(self.num_experts, self.n, self.k,
                             self.code_plane.data_ptr(), self.code_plane.stride(0),
                             self.scale_plane.data_ptr(), self.scale_plane.stride(0),
                             self.codebook.data_ptr(), self.codebook.stride(0))

    def expert(self, e: int) -> PackedMatrix:
        return PackedMatrix(self.n, self.k, self.code_plane[e], self.scale_plane[e], self.codebook[e])

    @property
    def payload_bytes_per_expert(self) -> int:
        return self.n * self.k * 13 // 32


def empty_stack(num_experts: int, n: int, k: int, device) -> ExpertStack:
    L = q3_layout(n, k)
    return ExpertStack(num_experts, n, k,
                       torch.empty((num_experts, L["code_plane_bytes"]), dtype=torch.uint8, device=device),
                       torch.empty((num_experts, L["scale_plane_bytes"]), dtype=torch.uint8, device=device),
                       torch.empty((num_experts, n, 8), dtype=torch.uint8, device=device))


def q3_grouped_expert_gemv(stack: ExpertStack, x: torch.Tensor, topk_ids: torch.Tensor, x_by_slot: bool,
                           y: torch.Tensor = None) -> torch.Tensor:
    """y[t*topk+j] = W[topk_ids[t][j]] . (x[t] or x[t*topk+j]); only picked experts are read."""
    _dev(x, "x"), _dev(topk_ids, "topk_ids")
    t, topk = topk_ids.shape
    if topk_ids.dtype != torch.int32 or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be contiguous int32 [t][topk]")
    if x.dim() != 2 or x.shape[1] != stack.k or x.stride(1) != 1:
        raise ValueError("x must be [rows][k] with contiguous rows")
    if x.shape[0] < (t * topk if x_by_slot else t):
        raise ValueError("x needs one row per token (gate/up) or per (token, slot) pair (down)")
    y = _out(y, t * topk, stack.n, x.device)
    d = stack.desc()
    _check("q3_grouped_expert_gemv",
           lib().q3_grouped_expert_gemv(ctypes.byref(d), x.data_ptr(), x.stride(0), 1 if x_by_slot else 0,
                                        topk_ids.data_ptr(), t, topk, y.data_ptr(), y.stride(0), _stream(x)))
    return y
