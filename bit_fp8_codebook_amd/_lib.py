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


class Q3Mxfp8Matrix(ctypes.Structure):
    _fields_ = [("n", c_i64), ("k", c_i64), ("elements", c_vp), ("ld_elements", c_i64), ("scales", c_vp),
                ("ld_scales", c_i64)]


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
    "q3_gemm_small_m_workspace_bytes": (c_i64, [c_i64, c_i64, c_i64]),
    "q3_gemm_small_m_ws": (ctypes.c_int, [ctypes.POINTER(Q3Matrix), c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64,
                                          c_vp]),
    "q3_moe_topk": (ctypes.c_int, [c_vp, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "q3_grouped_expert_gemv": (ctypes.c_int, [ctypes.POINTER(Q3ExpertStack), c_vp, c_i64, c_i32, c_vp, c_i32,
                                              c_i32, c_vp, c_i64, c_vp]),
    "q3_quantize": (ctypes.c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp]),
    "q3_fit_codebook": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]),
    "q3_moe_budget_topk": (ctypes.c_int, [c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_vp]),
    "q3_moe_mlp_workspace_bytes": (c_i64, [c_i64, c_i64, c_i32, c_i32]),
    "q3_moe_mlp": (ctypes.c_int, [ctypes.POINTER(Q3ExpertStack), ctypes.POINTER(Q3ExpertStack), c_vp, c_i64, c_vp,
                                  c_i32, c_i32, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp]),
    "q3_moe_mlp_noalloc_max_bytes": (c_i64, []),
    "q3_moe_mlp_noalloc": (ctypes.c_int, [ctypes.POINTER(Q3ExpertStack), ctypes.POINTER(Q3ExpertStack), c_vp, c_i64,
                                          c_vp, c_i32, c_i32, c_vp, c_i64, c_vp, c_i64, c_vp]),
    "q3_layout2": (ctypes.c_int, [c_i64, c_i64, ctypes.POINTER(Q3LayoutInfo)]),
    "q3_pack2": (ctypes.c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "q3_unpack2": (ctypes.c_int, [ctypes.POINTER(Q3Matrix), c_vp, c_vp, c_vp]),
    "q3_head2_scores": (ctypes.c_int, [ctypes.POINTER(Q3Matrix), c_vp, c_i64, c_i64, c_vp, c_i64, c_vp]),
    "q3_shortlist_workspace_bytes": (c_i64, [c_i64]),
    "q3_shortlist": (ctypes.c_int, [c_vp, c_i64, c_i64, c_i64, c_i32, c_vp, c_i64, c_vp, c_vp, c_vp]),
    "q3_rescore_fp8": (ctypes.c_int, [ctypes.POINTER(Q3Mxfp8Matrix), c_vp, c_i64, c_i64, c_vp, c_i32, c_vp, c_vp,
                                      c_vp]),
    "q3_draft_head_workspace_bytes": (c_i64, [c_i64, c_i64]),
    "q3_draft_head": (ctypes.c_int, [ctypes.POINTER(Q3Matrix), ctypes.POINTER(Q3Mxfp8Matrix), c_vp, c_i64, c_i64,
                                     c_i32, c_vp, c_i64, c_vp, c_vp, c_vp, c_vp]),
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


def _ld(t: torch.Tensor) -> int:
    """Row pitch in elements of a 2-D tensor with contiguous rows; a single row's
    pitch is meaningless to torch (it may report 0), so pass the row length."""
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _workspace(t: torch.Tensor, device):
    """A caller-supplied workspace: a contiguous device tensor on the inputs'
    device; its size in bytes goes to the library, which checks it."""
    if not isinstance(t, torch.Tensor) or t.device != torch.device(device):
        raise ValueError(f"workspace must be a tensor on {device} (the inputs' device)")
    if not t.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return t


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


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
    _check("q3_pack", lib().q3_pack(codes.data_ptr(), _ld(codes), scales.data_ptr(), _ld(scales), n, k,
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


def _out(y, m, n, device, name="y"):
    """A caller-supplied output must be exactly [m][n] float32 with contiguous
    rows on the inputs' device (its row pitch goes to the library, which writes
    m rows of n values); None allocates one."""
    if y is None:
        return torch.empty((m, n), dtype=torch.float32, device=device)
    _check_out(y, (m, n), torch.float32, device, name)
    return y


def _check_out(t, shape, dtype, device, name):
    if not isinstance(t, torch.Tensor) or t.device != torch.device(device):
        raise ValueError(f"{name} must be a tensor on {device} (the inputs' device)")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if len(shape) == 2 and shape[0] > 0 and shape[1] > 0 and t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous rows")
    if len(shape) == 2 and shape[0] > 1 and shape[1] > 0 and t.stride(0) < shape[1]:
        raise ValueError(f"{name} rows overlap (row pitch below the row length)")
    if len(shape) == 1 and shape[0] > 1 and t.stride(0) != 1:
        raise ValueError(f"{name} must be contiguous")


def q3_quantize(w: torch.Tensor, codebook: torch.Tensor, codes: torch.Tensor = None, scales: torch.Tensor = None):
    """fp32 weights [n][k] and E4M3FN codebooks [n][8] -> (codes uint8 [n][k], scales uint8 [n][k/32])."""
    _dev(w, "w"), _dev(codebook, "codebook")
    if w.dtype != torch.float32 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be float32 [n][k] with contiguous rows")
    n, k = w.shape
    if codebook.dtype != torch.uint8 or tuple(codebook.shape) != (n, 8) or not codebook.is_contiguous():
        raise ValueError("codebook must be contiguous uint8 [n][8]")
    if codes is None:
        codes = torch.empty((n, k), dtype=torch.uint8, device=w.device)
    else:
        _check_out(codes, (n, k), torch.uint8, w.device, "codes")
    if scales is None:
        scales = torch.empty((n, k // 32), dtype=torch.uint8, device=w.device)
    else:
        _check_out(scales, (n, k // 32), torch.uint8, w.device, "scales")
    _check("q3_quantize", lib().q3_quantize(w.data_ptr(), _ld(w), codebook.data_ptr(), n, k, codes.data_ptr(),
                                            _ld(codes), scales.data_ptr(), _ld(scales), _stream(w)))
    return codes, scales


def q3_fit_codebook(w: torch.Tensor, codebook: torch.Tensor = None) -> torch.Tensor:
    """fp32 weights [n][k] -> fitted per-row codebooks uint8 [n][8] (E4M3FN, ascending)."""
    _dev(w, "w")
    if w.dtype != torch.float32 or w.dim() != 2 or w.stride(1) != 1:
        raise ValueError("w must be float32 [n][k] with contiguous rows")
    n, k = w.shape
    if codebook is None:
        codebook = torch.empty((n, 8), dtype=torch.uint8, device=w.device)
    else:
        _check_out(codebook, (n, 8), torch.uint8, w.device, "codebook")
        if not codebook.is_contiguous():
            raise ValueError("codebook must be contiguous")
    _check("q3_fit_codebook", lib().q3_fit_codebook(w.data_ptr(), _ld(w), n, k, codebook.data_ptr(), _stream(w)))
    return codebook


def q3_gemv(w: PackedMatrix, x: torch.Tensor, y: torch.Tensor = None) -> torch.Tensor:
    """y[m][n] = x[m] . w[n] for m <= 8 on the vector ALUs."""
    x = _tokens(x, w.k)
    m = x.shape[0]
    y = _out(y, m, w.n, x.device)
    d = w.desc()
    _check("q3_gemv", lib().q3_gemv(ctypes.byref(d), x.data_ptr(), m, _ld(x), y.data_ptr(), _ld(y),
                                    _stream(x)))
    return y


def q3_gemm_small_m(w: PackedMatrix, x: torch.Tensor, y: torch.Tensor = None) -> torch.Tensor:
    """y[m][n] = x[m] . w[n] for m <= 64 on the matrix cores."""
    x = _tokens(x, w.k)
    m = x.shape[0]
    y = _out(y, m, w.n, x.device)
    d = w.desc()
    _check("q3_gemm_small_m", lib().q3_gemm_small_m(ctypes.byref(d), x.data_ptr(), m, _ld(x), y.data_ptr(),
                                                    _ld(y), _stream(x)))
    return y


def q3_gemm_small_m_workspace_bytes(n: int, k: int, m: int) -> int:
    return lib().q3_gemm_small_m_workspace_bytes(n, k, m)


def q3_gemm_small_m_ws(w: PackedMatrix, x: torch.Tensor, y: torch.Tensor = None,
                       workspace: torch.Tensor = None) -> torch.Tensor:
    """q3_gemm_small_m with a workspace (uint8 device tensor); when none is
    given, one of q3_gemm_small_m_workspace_bytes bytes is allocated here."""
    x = _tokens(x, w.k)
    m = x.shape[0]
    y = _out(y, m, w.n, x.device)
    if workspace is None:
        nbytes = q3_gemm_small_m_workspace_bytes(w.n, w.k, m)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    else:
        _workspace(workspace, x.device)
    d = w.desc()
    _check("q3_gemm_small_m_ws", lib().q3_gemm_small_m_ws(ctypes.byref(d), x.data_ptr(), m, _ld(x), y.data_ptr(),
                                                          _ld(y), workspace.data_ptr(), _nbytes(workspace),
                                                          _stream(x)))
    return y


def q3_moe_topk(logits: torch.Tensor, topk: int, ids: torch.Tensor = None) -> torch.Tensor:
    _dev(logits, "logits")
    if logits.dtype != torch.float32 or not logits.is_contiguous():
        raise ValueError("logits must be contiguous float32 [t][E]")
    t, E = logits.shape
    if ids is None:
        ids = torch.empty((t, topk), dtype=torch.int32, device=logits.device)
    else:
        _check_out(ids, (t, topk), torch.int32, logits.device, "ids")
        if not ids.is_contiguous():
            raise ValueError("ids must be contiguous")
    _check("q3_moe_topk", lib().q3_moe_topk(logits.data_ptr(), t, E, topk, ids.data_ptr(), _stream(logits)))
    return ids


def q3_moe_budget_topk(logits: torch.Tensor, topk: int, budget: int, ids: torch.Tensor = None,
                       experts: torch.Tensor = None):
    """Expert-budget routing of a verify round -> (ids int32 [t][topk], kept experts int32 [budget] ascending)."""
    _dev(logits, "logits")
    if logits.dtype != torch.float32 or not logits.is_contiguous():
        raise ValueError("logits must be contiguous float32 [t][E]")
    t, E = logits.shape
    if ids is None:
        ids = torch.empty((t, topk), dtype=torch.int32, device=logits.device)
    else:
        _check_out(ids, (t, topk), torch.int32, logits.device, "ids")
        if not ids.is_contiguous():
            raise ValueError("ids must be contiguous")
    if experts is None:
        experts = torch.empty(budget, dtype=torch.int32, device=logits.device)
    else:
        _check_out(experts, (budget,), torch.int32, logits.device, "experts")
    _check("q3_moe_budget_topk", lib().q3_moe_budget_topk(logits.data_ptr(), t, E, topk, budget, ids.data_ptr(),
                                                          experts.data_ptr(), _stream(logits)))
    return ids, experts


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
           lib().q3_grouped_expert_gemv(ctypes.byref(d), x.data_ptr(), _ld(x), 1 if x_by_slot else 0,
                                        topk_ids.data_ptr(), t, topk, y.data_ptr(), _ld(y), _stream(x)))
    return y


def moe_mlp_workspace(gate_up: ExpertStack, down: ExpertStack, t: int, topk: int, device) -> torch.Tensor:
    """Workspace for q3_moe_mlp (reusable across calls in stream order)."""
    nbytes = lib().q3_moe_mlp_workspace_bytes(gate_up.n, down.n, t, topk)
    if nbytes <= 0:
        raise ValueError("unsupported fused-MLP shape")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def q3_moe_mlp(gate_up: ExpertStack, down: ExpertStack, x: torch.Tensor, topk_ids: torch.Tensor,
               logits: torch.Tensor, workspace: torch.Tensor = None, out: torch.Tensor = None) -> torch.Tensor:
    """Fused expert MLP of a verify round: out[t] = sum_j p[t][j] * down_e . (silu(gate_e . x[t]) * (up_e . x[t]))."""
    _dev(x, "x"), _dev(topk_ids, "topk_ids"), _dev(logits, "logits")
    t, topk = topk_ids.shape
    if topk_ids.dtype != torch.int32 or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be contiguous int32 [t][topk]")
    if x.dim() != 2 or x.shape[1] != gate_up.k or x.stride(1) != 1 or x.shape[0] < t:
        raise ValueError("x must be [t][k] with contiguous rows")
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1 or logits.shape[0] < t:
        raise ValueError("logits must be fp32 [t][num_experts] with contiguous rows")
    if workspace is None:
        workspace = moe_mlp_workspace(gate_up, down, t, topk, x.device)
    else:
        _workspace(workspace, x.device)
    out = _out(out, t, down.n, x.device, "out")
    gd, dd = gate_up.desc(), down.desc()
    _check("q3_moe_mlp", lib().q3_moe_mlp(ctypes.byref(gd), ctypes.byref(dd), x.data_ptr(), _ld(x),
                                          topk_ids.data_ptr(), t, topk, logits.data_ptr(), _ld(logits),
                                          workspace.data_ptr(), _nbytes(workspace), out.data_ptr(), _ld(out),
                                          _stream(x)))
    return out


def q3_moe_mlp_noalloc(gate_up: ExpertStack, down: ExpertStack, x: torch.Tensor, topk_ids: torch.Tensor,
                       logits: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
    """q3_moe_mlp with the library's own scratch memory instead of a workspace
    (for callers that cannot allocate; calls that overlap on one GPU race)."""
    _dev(x, "x"), _dev(topk_ids, "topk_ids"), _dev(logits, "logits")
    t, topk = topk_ids.shape
    if topk_ids.dtype != torch.int32 or not topk_ids.is_contiguous():
        raise ValueError("topk_ids must be contiguous int32 [t][topk]")
    if x.dim() != 2 or x.shape[1] != gate_up.k or x.stride(1) != 1 or x.shape[0] < t:
        raise ValueError("x must be [t][k] with contiguous rows")
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.stride(1) != 1 or logits.shape[0] < t:
        raise ValueError("logits must be fp32 [t][num_experts] with contiguous rows")
    out = _out(out, t, down.n, x.device, "out")
    gd, dd = gate_up.desc(), down.desc()
    _check("q3_moe_mlp_noalloc", lib().q3_moe_mlp_noalloc(ctypes.byref(gd), ctypes.byref(dd), x.data_ptr(), _ld(x),
                                                          topk_ids.data_ptr(), t, topk, logits.data_ptr(),
                                                          _ld(logits), out.data_ptr(), _ld(out), _stream(x)))
    return out


def q3_moe_mlp_noalloc_max_bytes() -> int:
    return lib().q3_moe_mlp_noalloc_max_bytes()


# ------------------------------------------------------- two-bit draft head

def q3_layout2(n: int, k: int) -> dict:
    info = Q3LayoutInfo()
    _check("q3_layout2", lib().q3_layout2(n, k, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in Q3LayoutInfo._fields_}


@dataclass
class PackedHead2:
    """Device-resident 2-bit copy of a draft head (planes as uint8 tensors, codebook [n][4])."""
    n: int
    k: int
    code_plane: torch.Tensor
    scale_plane: torch.Tensor
    codebook: torch.Tensor

    def desc(self) -> Q3Matrix:
        return Q3Matrix(self.n, self.k, self.code_plane.data_ptr(), self.scale_plane.data_ptr(),
                        self.codebook.data_ptr())

    @property
    def payload_bytes(self) -> int:
        return self.n * self.k * 9 // 32


@dataclass
class Mxfp8Head:
    """The FP8 (MXFP8) head: elements uint8 [n][k] E4M3FN, scales uint8 [n][k/32] E8M0."""
    n: int
    k: int
    elements: torch.Tensor
    scales: torch.Tensor

    def desc(self) -> Q3Mxfp8Matrix:
        return Q3Mxfp8Matrix(self.n, self.k, self.elements.data_ptr(), _ld(self.elements),
                             self.scales.data_ptr(), _ld(self.scales))


def q3_pack2(codes: torch.Tensor, scales: torch.Tensor, codebook: torch.Tensor) -> PackedHead2:
    """codes uint8 [n][k] (0..3), scales uint8 [n][k/32], codebook uint8 [n][4] -> PackedHead2."""
    _dev(codes, "codes"), _dev(scales, "scales"), _dev(codebook, "codebook")
    n, k = codes.shape
    if codes.stride(1) != 1 or scales.stride(1) != 1:
        raise ValueError("codes and scales rows must be contiguous")
    L = q3_layout2(n, k)
    w = PackedHead2(n, k, torch.empty(L["code_plane_bytes"], dtype=torch.uint8, device=codes.device),
                    torch.empty(L["scale_plane_bytes"], dtype=torch.uint8, device=codes.device),
                    codebook.contiguous().clone())
    _check("q3_pack2", lib().q3_pack2(codes.data_ptr(), _ld(codes), scales.data_ptr(), _ld(scales), n, k,
                                      w.code_plane.data_ptr(), w.scale_plane.data_ptr(), _stream(codes)))
    return w


def q3_unpack2(w: PackedHead2):
    codes = torch.empty((w.n, w.k), dtype=torch.uint8, device=w.code_plane.device)
    scales = torch.empty((w.n, w.k // 32), dtype=torch.uint8, device=w.code_plane.device)
    d = w.desc()
    _check("q3_unpack2", lib().q3_unpack2(ctypes.byref(d), codes.data_ptr(), scales.data_ptr(),
                                          _stream(w.code_plane)))
    return codes, scales


def q3_head2_scores(w: PackedHead2, x: torch.Tensor, y: torch.Tensor = None) -> torch.Tensor:
    """2-bit scores of every row: y[m][n] = x[m] . w2[n], m <= 16."""
    x = _tokens(x, w.k)
    m = x.shape[0]
    y = _out(y, m, w.n, x.device)
    d = w.desc()
    _check("q3_head2_scores", lib().q3_head2_scores(ctypes.byref(d), x.data_ptr(), m, _ld(x), y.data_ptr(),
                                                    _ld(y), _stream(x)))
    return y


def q3_shortlist(scores: torch.Tensor, size: int = 16, workspace: torch.Tensor = None):
    """Per query the `size` rows with the largest scores (ties to the lower row) -> (ids int32, vals fp32)."""
    _dev(scores, "scores")
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be float32 [m][n] with contiguous rows")
    m, n = scores.shape
    if workspace is None:
        workspace = torch.empty(lib().q3_shortlist_workspace_bytes(m), dtype=torch.uint8, device=scores.device)
    else:
        _workspace(workspace, scores.device)
    ids = torch.empty((m, size), dtype=torch.int32, device=scores.device)
    vals = torch.empty((m, size), dtype=torch.float32, device=scores.device)
    _check("q3_shortlist", lib().q3_shortlist(scores.data_ptr(), m, n, _ld(scores), size, workspace.data_ptr(),
                                              _nbytes(workspace), ids.data_ptr(), vals.data_ptr(),
                                              _stream(scores)))
    return ids, vals


def q3_rescore_fp8(h: Mxfp8Head, x: torch.Tensor, ids: torch.Tensor):
    """FP8 scores of listed rows and the decision -> (y8 fp32 [m][size], best int32 [m])."""
    x = _tokens(x, h.k)
    _dev(ids, "ids")
    if ids.dtype != torch.int32 or not ids.is_contiguous():
        raise ValueError("ids must be contiguous int32 [m][size]")
    m, size = ids.shape
    y = torch.empty((m, size), dtype=torch.float32, device=x.device)
    best = torch.empty(m, dtype=torch.int32, device=x.device)
    d = h.desc()
    _check("q3_rescore_fp8", lib().q3_rescore_fp8(ctypes.byref(d), x.data_ptr(), m, _ld(x), ids.data_ptr(), size,
                                                  y.data_ptr(), best.data_ptr(), _stream(x)))
    return y, best


def draft_head_workspace(m: int, n: int, device) -> torch.Tensor:
    return torch.empty(lib().q3_draft_head_workspace_bytes(m, n), dtype=torch.uint8, device=device)


def q3_draft_head(w2: PackedHead2, h: Mxfp8Head, x: torch.Tensor, size: int = 16, workspace: torch.Tensor = None):
    """2-bit shortlist, FP8 rescoring and decision -> (ids int32 [m][size], y8 fp32 [m][size], best int32 [m])."""
    x = _tokens(x, w2.k)
    m = x.shape[0]
    if workspace is None:
        workspace = draft_head_workspace(m, w2.n, x.device)
    else:
        _workspace(workspace, x.device)
    ids = torch.empty((m, size), dtype=torch.int32, device=x.device)
    y8 = torch.empty((m, size), dtype=torch.float32, device=x.device)
    best = torch.empty(m, dtype=torch.int32, device=x.device)
    d2, d8 = w2.desc(), h.desc()
    _check("q3_draft_head", lib().q3_draft_head(ctypes.byref(d2), ctypes.byref(d8), x.data_ptr(), m, _ld(x),
                                                size, workspace.data_ptr(), _nbytes(workspace), ids.data_ptr(),
                                                y8.data_ptr(), best.data_ptr(), _stream(x)))
    return ids, y8, best
