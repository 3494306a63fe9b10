"""Batch-invariant W8A16 decode projection for MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI of libw8inv.so (include/w8inv.h).  Each
function has the name of the C entry point it calls and only marshals
arguments: torch tensors supply device memory and the current HIP stream; every
step of the computation runs in the library's HIP kernels.  There is no other
implementation behind these names: if the library is missing, importing this
package raises.

Storage formats: int8 weight codes; fp16 scales (torch.float16, or their bit
patterns as torch.int16); bf16 activations and logits (torch.bfloat16); int64 targets.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw8inv.so")

W8I_OK = 0
STATUS = {0: "W8I_OK", -1: "W8I_ENULL", -2: "W8I_ESHAPE", -3: "W8I_EALIGN", -4: "W8I_ET", -5: "W8I_EBLOCK",
          -6: "W8I_EWORKSPACE", -7: "W8I_EHIP", -8: "W8I_ESCRATCH"}

EXPORTS = ("w8i_status_string", "w8i_version", "w8_linear_invariant_workspace_bytes", "w8_linear_invariant",
           "w8_linear_invariant_kernel", "w8_linear_add_invariant", "w8_linear_swiglu_invariant",
           "w8_pack_bytes", "w8_pack", "w8_linear_invariant_packed", "w8_linear_invariant_packed_kernel",
           "w8_linear_add_invariant_packed", "w8_linear_swiglu_invariant_packed",
           "vocab_block_logprob_workspace_bytes", "vocab_block_logprob", "vocab_block_logprob_direct",
           "vocab_argmax_workspace_bytes", "vocab_argmax", "w8i_rmsnorm", "w8i_swiglu",
           "w8i_residual_add", "w8i_exp32", "w8i_log32", "vocab_block_logprob_noalloc",
           "w8_linear_pair_invariant", "w8_linear_pair_invariant_packed", "w8_attn_input_proj_workspace_bytes",
           "w8_attn_input_proj_invariant", "w8_attn_input_proj_invariant_packed", "w8_head_logprob_workspace_bytes",
           "w8_head_logprob_invariant", "w8_head_logprob_invariant_packed",
           "w8_linear_invariant_packed_workspace_bytes")


class W8InvError(ValueError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {status} ({_lib.w8i_status_string(status).decode()})")


def _load(path: str = LIB_PATH):
    """Open a build of the library at `path` and declare the C signatures of its entry points."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(path)
    P, I32, I64, SZ, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    L.w8i_status_string.argtypes, L.w8i_status_string.restype = [ctypes.c_int], ctypes.c_char_p
    L.w8i_version.argtypes, L.w8i_version.restype = [], ctypes.c_char_p
    L.w8_linear_invariant_workspace_bytes.argtypes = [I64, I64, I32]
    L.w8_linear_invariant_workspace_bytes.restype = SZ
    L.w8_linear_invariant.argtypes = [P, P, P, I32, I32, P, I64, I64, I64, I64, P, SZ, P]
    L.w8_linear_invariant.restype = ctypes.c_int
    L.w8_linear_invariant_kernel.argtypes, L.w8_linear_invariant_kernel.restype = [I64, I64, I32, P], ctypes.c_char_p
    L.w8_linear_add_invariant.argtypes = [P, P, P, P, I32, I32, P, I64, I64, I64, I64, I64, P]
    L.w8_linear_swiglu_invariant.argtypes = [P, P, P, I32, I32, P, I64, I64, I64, I64, P]
    L.w8_pack_bytes.argtypes = [I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
    L.w8_pack.argtypes = [P, P, I64, I64, P, P, P]
    L.w8_linear_invariant_packed.argtypes = [P, P, P, I32, I32, P, I64, I64, I64, I64, P, SZ, P]
    L.w8_linear_invariant_packed_workspace_bytes.argtypes = [I64, I64, I32]
    L.w8_linear_invariant_packed_workspace_bytes.restype = SZ
    L.w8_linear_add_invariant_packed.argtypes = [P, P, P, P, I32, I32, P, I64, I64, I64, I64, I64, P]
    L.w8_linear_swiglu_invariant_packed.argtypes = [P, P, P, I32, I32, P, I64, I64, I64, I64, P]
    L.w8_linear_invariant_packed_kernel.argtypes = [I64, I64, I32]
    L.w8_linear_invariant_packed_kernel.restype = ctypes.c_char_p
    L.vocab_block_logprob_workspace_bytes.argtypes = [I32, I64, I32]
    L.vocab_block_logprob_workspace_bytes.restype = SZ
    L.vocab_block_logprob.argtypes = [P, P, I32, P, I32, I64, I64, P, SZ, P]
    L.vocab_block_logprob.restype = ctypes.c_int
    L.vocab_block_logprob_direct.argtypes = [P, P, I32, P, I32, I64, I64, P, SZ, P]
    L.vocab_block_logprob_direct.restype = ctypes.c_int
    L.w8_linear_pair_invariant.argtypes = [P, P, P, P, P, I32, I32, P, P, I64, I64, I64, I64, I64, I64, P]
    L.w8_linear_pair_invariant_packed.argtypes = [P, P, P, P, P, I32, I32, P, P, I64, I64, I64, I64, I64, I64, P]
    L.w8_attn_input_proj_workspace_bytes.argtypes = [I32, I64]
    L.w8_attn_input_proj_workspace_bytes.restype = SZ
    L.w8_attn_input_proj_invariant.argtypes = [P, P, F32, P, P, I32, I32, P, I64, I64, I64, I64, P, SZ, P]
    L.w8_attn_input_proj_invariant_packed.argtypes = [P, P, F32, P, P, I32, I32, P, I64, I64, I64, I64, P, SZ, P]
    for name in ("w8_linear_pair_invariant", "w8_linear_pair_invariant_packed", "w8_attn_input_proj_invariant",
                 "w8_attn_input_proj_invariant_packed"):
        getattr(L, name).restype = ctypes.c_int
    L.w8_head_logprob_workspace_bytes.argtypes = [I32, I64, I32]
    L.w8_head_logprob_workspace_bytes.restype = SZ
    for name in ("w8_head_logprob_invariant", "w8_head_logprob_invariant_packed"):
        getattr(L, name).argtypes = [P, P, P, P, I32, I32, I32, P, P, I64, I64, I64, I64, P, SZ, P]
        getattr(L, name).restype = ctypes.c_int
    L.vocab_block_logprob_noalloc.argtypes = [P, P, I32, P, I32, I64, I64, P]
    L.vocab_block_logprob_noalloc.restype = ctypes.c_int
    L.vocab_argmax_workspace_bytes.argtypes, L.vocab_argmax_workspace_bytes.restype = [I32, I64], SZ
    L.vocab_argmax.argtypes, L.vocab_argmax.restype = [P, P, I32, I64, I64, P, SZ, P], ctypes.c_int
    L.w8i_rmsnorm.argtypes = [P, P, F32, P, I32, I64, I64, I64, P]
    L.w8i_swiglu.argtypes = [P, P, I32, I64, I64, I64, P]
    L.w8i_residual_add.argtypes = [P, P, P, I32, I64, I64, I64, I64, P]
    L.w8i_exp32.argtypes = [P, P, I64, P]
    L.w8i_log32.argtypes = [P, P, I64, P]
    for name in ("w8_linear_add_invariant", "w8_linear_swiglu_invariant", "w8_pack_bytes", "w8_pack",
                 "w8_linear_invariant_packed", "w8_linear_add_invariant_packed", "w8_linear_swiglu_invariant_packed",
                 "w8i_rmsnorm", "w8i_swiglu", "w8i_residual_add", "w8i_exp32", "w8i_log32"):
        getattr(L, name).restype = ctypes.c_int
    return L


_lib = _load()


def lib():
    return _lib


def _check(fn: str, status: int):
    if status != W8I_OK:
        raise W8InvError(fn, status)


def _launch(fn, device, *args):
    """Call library function `fn` with `device` current and its current stream as the last argument
    (HIP launches on a stream of the current device; the library also sizes some grids from it)."""
    with torch.cuda.device(device):
        return fn(*args, ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _row_major(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    return t.stride(0) if t.size(0) > 1 else max(t.stride(0), t.size(1))


def _same_gpu(*named):
    """Every tensor must live on one GPU: a host pointer must never reach a kernel."""
    dev = None
    for name, ten in named:
        if ten is None:
            continue
        if not isinstance(ten, torch.Tensor) or ten.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA (HIP) tensor")
        if dev is None:
            dev = ten.device
        elif ten.device != dev:
            raise ValueError(f"{name} is on {ten.device}, expected {dev}")


def _dtype(ten, name, *dtypes):
    if ten is not None and ten.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {ten.dtype}")


def version() -> str:
    return _lib.w8i_version().decode()


def _projection_args(W_q, scales, x, t, y, y_cols):
    if W_q.dtype != torch.int8 or W_q.dim() != 2 or not W_q.is_contiguous():
        raise ValueError("W_q must be a contiguous int8 [N, K] tensor")
    N, K = W_q.shape
    if scales.dtype not in (torch.float16, torch.int16) or tuple(scales.shape) != (N, K // 32) \
            or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous fp16 [N, K/32] tensor")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.size(1) != K or x.size(0) < t:
        raise ValueError("x must be a bf16 [>=t, K] tensor")
    ldx = _row_major(x, "x")
    if y is None:
        y = torch.empty((t, y_cols), dtype=torch.bfloat16, device=W_q.device)
    if y.dtype != torch.bfloat16 or y.dim() != 2 or y.size(1) != y_cols or y.size(0) < t:
        raise ValueError(f"y must be a bf16 [>=t, {y_cols}] tensor")
    ldy = _row_major(y, "y")
    _same_gpu(("W_q", W_q), ("scales", scales), ("x", x), ("y", y))
    return N, K, ldx, y, ldy


def _projection_workspace(workspace, need: int, device):
    """The optional workspace of a projection: None passes none (the one-launch kernel runs), "auto"
    allocates the queried size (none if it is 0; small N then runs its K-slices on separate workgroups
    and a fold launch), a contiguous uint8 tensor is used as given."""
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a uint8 tensor')
        return torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None
    if workspace is not None and (workspace.dtype != torch.uint8 or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor")
    return workspace


def w8_linear_invariant_workspace_bytes(N: int, K: int, T_pad: int) -> int:
    return int(_lib.w8_linear_invariant_workspace_bytes(int(N), int(K), int(T_pad)))


def w8_linear_invariant_packed_workspace_bytes(N: int, K: int, T_pad: int) -> int:
    return int(_lib.w8_linear_invariant_packed_workspace_bytes(int(N), int(K), int(T_pad)))


def w8_linear_invariant(W_q: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, t: int, T_pad: int,
                        y: torch.Tensor | None = None, workspace=None) -> torch.Tensor:
    """y[:t] = bf16(dequant(W_q, scales) @ x[:t]^T) at the fixed width T_pad.

    W_q int8 [N, K]; scales fp16 [N, K/32]; x bf16 [>=t, K] (token rows); y bf16 [t, N] (allocated if None).
    workspace: None (the one-launch kernel), "auto" (the size w8_linear_invariant_workspace_bytes asks for;
    small N then runs its K-slices on separate workgroups and a fold launch), or a uint8 tensor.  The bits
    do not depend on it.
    """
    N, K, ldx, y, ldy = _projection_args(W_q, scales, x, t, y, W_q.shape[0])
    ws = _projection_workspace(workspace, w8_linear_invariant_workspace_bytes(N, K, T_pad), W_q.device)
    if ws is not None:
        _same_gpu(("W_q", W_q), ("workspace", ws))
    st = _launch(_lib.w8_linear_invariant, W_q.device, _ptr(W_q), _ptr(scales), _ptr(x), int(t), int(T_pad), _ptr(y),
                 N, K, ldx, ldy, _ptr(ws), ws.numel() if ws is not None else 0)
    _check("w8_linear_invariant", st)
    return y


def w8_linear_add_invariant(W_q: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, residual: torch.Tensor,
                            t: int, T_pad: int, y: torch.Tensor | None = None) -> torch.Tensor:
    """y[:t] = residual add of w8_linear_invariant(...) and residual[:t]; y may be `residual` itself."""
    N, K, ldx, y, ldy = _projection_args(W_q, scales, x, t, y, W_q.shape[0])
    _same_gpu(("W_q", W_q), ("residual", residual))
    if residual.dtype != torch.bfloat16 or residual.dim() != 2 or residual.size(1) != N or residual.size(0) < t:
        raise ValueError("residual must be a bf16 [>=t, N] tensor")
    st = _launch(_lib.w8_linear_add_invariant, W_q.device, _ptr(W_q), _ptr(scales), _ptr(x), _ptr(residual), int(t),
                 int(T_pad), _ptr(y), N, K, ldx, _row_major(residual, "residual"), ldy)
    _check("w8_linear_add_invariant", st)
    return y


def w8_linear_swiglu_invariant(W_q: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, t: int, T_pad: int,
                               y: torch.Tensor | None = None) -> torch.Tensor:
    """y[:t] = SwiGLU of the gate+up projection: W_q int8 [2F, K] (gate rows, then up rows); y bf16 [t, F]."""
    if W_q.dim() != 2 or W_q.shape[0] % 2:
        raise ValueError("W_q must be [2F, K]")
    F = W_q.shape[0] // 2
    N, K, ldx, y, ldy = _projection_args(W_q, scales, x, t, y, F)
    st = _launch(_lib.w8_linear_swiglu_invariant, W_q.device, _ptr(W_q), _ptr(scales), _ptr(x), int(t), int(T_pad),
                 _ptr(y), F, K, ldx, ldy)
    _check("w8_linear_swiglu_invariant", st)
    return y


def w8_pack_bytes(N: int, K: int) -> tuple[int, int]:
    """(codes bytes, scale bytes) of the packed layout of an [N, K] projection."""
    wb, sb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check("w8_pack_bytes", _lib.w8_pack_bytes(int(N), int(K), ctypes.byref(wb), ctypes.byref(sb)))
    return wb.value, sb.value


def w8_pack(W_q: torch.Tensor, scales: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """The packed layout (Wp int8, Sp fp16-as-int16) of W_q int8 [N, K] and scales fp16 [N, K/32]."""
    if W_q.dtype != torch.int8 or W_q.dim() != 2 or not W_q.is_contiguous():
        raise ValueError("W_q must be a contiguous int8 [N, K] tensor")
    N, K = W_q.shape
    if scales.dtype not in (torch.float16, torch.int16) or tuple(scales.shape) != (N, K // 32) \
            or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous fp16 [N, K/32] tensor")
    _same_gpu(("W_q", W_q), ("scales", scales))
    wb, sb = w8_pack_bytes(N, K)
    Wp = torch.empty(wb, dtype=torch.int8, device=W_q.device)
    Sp = torch.empty(sb // 2, dtype=torch.int16, device=W_q.device)
    _check("w8_pack", _launch(_lib.w8_pack, W_q.device, _ptr(W_q), _ptr(scales), N, K, _ptr(Wp), _ptr(Sp)))
    return Wp, Sp


def _packed_args(Wp, Sp, x, t, N, rows, y, y_cols):
    """Checks of a packed-layout call: Wp / Sp from w8_pack of a [rows, K] projection."""
    K = x.size(1)
    wb, sb = w8_pack_bytes(rows, K)
    if Wp.dtype != torch.int8 or Wp.numel() != wb or not Wp.is_contiguous():
        raise ValueError("Wp must be the contiguous int8 output of w8_pack for this shape")
    if Sp.dtype not in (torch.int16, torch.float16) or Sp.numel() * 2 != sb or not Sp.is_contiguous():
        raise ValueError("Sp must be the contiguous output of w8_pack for this shape")
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.size(0) < t:
        raise ValueError("x must be a bf16 [>=t, K] tensor")
    if y is None:
        y = torch.empty((t, y_cols), dtype=torch.bfloat16, device=Wp.device)
    if y.dtype != torch.bfloat16 or y.dim() != 2 or y.size(1) != y_cols or y.size(0) < t:
        raise ValueError(f"y must be a bf16 [>=t, {y_cols}] tensor")
    _same_gpu(("Wp", Wp), ("Sp", Sp), ("x", x), ("y", y))
    return K, y


def w8_linear_invariant_packed(Wp: torch.Tensor, Sp: torch.Tensor, x: torch.Tensor, t: int, T_pad: int, N: int,
                               y: torch.Tensor | None = None, workspace=None) -> torch.Tensor:
    """w8_linear_invariant over the packed layout from w8_pack (same bits).  x bf16 [>=t, K]; y bf16 [t, N];
    workspace as for w8_linear_invariant."""
    K, y = _packed_args(Wp, Sp, x, t, N, N, y, N)
    ws = _projection_workspace(workspace, w8_linear_invariant_packed_workspace_bytes(N, K, T_pad), Wp.device)
    if ws is not None:
        _same_gpu(("Wp", Wp), ("workspace", ws))
    st = _launch(_lib.w8_linear_invariant_packed, Wp.device, _ptr(Wp), _ptr(Sp), _ptr(x), int(t), int(T_pad), _ptr(y),
                 int(N), K, _row_major(x, "x"), _row_major(y, "y"), _ptr(ws), ws.numel() if ws is not None else 0)
    _check("w8_linear_invariant_packed", st)
    return y


def w8_linear_add_invariant_packed(Wp: torch.Tensor, Sp: torch.Tensor, x: torch.Tensor, residual: torch.Tensor,
                                   t: int, T_pad: int, N: int, y: torch.Tensor | None = None) -> torch.Tensor:
    """w8_linear_add_invariant over the packed layout (same bits); y may be `residual` itself."""
    K, y = _packed_args(Wp, Sp, x, t, N, N, y, N)
    _same_gpu(("Wp", Wp), ("residual", residual))
    if residual.dtype != torch.bfloat16 or residual.dim() != 2 or residual.size(1) != N or residual.size(0) < t:
        raise ValueError("residual must be a bf16 [>=t, N] tensor")
    st = _launch(_lib.w8_linear_add_invariant_packed, Wp.device, _ptr(Wp), _ptr(Sp), _ptr(x), _ptr(residual), int(t),
                 int(T_pad), _ptr(y), int(N), K, _row_major(x, "x"), _row_major(residual, "residual"),
                 _row_major(y, "y"))
    _check("w8_linear_add_invariant_packed", st)
    return y


def w8_linear_swiglu_invariant_packed(Wp: torch.Tensor, Sp: torch.Tensor, x: torch.Tensor, t: int, T_pad: int,
                                      F: int, y: torch.Tensor | None = None) -> torch.Tensor:
    """w8_linear_swiglu_invariant over the packed layout of the [2F, K] gate+up projection (same bits)."""
    K, y = _packed_args(Wp, Sp, x, t, F, 2 * F, y, F)
    st = _launch(_lib.w8_linear_swiglu_invariant_packed, Wp.device, _ptr(Wp), _ptr(Sp), _ptr(x), int(t), int(T_pad),
                 _ptr(y), int(F), K, _row_major(x, "x"), _row_major(y, "y"))
    _check("w8_linear_swiglu_invariant_packed", st)
    return y


def w8_linear_pair_invariant(Wa: torch.Tensor, Sa: torch.Tensor, Wb: torch.Tensor, Sb: torch.Tensor,
                             x: torch.Tensor, t: int, T_pad: int, ya: torch.Tensor | None = None,
                             yb: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Two projections of the same x in one launch: (w8_linear_invariant(Wa, Sa, x), w8_linear_invariant(Wb, Sb, x)),
    bit for bit.  Wa int8 [Na, K], Wb int8 [Nb, K] with their fp16 scales; x bf16 [>=t, K]."""
    Na, K, ldx, ya, ldya = _projection_args(Wa, Sa, x, t, ya, Wa.shape[0])
    Nb, Kb, _, yb, ldyb = _projection_args(Wb, Sb, x, t, yb, Wb.shape[0])
    if Kb != K:
        raise ValueError("Wa and Wb must have the same K")
    st = _launch(_lib.w8_linear_pair_invariant, Wa.device, _ptr(Wa), _ptr(Sa), _ptr(Wb), _ptr(Sb), _ptr(x), int(t),
                 int(T_pad), _ptr(ya), _ptr(yb), Na, Nb, K, ldx, ldya, ldyb)
    _check("w8_linear_pair_invariant", st)
    return ya, yb


def w8_linear_pair_invariant_packed(Wpa: torch.Tensor, Spa: torch.Tensor, Wpb: torch.Tensor, Spb: torch.Tensor,
                                    x: torch.Tensor, t: int, T_pad: int, Na: int, Nb: int,
                                    ya: torch.Tensor | None = None,
                                    yb: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """w8_linear_pair_invariant over two projections in the packed layout (w8_pack of each); same bits."""
    K, ya = _packed_args(Wpa, Spa, x, t, Na, Na, ya, Na)
    _, yb = _packed_args(Wpb, Spb, x, t, Nb, Nb, yb, Nb)
    st = _launch(_lib.w8_linear_pair_invariant_packed, Wpa.device, _ptr(Wpa), _ptr(Spa), _ptr(Wpb), _ptr(Spb),
                 _ptr(x), int(t), int(T_pad), _ptr(ya), _ptr(yb), int(Na), int(Nb), K, _row_major(x, "x"),
                 _row_major(ya, "ya"), _row_major(yb, "yb"))
    _check("w8_linear_pair_invariant_packed", st)
    return ya, yb


def w8_attn_input_proj_workspace_bytes(t: int, H: int) -> int:
    return int(_lib.w8_attn_input_proj_workspace_bytes(int(t), int(H)))


def _attn_input_proj(packed, h, norm_weight, eps, W, S, t, T_pad, N, y, workspace):
    if h.dtype != torch.bfloat16 or h.dim() != 2 or h.size(0) < t:
        raise ValueError("h must be a bf16 [>=t, H] tensor")
    H = h.size(1)
    _dtype(norm_weight, "norm_weight", torch.bfloat16)
    if norm_weight is not None and (norm_weight.numel() < H or not norm_weight.is_contiguous()):
        raise ValueError("norm_weight must be a contiguous bf16 [H] tensor")
    if y is None:
        y = torch.empty((t, N), dtype=torch.bfloat16, device=h.device)
    if y.dtype != torch.bfloat16 or y.dim() != 2 or y.size(1) != N or y.size(0) < t:
        raise ValueError(f"y must be a bf16 [>=t, {N}] tensor")
    need = w8_attn_input_proj_workspace_bytes(t, H)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=h.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    _same_gpu(("h", h), ("norm_weight", norm_weight), ("W", W), ("S", S), ("y", y), ("workspace", workspace))
    fn = _lib.w8_attn_input_proj_invariant_packed if packed else _lib.w8_attn_input_proj_invariant
    st = _launch(fn, h.device, _ptr(h), _ptr(norm_weight), float(eps), _ptr(W), _ptr(S), int(t), int(T_pad), _ptr(y),
                 int(N), H, _row_major(h, "h"), _row_major(y, "y"), _ptr(workspace), workspace.numel())
    _check("w8_attn_input_proj_invariant" + ("_packed" if packed else ""), st)
    return y


def w8_attn_input_proj_invariant(h: torch.Tensor, norm_weight: torch.Tensor | None, eps: float, W_q: torch.Tensor,
                                 scales: torch.Tensor, t: int, T_pad: int, y: torch.Tensor | None = None,
                                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[:t] = w8_linear_invariant(W_q, scales, w8i_rmsnorm(h, eps, norm_weight)) bit for bit (one call, the
    normalised activations in `workspace`).  h bf16 [>=t, H]; W_q int8 [N, H]; scales fp16 [N, H/32]."""
    if W_q.dtype != torch.int8 or W_q.dim() != 2 or not W_q.is_contiguous():
        raise ValueError("W_q must be a contiguous int8 [N, H] tensor")
    if scales.dtype not in (torch.float16, torch.int16) or tuple(scales.shape) != (W_q.shape[0], W_q.shape[1] // 32):
        raise ValueError("scales must be fp16 [N, H/32]")
    if W_q.shape[1] != h.size(1):
        raise ValueError("W_q must have H columns")
    return _attn_input_proj(False, h, norm_weight, eps, W_q, scales, t, T_pad, W_q.shape[0], y, workspace)


def w8_attn_input_proj_invariant_packed(h: torch.Tensor, norm_weight: torch.Tensor | None, eps: float,
                                        Wp: torch.Tensor, Sp: torch.Tensor, t: int, T_pad: int, N: int,
                                        y: torch.Tensor | None = None,
                                        workspace: torch.Tensor | None = None) -> torch.Tensor:
    """w8_attn_input_proj_invariant over weights packed by w8_pack (same bits)."""
    wb, sb = w8_pack_bytes(N, h.size(1))
    if Wp.dtype != torch.int8 or Wp.numel() != wb or Sp.numel() * 2 != sb:
        raise ValueError("Wp / Sp must be the output of w8_pack for [N, H]")
    return _attn_input_proj(True, h, norm_weight, eps, Wp, Sp, t, T_pad, int(N), y, workspace)


def w8_head_logprob_workspace_bytes(t: int, V: int, block: int) -> int:
    return int(_lib.w8_head_logprob_workspace_bytes(int(t), int(V), int(block)))


def _head_logprob(packed, W, S, x, targets, t, T_pad, block, V, K, logits, out, workspace):
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.size(1) != K or x.size(0) < t:
        raise ValueError("x must be a bf16 [>=t, K] tensor")
    if targets.dtype != torch.int64 or targets.numel() < t or not targets.is_contiguous():
        raise ValueError("targets must be a contiguous int64 [t] tensor")
    if logits is None:
        logits = torch.empty((t, V), dtype=torch.bfloat16, device=x.device)
    if logits.dtype != torch.bfloat16 or logits.dim() != 2 or logits.size(1) != V or logits.size(0) < t:
        raise ValueError(f"logits must be a bf16 [>=t, {V}] tensor")
    if out is None:
        out = torch.empty(t, dtype=torch.float32, device=x.device)
    _dtype(out, "out", torch.float32)
    if out.numel() < t or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [t] tensor")
    need = w8_head_logprob_workspace_bytes(t, V, block)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    _same_gpu(("W", W), ("S", S), ("x", x), ("targets", targets), ("logits", logits), ("out", out),
              ("workspace", workspace))
    fn = _lib.w8_head_logprob_invariant_packed if packed else _lib.w8_head_logprob_invariant
    st = _launch(fn, x.device, _ptr(W), _ptr(S), _ptr(x), _ptr(targets), int(t), int(T_pad), int(block), _ptr(logits),
                 _ptr(out), int(V), int(K), _row_major(x, "x"), _row_major(logits, "logits"), _ptr(workspace),
                 workspace.numel())
    _check("w8_head_logprob_invariant" + ("_packed" if packed else ""), st)
    return logits, out


def w8_head_logprob_invariant(W_q: torch.Tensor, scales: torch.Tensor, x: torch.Tensor, targets: torch.Tensor, t: int,
                              T_pad: int, block: int, logits: torch.Tensor | None = None,
                              out: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """(logits, logprob): the LM head w8_linear_invariant(W_q, scales, x) fused with the row-max pass of
    vocab_block_logprob(logits, targets, block); both bit for bit the unfused results."""
    if W_q.dtype != torch.int8 or W_q.dim() != 2 or not W_q.is_contiguous():
        raise ValueError("W_q must be a contiguous int8 [V, K] tensor")
    V, K = W_q.shape
    if scales.dtype not in (torch.float16, torch.int16) or tuple(scales.shape) != (V, K // 32):
        raise ValueError("scales must be fp16 [V, K/32]")
    return _head_logprob(False, W_q, scales, x, targets, t, T_pad, block, V, K, logits, out, workspace)


def w8_head_logprob_invariant_packed(Wp: torch.Tensor, Sp: torch.Tensor, x: torch.Tensor, targets: torch.Tensor,
                                     t: int, T_pad: int, block: int, V: int, logits: torch.Tensor | None = None,
                                     out: torch.Tensor | None = None,
                                     workspace: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """w8_head_logprob_invariant over the head's weights packed by w8_pack (same bits)."""
    K = x.size(1)
    wb, sb = w8_pack_bytes(V, K)
    if Wp.dtype != torch.int8 or Wp.numel() != wb or Sp.numel() * 2 != sb:
        raise ValueError("Wp / Sp must be the output of w8_pack for [V, K]")
    return _head_logprob(True, Wp, Sp, x, targets, t, T_pad, block, int(V), K, logits, out, workspace)


def w8_linear_invariant_packed_kernel(N: int, K: int, T_pad: int) -> str:
    """Name of the kernel w8_linear_invariant_packed runs for this shape.  Host-side only."""
    return _lib.w8_linear_invariant_packed_kernel(int(N), int(K), int(T_pad)).decode()


def w8_linear_invariant_kernel(N: int, K: int, T_pad: int, scales: torch.Tensor | None = None) -> str:
    """Name of the kernel w8_linear_invariant runs for this shape (the choice also looks at whether
    `scales` is 16-byte aligned; None means aligned).  Host-side only."""
    ptr = ctypes.c_void_p(scales.data_ptr() if scales is not None else 256)
    return _lib.w8_linear_invariant_kernel(int(N), int(K), int(T_pad), ptr).decode()


def vocab_block_logprob_workspace_bytes(t: int, V: int, block: int) -> int:
    return int(_lib.vocab_block_logprob_workspace_bytes(int(t), int(V), int(block)))


def vocab_block_logprob(logits: torch.Tensor, targets: torch.Tensor, block: int, out: torch.Tensor | None = None,
                        t: int | None = None, workspace: torch.Tensor | None = None,
                        direct: bool = False) -> torch.Tensor:
    """fp32 [t] target logprobs by `block`-wide vocabulary blocks.  logits bf16 [t, V] (rows contiguous).
    direct=True calls vocab_block_logprob_direct (the +0.0 form)."""
    if logits.dtype != torch.bfloat16 or logits.dim() != 2:
        raise ValueError("logits must be a bf16 [t, V] tensor")
    t = logits.size(0) if t is None else int(t)
    V = logits.size(1)
    ldl = _row_major(logits, "logits")
    if targets.dtype != torch.int64 or targets.numel() < t or not targets.is_contiguous():
        raise ValueError("targets must be a contiguous int64 [t] tensor")
    if out is None:
        out = torch.empty(t, dtype=torch.float32, device=logits.device)
    _dtype(out, "out", torch.float32)
    if out.numel() < t or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [t] tensor")
    need = vocab_block_logprob_workspace_bytes(t, V, block)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=logits.device)
    _same_gpu(("logits", logits), ("targets", targets), ("out", out), ("workspace", workspace))
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    fn = _lib.vocab_block_logprob_direct if direct else _lib.vocab_block_logprob
    st = _launch(fn, logits.device, _ptr(logits), _ptr(targets), int(block), _ptr(out), t, V, ldl, _ptr(workspace),
                 workspace.numel())
    _check("vocab_block_logprob_direct" if direct else "vocab_block_logprob", st)
    return out


def vocab_block_logprob_direct(logits: torch.Tensor, targets: torch.Tensor, block: int, **kw) -> torch.Tensor:
    """The blockwise-direct form, target - log(sum_exp): +0.0 for a certain token."""
    return vocab_block_logprob(logits, targets, block, direct=True, **kw)


# bytes of the library's fixed device scratch used by vocab_block_logprob_noalloc (W8I_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 1 << 20


def vocab_block_logprob_noalloc(logits: torch.Tensor, targets: torch.Tensor, block: int, out: torch.Tensor,
                                t: int | None = None) -> torch.Tensor:
    """vocab_block_logprob with no workspace: the library's fixed device scratch holds the block maxima
    and partials (for callers that cannot allocate; `out` must be given).  Same bits as
    vocab_block_logprob; calls that overlap in time on one GPU race on the scratch."""
    if logits.dtype != torch.bfloat16 or logits.dim() != 2:
        raise ValueError("logits must be a bf16 [t, V] tensor")
    t = logits.size(0) if t is None else int(t)
    V = logits.size(1)
    ldl = _row_major(logits, "logits")
    if targets.dtype != torch.int64 or targets.numel() < t or not targets.is_contiguous():
        raise ValueError("targets must be a contiguous int64 [t] tensor")
    _dtype(out, "out", torch.float32)
    if out.numel() < t or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [t] tensor")
    _same_gpu(("logits", logits), ("targets", targets), ("out", out))
    st = _launch(_lib.vocab_block_logprob_noalloc, logits.device, _ptr(logits), _ptr(targets), int(block), _ptr(out),
                 t, V, ldl)
    _check("vocab_block_logprob_noalloc", st)
    return out


def vocab_argmax_workspace_bytes(t: int, V: int) -> int:
    return int(_lib.vocab_argmax_workspace_bytes(int(t), int(V)))


def vocab_argmax(logits: torch.Tensor, out: torch.Tensor | None = None, t: int | None = None,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """int64 [t]: each column's canonical greedy argmax (lowest index among equal maxima, +-0 equal,
    the first NaN if any).  logits bf16 [t, V] (rows contiguous)."""
    if logits.dtype != torch.bfloat16 or logits.dim() != 2:
        raise ValueError("logits must be a bf16 [t, V] tensor")
    t = logits.size(0) if t is None else int(t)
    V = logits.size(1)
    ldl = _row_major(logits, "logits")
    if out is None:
        out = torch.empty(t, dtype=torch.int64, device=logits.device)
    _dtype(out, "out", torch.int64)
    if out.numel() < t or not out.is_contiguous():
        raise ValueError("out must be a contiguous int64 [t] tensor")
    need = vocab_argmax_workspace_bytes(t, V)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=logits.device)
    _same_gpu(("logits", logits), ("out", out), ("workspace", workspace))
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    st = _launch(_lib.vocab_argmax, logits.device, _ptr(logits), _ptr(out), t, V, ldl, _ptr(workspace),
                 workspace.numel())
    _check("vocab_argmax", st)
    return out


def w8i_rmsnorm(x: torch.Tensor, eps: float, weight: torch.Tensor | None = None,
                y: torch.Tensor | None = None) -> torch.Tensor:
    t, H = x.shape
    ldx = _row_major(x, "x")
    y = torch.empty((t, H), dtype=torch.bfloat16, device=x.device) if y is None else y
    _same_gpu(("x", x), ("weight", weight), ("y", y))
    _dtype(x, "x", torch.bfloat16), _dtype(weight, "weight", torch.bfloat16), _dtype(y, "y", torch.bfloat16)
    if weight is not None and (weight.numel() < H or not weight.is_contiguous()):
        raise ValueError("weight must be a contiguous bf16 [H] tensor")
    if y.shape[0] < t or y.shape[1] != H:
        raise ValueError("y must be bf16 [t, H]")
    st = _launch(_lib.w8i_rmsnorm, x.device, _ptr(x), _ptr(weight), float(eps), _ptr(y), t, H, ldx, _row_major(y, "y"))
    _check("w8i_rmsnorm", st)
    return y


def w8i_swiglu(gate_up: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    t, F2 = gate_up.shape
    F = F2 // 2
    y = torch.empty((t, F), dtype=torch.bfloat16, device=gate_up.device) if y is None else y
    _same_gpu(("gate_up", gate_up), ("y", y))
    _dtype(gate_up, "gate_up", torch.bfloat16), _dtype(y, "y", torch.bfloat16)
    if y.shape[0] < t or y.shape[1] != F:
        raise ValueError("y must be bf16 [t, F]")
    st = _launch(_lib.w8i_swiglu, gate_up.device, _ptr(gate_up), _ptr(y), t, F, _row_major(gate_up, "gate_up"),
                 _row_major(y, "y"))
    _check("w8i_swiglu", st)
    return y


def w8i_residual_add(a: torch.Tensor, b: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    t, H = a.shape
    y = torch.empty((t, H), dtype=torch.bfloat16, device=a.device) if y is None else y
    _same_gpu(("a", a), ("b", b), ("y", y))
    for name, ten in (("a", a), ("b", b), ("y", y)):
        _dtype(ten, name, torch.bfloat16)
        if ten.dim() != 2 or ten.shape[0] < t or ten.shape[1] != H:
            raise ValueError(f"{name} must be bf16 [t, H]")
    st = _launch(_lib.w8i_residual_add, a.device, _ptr(a), _ptr(b), _ptr(y), t, H, _row_major(a, "a"),
                 _row_major(b, "b"), _row_major(y, "y"))
    _check("w8i_residual_add", st)
    return y


def w8i_exp32(x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    x = x.contiguous()
    y = torch.empty_like(x) if y is None else y
    _same_gpu(("x", x), ("y", y))
    _dtype(x, "x", torch.float32), _dtype(y, "y", torch.float32)
    if y.numel() < x.numel() or not y.is_contiguous():
        raise ValueError("y must be a contiguous fp32 tensor as large as x")
    _check("w8i_exp32", _launch(_lib.w8i_exp32, x.device, _ptr(x), _ptr(y), x.numel()))
    return y


def w8i_log32(x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    x = x.contiguous()
    y = torch.empty_like(x) if y is None else y
    _same_gpu(("x", x), ("y", y))
    _dtype(x, "x", torch.float32), _dtype(y, "y", torch.float32)
    if y.numel() < x.numel() or not y.is_contiguous():
        raise ValueError("y must be a contiguous fp32 tensor as large as x")
    _check("w8i_log32", _launch(_lib.w8i_log32, x.device, _ptr(x), _ptr(y), x.numel()))
    return y


def _code_only(src: str) -> str:
    """C++ source without comments, whitespace runs collapsed (string and character literals kept)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_digest() -> str:
    """SHA-256 over the GEMM kernel's code (its sources without comments or layout): identifies which
    kernel a stored counter profile measured."""
    import hashlib
    h = hashlib.sha256()
    for name in ("w8inv_gemm.hip", "w8inv_gemm_common.h", "w8inv_math.h", "w8inv_internal.h"):
        with open(os.path.join(_HERE, "csrc", name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]
