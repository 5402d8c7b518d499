"""Python binding of libsq, the SmoothQuant W8A8 linear path on MI355X (gfx950).

Every function has the name of the C entry point it calls (include/sq.h) and
only marshals arguments: torch tensors become device pointers, shapes and
row strides; the stream is torch's current stream unless one is given. All
computation happens in the HIP kernels of libsq.so. If the library is not
built, importing this package still works, but the first call raises
LibraryNotBuilt: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsq.so")

SQ_OK = 0
SQ_ERR_INVALID_ARG = -1
SQ_ERR_UNSUPPORTED_DTYPE = -2
SQ_ERR_MISALIGNED = -3
SQ_ERR_UNSUPPORTED_ARCH = -4
SQ_ERR_WORKSPACE = -5
SQ_ERR_HIP = -6

SQ_F32, SQ_F16, SQ_BF16 = 0, 1, 2
SQ_ACT_PER_TOKEN_DYNAMIC, SQ_ACT_PER_TENSOR_STATIC = 0, 1
SQ_MAX_LORA_RANK = 128
SQ_MAX_LORA_PARTS = 4

MODES = {"dynamic": SQ_ACT_PER_TOKEN_DYNAMIC, "static": SQ_ACT_PER_TENSOR_STATIC}
_DT = {torch.float32: SQ_F32, torch.float16: SQ_F16, torch.bfloat16: SQ_BF16}

# Every exported symbol and its C signature.
_c_int, _c_i64, _vp, _c_f, _c_d, _c_sz = (ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_float, ctypes.c_double, ctypes.c_size_t)
SIGNATURES = {
    "sq_query_support": (_c_int, [_c_int, ctypes.POINTER(_c_int)]),
    "sq_status_string": (ctypes.c_char_p, [_c_int]),
    "sq_calibrate_absmax": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _vp]),
    "sq_smooth_scale": (_c_int, [_vp, _vp, _c_int, _c_i64, _c_i64, _c_i64, _c_d, _vp, _vp]),
    "sq_fold_quant_weights": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _vp]),
    "sq_smooth_fold": (_c_int, [_vp, _vp, _c_int, _c_i64, _c_i64, _c_i64, _c_d, _vp, _vp, _vp, _vp]),
    "sq_static_act_scale": (_c_int, [_vp, _vp, _c_i64, _vp, _vp]),
    "sq_quant_per_token": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _c_int, _vp, _vp, _vp]),
    "sq_fold_norm_weight": (_c_int, [_vp, _vp, _c_int, _c_i64, _vp, _vp, _vp, _vp]),
    "sq_norm_quant": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp, _vp, _c_f, _c_int,
                               _vp, _vp, _vp, _vp]),
    "sq_quant_shrink": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _c_int, _vp, _vp, _vp,
                                 _c_int, _vp, _c_i64, _vp]),
    "sq_quant_static_clipped": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _vp, _vp, _vp,
                                         _vp]),
    "sq_w8a8_gemm": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _c_i64, _c_i64, _c_i64, _vp, _c_int,
                              _c_i64, _vp]),
    "sq_w8a8_gemm_i32": (_c_int, [_vp, _vp, _c_i64, _c_i64, _c_i64, _vp, _vp]),
    "sq_w8a8_gemm_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64]),
    "sq_w8a8_gemm_ws": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _c_i64, _c_i64, _c_i64, _vp, _c_int,
                                 _c_i64, _vp, _c_sz, _vp]),
    "sq_w8a8_gemm_lora": (_c_int, [_vp, _vp, _vp, _c_int, _vp, _c_i64, _c_i64, _c_i64, _vp, _c_i64,
                                   _vp, _c_int, _c_f, _vp, _c_int, _c_i64, _vp]),
    "sq_lora_shrink": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _c_int, _vp, _c_i64, _vp,
                                _c_sz, _vp]),
    "sq_lora_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_int]),
    "sq_lora_apply": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _vp, _c_int, _c_f, _vp,
                               _c_int, _c_i64, _c_i64, _vp, _c_sz, _vp]),
    "sq_lora_apply_segmented": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp, _vp,
                                         _c_int, _vp, _vp, _vp, _c_int, _c_f, _vp, _c_int, _c_i64,
                                         _c_i64, _vp, _c_sz, _vp]),
    "sq_lora_apply_segmented_noalloc": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _c_int, _vp,
                                                 _vp, _c_int, _vp, _vp, _vp, _c_int, _c_f, _vp,
                                                 _c_int, _c_i64, _c_i64, _vp]),
    "sq_linear_group_run": (_c_int, [_vp, _c_int, _vp, _vp]),
    "sq_alpha_sweep_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64]),
    "sq_alpha_sweep": (_c_int, [_vp, _c_int, _c_i64, _c_i64, _c_i64, _vp, _c_int, _c_i64, _c_i64,
                                ctypes.POINTER(_c_d), _c_int, _c_int, _vp, _vp, _vp, _vp, _c_sz,
                                _vp]),
}

SQ_GROUP_CALIBRATE, SQ_GROUP_FOLD, SQ_GROUP_FORWARD = 1, 2, 4


class SqLinearGroup(ctypes.Structure):
    """Mirror of the C struct sq_linear_group (include/sq.h), field for field."""
    _fields_ = [
        ("X", _vp), ("xt", _c_int), ("M", _c_i64), ("ldx", _c_i64),
        ("X_cal", _vp), ("M_cal", _c_i64), ("ld_cal", _c_i64),
        ("W", _vp), ("wt", _c_int), ("N", _c_i64), ("K", _c_i64), ("ldw", _c_i64),
        ("alpha", _c_d), ("mode", _c_int),
        ("act_max", _vp), ("s", _vp), ("Wq", _vp), ("w_scale", _vp), ("Xq", _vp), ("a_scale", _vp),
        ("A", _vp), ("B", _vp), ("r", _c_int), ("lora_scale", _c_f), ("T", _vp), ("ldt", _c_i64),
        ("workspace", _vp), ("workspace_bytes", _c_sz),
        ("Y", _vp), ("yt", _c_int), ("ldy", _c_i64),
        ("lora_parts", _c_int), ("lora_n_end", _c_i64 * SQ_MAX_LORA_PARTS),
        ("lora_r_end", _c_int * SQ_MAX_LORA_PARTS),
    ]


class SqGroupEvents(ctypes.Structure):
    """Mirror of the C struct sq_group_events (include/sq.h)."""
    _fields_ = [("begin", _vp), ("quant_begin", _vp), ("shrink_begin", _vp),
                ("gemm_begin", _vp), ("gemm_end", _vp)]


class LibraryNotBuilt(RuntimeError):
    pass


class SQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libsq.so (once). Raises LibraryNotBuilt if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(
                f"{LIB_PATH} is missing: build it with `python -m w8a8_smoothquant_int8_amd.build` "
                "(there is no non-HIP fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sq_status_string(int(status)).decode()


def _check(fn: str, st: int) -> None:
    if st != SQ_OK:
        raise SQError(fn, st)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}") from None


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0)


# ---------------------------------------------------------------------------
def sq_query_support(device: int = 0) -> bool:
    out = ctypes.c_int(0)
    _check("sq_query_support", lib().sq_query_support(int(device), ctypes.byref(out)))
    return bool(out.value)


def sq_calibrate_absmax(X: torch.Tensor, act_max: torch.Tensor, stream=None) -> None:
    M, K = X.shape
    _check("sq_calibrate_absmax", lib().sq_calibrate_absmax(
        _ptr(X), _dt(X), M, K, _ld(X), _ptr(act_max), _stream(stream)))


def sq_smooth_scale(act_max: torch.Tensor, W: torch.Tensor, alpha: float, s_out: torch.Tensor,
                    stream=None) -> None:
    N, K = W.shape
    _check("sq_smooth_scale", lib().sq_smooth_scale(
        _ptr(act_max), _ptr(W), _dt(W), N, K, _ld(W), float(alpha), _ptr(s_out), _stream(stream)))


def sq_fold_quant_weights(W: torch.Tensor, s: Optional[torch.Tensor], Wq: torch.Tensor,
                          w_scale: torch.Tensor, stream=None) -> None:
    N, K = W.shape
    _check("sq_fold_quant_weights", lib().sq_fold_quant_weights(
        _ptr(W), _dt(W), N, K, _ld(W), _ptr(s), _ptr(Wq), _ptr(w_scale), _stream(stream)))


def sq_smooth_fold(act_max: torch.Tensor, W: torch.Tensor, alpha: float, s_out: torch.Tensor,
                   Wq: torch.Tensor, w_scale: torch.Tensor, stream=None) -> None:
    N, K = W.shape
    _check("sq_smooth_fold", lib().sq_smooth_fold(
        _ptr(act_max), _ptr(W), _dt(W), N, K, _ld(W), float(alpha), _ptr(s_out), _ptr(Wq),
        _ptr(w_scale), _stream(stream)))


def sq_static_act_scale(act_max: torch.Tensor, s: Optional[torch.Tensor], a_scale: torch.Tensor,
                        stream=None) -> None:
    _check("sq_static_act_scale", lib().sq_static_act_scale(
        _ptr(act_max), _ptr(s), act_max.numel(), _ptr(a_scale), _stream(stream)))


def sq_quant_per_token(X: torch.Tensor, s: Optional[torch.Tensor], Xq: torch.Tensor,
                       a_scale: torch.Tensor, mode: str = "dynamic", stream=None) -> None:
    M, K = X.shape
    _check("sq_quant_per_token", lib().sq_quant_per_token(
        _ptr(X), _dt(X), M, K, _ld(X), _ptr(s), MODES[mode], _ptr(Xq), _ptr(a_scale),
        _stream(stream)))


def sq_quant_shrink(X: torch.Tensor, s: Optional[torch.Tensor], Xq: torch.Tensor,
                    a_scale: torch.Tensor, A: torch.Tensor, T: torch.Tensor, mode: str = "dynamic",
                    stream=None) -> None:
    """Per-token quant of X and T = bf16(X A^T) from one read of X (16-bit X, K <= 8192)."""
    M, K = X.shape
    _check("sq_quant_shrink", lib().sq_quant_shrink(
        _ptr(X), _dt(X), M, K, _ld(X), _ptr(s), MODES[mode], _ptr(Xq), _ptr(a_scale), _ptr(A),
        A.shape[0], _ptr(T), _ld(T), _stream(stream)))


SQ_NORM = {"rms": 0, "layer": 1}


def sq_fold_norm_weight(gamma: torch.Tensor, beta: Optional[torch.Tensor], s: Optional[torch.Tensor],
                        gamma_out: torch.Tensor, beta_out: Optional[torch.Tensor],
                        stream=None) -> None:
    """gamma_out = fp32(gamma / s), beta_out = fp32(beta / s); fp32 outputs."""
    _check("sq_fold_norm_weight", lib().sq_fold_norm_weight(
        _ptr(gamma), _ptr(beta), _dt(gamma), gamma.numel(), _ptr(s), _ptr(gamma_out),
        _ptr(beta_out), _stream(stream)))


def sq_norm_quant(H: torch.Tensor, kind: str, gamma: torch.Tensor, beta: Optional[torch.Tensor],
                  eps: float, Xq: torch.Tensor, a_scale: torch.Tensor, mode: str = "dynamic",
                  stats: Optional[torch.Tensor] = None, stream=None) -> None:
    """RMSNorm / LayerNorm of H with the folded fp32 weight (and bias), then INT8 codes."""
    M, K = H.shape
    _check("sq_norm_quant", lib().sq_norm_quant(
        _ptr(H), _dt(H), M, K, _ld(H), SQ_NORM[kind], _ptr(gamma), _ptr(beta), float(eps),
        MODES[mode], _ptr(Xq), _ptr(a_scale), _ptr(stats), _stream(stream)))


def sq_quant_static_clipped(X: torch.Tensor, s: Optional[torch.Tensor], a_scale: torch.Tensor,
                            Xq: torch.Tensor, clipped: torch.Tensor, stream=None) -> None:
    """Static per-tensor quant; adds the number of clamped codes to clipped
    (one int64 element on the device, which the caller zeroes)."""
    M, K = X.shape
    _check("sq_quant_static_clipped", lib().sq_quant_static_clipped(
        _ptr(X), _dt(X), M, K, _ld(X), _ptr(s), _ptr(a_scale), _ptr(Xq), _ptr(clipped),
        _stream(stream)))


def sq_w8a8_gemm(Xq: torch.Tensor, Wq: torch.Tensor, a_scale: torch.Tensor, w_scale: torch.Tensor,
                 Y: torch.Tensor, mode: str = "dynamic", stream=None) -> None:
    M, K = Xq.shape
    N = Wq.shape[0]
    _check("sq_w8a8_gemm", lib().sq_w8a8_gemm(
        _ptr(Xq), _ptr(Wq), _ptr(a_scale), MODES[mode], _ptr(w_scale), M, N, K, _ptr(Y), _dt(Y),
        _ld(Y), _stream(stream)))


def sq_w8a8_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().sq_w8a8_gemm_workspace_bytes(int(M), int(N), int(K)))


def sq_w8a8_gemm_ws(Xq: torch.Tensor, Wq: torch.Tensor, a_scale: torch.Tensor, w_scale: torch.Tensor,
                    Y: torch.Tensor, ws, mode: str = "dynamic", stream=None) -> None:
    """ws: a uint8 device tensor of sq_w8a8_gemm_workspace_bytes(M, N, K) bytes, or None when that is 0."""
    M, K = Xq.shape
    N = Wq.shape[0]
    _check("sq_w8a8_gemm_ws", lib().sq_w8a8_gemm_ws(
        _ptr(Xq), _ptr(Wq), _ptr(a_scale), MODES[mode], _ptr(w_scale), M, N, K, _ptr(Y), _dt(Y),
        _ld(Y), _ptr(ws) if ws is not None else None, ws.numel() if ws is not None else 0,
        _stream(stream)))


def sq_w8a8_gemm_i32(Xq: torch.Tensor, Wq: torch.Tensor, acc: torch.Tensor, stream=None) -> None:
    M, K = Xq.shape
    N = Wq.shape[0]
    _check("sq_w8a8_gemm_i32", lib().sq_w8a8_gemm_i32(
        _ptr(Xq), _ptr(Wq), M, N, K, _ptr(acc), _stream(stream)))


def sq_w8a8_gemm_lora(Xq: torch.Tensor, Wq: torch.Tensor, a_scale: torch.Tensor,
                      w_scale: torch.Tensor, T: torch.Tensor, B: torch.Tensor, Y: torch.Tensor,
                      scale: float = 1.0, mode: str = "dynamic", stream=None) -> None:
    """T: [M, r] bf16 (may be a column slice of a wider tensor); B: [N, r] bf16."""
    M, K = Xq.shape
    N = Wq.shape[0]
    r = B.shape[1]
    _check("sq_w8a8_gemm_lora", lib().sq_w8a8_gemm_lora(
        _ptr(Xq), _ptr(Wq), _ptr(a_scale), MODES[mode], _ptr(w_scale), M, N, K, _ptr(T), _ld(T),
        _ptr(B), r, float(scale), _ptr(Y), _dt(Y), _ld(Y), _stream(stream)))


def sq_lora_shrink(X: torch.Tensor, A: torch.Tensor, T: torch.Tensor, ws: torch.Tensor,
                   stream=None) -> None:
    """T[:, :r] = bf16(bf16(X) A^T) for A [r, K] bf16; T may be wider than r."""
    M, K = X.shape
    r = A.shape[0]
    _check("sq_lora_shrink", lib().sq_lora_shrink(
        _ptr(X), _dt(X), M, K, _ld(X), _ptr(A), r, _ptr(T), _ld(T), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def sq_lora_workspace_bytes(M: int, K: int, max_rank: int) -> int:
    return int(lib().sq_lora_workspace_bytes(int(M), int(K), int(max_rank)))


def sq_lora_apply(X: torch.Tensor, A: torch.Tensor, B: torch.Tensor, Y: torch.Tensor,
                  ws: torch.Tensor, scale: float = 1.0, stream=None) -> None:
    M, K = X.shape
    r = A.shape[0]
    N = Y.shape[1]
    _check("sq_lora_apply", lib().sq_lora_apply(
        _ptr(X), _dt(X), M, K, _ld(X), _ptr(A), _ptr(B), r, float(scale), _ptr(Y), _dt(Y), N,
        _ld(Y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def sq_lora_apply_segmented(X: torch.Tensor, seg_start: torch.Tensor, seg_adapter: torch.Tensor,
                            A_ptrs: torch.Tensor, B_ptrs: torch.Tensor, ranks: torch.Tensor,
                            max_rank: int, Y: torch.Tensor, ws: torch.Tensor, scale: float = 1.0,
                            stream=None) -> None:
    """seg_start/seg_adapter/ranks: int32 device tensors; A_ptrs/B_ptrs: int64 device tensors
    holding each adapter's data_ptr()."""
    M, K = X.shape
    N = Y.shape[1]
    _check("sq_lora_apply_segmented", lib().sq_lora_apply_segmented(
        _ptr(X), _dt(X), M, K, _ld(X), seg_adapter.numel(), _ptr(seg_start), _ptr(seg_adapter),
        ranks.numel(), _ptr(A_ptrs), _ptr(B_ptrs), _ptr(ranks), int(max_rank), float(scale),
        _ptr(Y), _dt(Y), N, _ld(Y), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def sq_lora_apply_segmented_noalloc(X: torch.Tensor, seg_start: torch.Tensor,
                                    seg_adapter: torch.Tensor, A_ptrs: torch.Tensor,
                                    B_ptrs: torch.Tensor, ranks: torch.Tensor, max_rank: int,
                                    Y: torch.Tensor, scale: float = 1.0, stream=None) -> None:
    """sq_lora_apply_segmented with the library's own scratch memory (no workspace)."""
    M, K = X.shape
    N = Y.shape[1]
    _check("sq_lora_apply_segmented_noalloc", lib().sq_lora_apply_segmented_noalloc(
        _ptr(X), _dt(X), M, K, _ld(X), seg_adapter.numel(), _ptr(seg_start), _ptr(seg_adapter),
        ranks.numel(), _ptr(A_ptrs), _ptr(B_ptrs), _ptr(ranks), int(max_rank), float(scale),
        _ptr(Y), _dt(Y), N, _ld(Y), _stream(stream)))


def pointer_table(tensors: Sequence[torch.Tensor], device) -> torch.Tensor:
    """Device int64 tensor of the tensors' data pointers (for the segmented call)."""
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=device)


def sq_linear_group_desc(X: torch.Tensor, X_cal: Optional[torch.Tensor], W: torch.Tensor,
                         alpha: float, mode: str, act_max: torch.Tensor, s: torch.Tensor,
                         Wq: torch.Tensor, w_scale: torch.Tensor, Xq: torch.Tensor,
                         a_scale: torch.Tensor, Y: torch.Tensor, A: Optional[torch.Tensor] = None,
                         B: Optional[torch.Tensor] = None, T: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None,
                         lora_scale: float = 1.0,
                         lora_parts: Optional[Sequence[Tuple[int, int]]] = None) -> SqLinearGroup:
    """Fill an sq_linear_group from tensors. The struct holds raw pointers:
    the tensors must stay alive (and in place) while it is used.
    lora_parts: [(n_end, r_end)] per projection of a block-diagonal B (the
    projection's last output column + 1 and last stacked rank + 1)."""
    M, K = X.shape
    N = W.shape[0]
    d = SqLinearGroup()
    d.X, d.xt, d.M, d.ldx = X.data_ptr(), _dt(X), M, _ld(X)
    if X_cal is not None:
        d.X_cal, d.M_cal, d.ld_cal = X_cal.data_ptr(), X_cal.shape[0], _ld(X_cal)
    d.W, d.wt, d.N, d.K, d.ldw = W.data_ptr(), _dt(W), N, K, _ld(W)
    d.alpha, d.mode = float(alpha), MODES[mode]
    d.act_max, d.s, d.Wq, d.w_scale = (act_max.data_ptr(), s.data_ptr(), Wq.data_ptr(),
                                       w_scale.data_ptr())
    d.Xq, d.a_scale = Xq.data_ptr(), a_scale.data_ptr()
    if workspace is not None:
        d.workspace, d.workspace_bytes = workspace.data_ptr(), workspace.numel()
    if A is not None:
        d.A, d.B, d.r, d.lora_scale = A.data_ptr(), B.data_ptr(), A.shape[0], float(lora_scale)
        d.T, d.ldt = T.data_ptr(), _ld(T)
        if lora_parts and len(lora_parts) > 1:
            if len(lora_parts) > SQ_MAX_LORA_PARTS:
                raise ValueError(f"at most {SQ_MAX_LORA_PARTS} LoRA parts")
            d.lora_parts = len(lora_parts)
            for i, (n_end, r_end) in enumerate(lora_parts):
                d.lora_n_end[i], d.lora_r_end[i] = int(n_end), int(r_end)
    d.Y, d.yt, d.ldy = Y.data_ptr(), _dt(Y), _ld(Y)
    return d


EVENT_FIELDS = ("begin", "quant_begin", "shrink_begin", "gemm_begin", "gemm_end")


def sq_group_events(**events) -> SqGroupEvents:
    """An sq_group_events from torch.cuda.Event objects (already created, e.g.
    recorded once) or raw hipEvent_t handles; missing or None entries are not
    recorded."""
    ev = SqGroupEvents()
    for k, e in events.items():
        if k not in EVENT_FIELDS:
            raise KeyError(k)
        if e is not None:
            setattr(ev, k, e.cuda_event if hasattr(e, "cuda_event") else int(e))
    return ev


def sq_linear_group_run(desc: SqLinearGroup, flags: int, stream=None,
                        events: Optional[SqGroupEvents] = None) -> None:
    """events: None or an SqGroupEvents (sq_group_events(...))."""
    _check("sq_linear_group_run", lib().sq_linear_group_run(
        ctypes.byref(desc), int(flags), _stream(stream),
        ctypes.byref(events) if events is not None else None))


def sq_alpha_sweep_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(lib().sq_alpha_sweep_workspace_bytes(M, N, K))


def sq_alpha_sweep(X: torch.Tensor, W: torch.Tensor, alphas, err: torch.Tensor, ws: torch.Tensor,
                   mode: str = "dynamic", rel: Optional[torch.Tensor] = None,
                   best: Optional[torch.Tensor] = None, stream=None) -> None:
    """err: [len(alphas), 2] float64 on the device, written with (sum of squared
    errors, sum of squared reference outputs) per alpha. rel: None or a
    [len(alphas)] float64 device tensor (err[:, 0] / err[:, 1]); best: None or
    a [1] int32 device tensor (index of the smallest rel, the first on ties)."""
    M, K = X.shape
    N = W.shape[0]
    a = (_c_d * len(alphas))(*[float(v) for v in alphas])
    _check("sq_alpha_sweep", lib().sq_alpha_sweep(
        _ptr(X), _dt(X), M, K, _ld(X), _ptr(W), _dt(W), N, _ld(W), a, len(alphas), MODES[mode],
        _ptr(err), _ptr(rel), _ptr(best), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))
