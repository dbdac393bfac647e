"""MI355X-native fused attention KL divergence (StreamKL) - Python binding.

A thin ctypes layer over ``libstreamkl.so`` (declared in ``include/streamkl.h``)
with the same entry-point names.  It only marshals arguments: torch tensors
provide device memory and the current HIP stream, every computation runs in
the library's HIP kernels.  There is no fallback: if the library is missing
or broken, ``load()`` and every entry point raise.

Tensors are [B, H, N, d] (any b/h/n strides with a contiguous d axis, so
[B, N, H, d] storage viewed as [B, H, N, d] works too); per-row vectors are
contiguous fp32 [B, H, N_Q].
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = [
    "load", "SklError", "skl_forward", "skl_forward_splitk", "skl_reduce",
    "skl_backward_student", "skl_backward_teacher", "skl_backward_joint", "skl_recommended_splits",
    "skl_backward_joint_workspace_size",
    "skl_forward_splitk_workspace_size", "skl_backward_workspace_size",
    "skl_version", "skl_set_kernel_events", "LIB_PATH",
    "skl_forward_splitk_noalloc", "skl_noalloc_scratch_bytes",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstreamkl.so")

SKL_BF16, SKL_F32 = 0, 1
SKL_BWD_SPLIT, SKL_BWD_FUSED_ATOMIC = 0, 1
_ALGOS = {"split": SKL_BWD_SPLIT, "fused_atomic": SKL_BWD_FUSED_ATOMIC}
_STATUS = {0: "SKL_OK", 1: "SKL_ERR_INVALID_ARGUMENT", 2: "SKL_ERR_UNSUPPORTED",
           3: "SKL_ERR_WORKSPACE_TOO_SMALL", 4: "SKL_ERR_HIP"}


class SklError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


class SklShape(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("NQ", ctypes.c_int64), ("NK", ctypes.c_int64),
        ("d1", ctypes.c_int32), ("d2", ctypes.c_int32), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("sq1", ctypes.c_int64 * 3), ("sk1", ctypes.c_int64 * 3),
        ("sq2", ctypes.c_int64 * 3), ("sk2", ctypes.c_int64 * 3),
    ]


_lib: Optional[ctypes.CDLL] = None

_P = ctypes.c_void_p
_F = ctypes.c_float
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SP = ctypes.POINTER(SklShape)

_SIGS = {
    "skl_forward": (_I, [_SP, _P, _P, _P, _P, _F, _F, _I, _P, _P, _P, _P]),
    "skl_forward_splitk_workspace_size": (_SZ, [_SP, _I]),
    "skl_forward_splitk": (_I, [_SP, _P, _P, _P, _P, _F, _F, _I, _I, _P, _SZ, _P]),
    "skl_reduce": (_I, [_SP, _I, _P, _SZ, _P, _P, _P, _P]),
    "skl_backward_workspace_size": (_SZ, [_SP, _I, _I]),
    "skl_backward_student": (_I, [_SP, _P, _P, _P, _P, _F, _F, _I, _P, _P, _P, _P, _P, _I, _P, _SZ, _P]),
    "skl_backward_teacher": (_I, [_SP, _P, _P, _P, _P, _F, _F, _I, _P, _P, _P, _P, _P, _P, _I, _P, _SZ, _P]),
    "skl_backward_joint_workspace_size": (_SZ, [_SP]),
    "skl_backward_joint": (_I, [_SP, _P, _P, _P, _P, _F, _F, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "skl_recommended_splits": (_I, [_SP, _I, _I]),
    "skl_noalloc_scratch_bytes": (_SZ, []),
    "skl_forward_splitk_noalloc": (_I, [_SP, _P, _P, _P, _P, _F, _F, _I, _I, _P, _P, _P, _P]),
    "skl_status_string": (ctypes.c_char_p, [_I]),
    "skl_last_error": (ctypes.c_char_p, []),
    "skl_version": (_I, []),
    "skl_set_kernel_events": (_I, [ctypes.POINTER(ctypes.c_void_p), _I]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libstreamkl.so (built by ``python -m attention_kl_divergence_skl_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libstreamkl.so not built: {path} is missing "
                           "(run python -m attention_kl_divergence_skl_amd.build)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        msg = load().skl_last_error().decode(errors="replace")
        raise SklError(status, msg)


def skl_version() -> int:
    return load().skl_version()


def skl_set_kernel_events(events=()) -> None:
    """Have the library record ``events`` (torch.cuda.Event objects, up to 4)
    around the main kernels of every following call on this thread: events[0]
    before the first main kernel, events[k] after the k-th.  An empty list
    switches it off.  Each event must already exist on the device (record it
    once first)."""
    handles = []
    for e in events:
        if not e.cuda_event:
            raise SklError(1, "event not created yet: record it once before passing it")
        handles.append(e.cuda_event)
    arr = (ctypes.c_void_p * max(1, len(handles)))(*handles)
    _check(load().skl_set_kernel_events(arr, len(handles)))


# ------------------------------------------------------------- marshalling ----

def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return SKL_BF16
    if t.dtype == torch.float32:
        return SKL_F32
    raise SklError(2, f"unsupported dtype {t.dtype}")


def _bhn_strides(t):
    if t.dim() != 4:
        raise SklError(1, f"expected a [B, H, N, d] tensor, got shape {tuple(t.shape)}")
    if t.shape[3] > 1 and t.stride(3) != 1:
        raise SklError(2, "the d axis must be contiguous")
    return (t.stride(0), t.stride(1), t.stride(2))


def make_shape(q1, k1, q2, k2) -> SklShape:
    """skl_shape of four [B, H, N, d] tensors (pure host arithmetic)."""
    B, H, NQ, d1 = q1.shape
    NK = k1.shape[2]
    d2 = q2.shape[3]
    if tuple(k1.shape) != (B, H, NK, d1) or tuple(q2.shape) != (B, H, NQ, d2) or tuple(k2.shape) != (B, H, NK, d2):
        raise SklError(1, f"inconsistent shapes q1{tuple(q1.shape)} k1{tuple(k1.shape)} "
                          f"q2{tuple(q2.shape)} k2{tuple(k2.shape)}")
    dt = _dtype_code(q1)
    for t in (k1, q2, k2):
        if _dtype_code(t) != dt:
            raise SklError(1, "q1, k1, q2, k2 must share one dtype")
    s = SklShape()
    s.B, s.H, s.NQ, s.NK, s.d1, s.d2, s.dtype, s.reserved = B, H, NQ, NK, d1, d2, dt, 0
    for name, t in (("sq1", q1), ("sk1", k1), ("sq2", q2), ("sk2", k2)):
        getattr(s, name)[:] = _bhn_strides(t)
    return s


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t) -> int:
    import torch

    return torch.cuda.current_stream(t.device).cuda_stream


def _check_device(*ts) -> None:
    dev = ts[0].device
    if dev.type != "cuda":
        raise SklError(1, "tensors must live on a GPU")
    for t in ts:
        if t is not None and t.device != dev:
            raise SklError(1, "all tensors must be on one device")


def _rowvec(t, B, H, NQ, name):
    import torch

    if t is None or t.dtype != torch.float32 or tuple(t.shape) != (B, H, NQ) or not t.is_contiguous():
        raise SklError(1, f"{name} must be a contiguous fp32 [B, H, N_Q] tensor")
    return t


def _scales(q1, q2, scale1, scale2):
    s1 = 1.0 / math.sqrt(q1.shape[3]) if scale1 is None else float(scale1)
    s2 = 1.0 / math.sqrt(q2.shape[3]) if scale2 is None else float(scale2)
    return s1, s2


# ------------------------------------------------------------ entry points ----

def skl_forward(q1, k1, q2, k2, scale1=None, scale2=None, causal: bool = False):
    """(kl, lse1, lse2), each fp32 [B, H, N_Q].  Scales default to 1/sqrt(d)."""
    import torch

    _check_device(q1, k1, q2, k2)
    s = make_shape(q1, k1, q2, k2)
    s1, s2 = _scales(q1, q2, scale1, scale2)
    out = [torch.empty((s.B, s.H, s.NQ), dtype=torch.float32, device=q1.device) for _ in range(3)]
    _check(load().skl_forward(ctypes.byref(s), _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), s1, s2, int(causal),
                              _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _stream(q1)))
    return tuple(out)


def skl_forward_splitk_workspace_size(q1, k1, q2, k2, num_splits: int) -> int:
    s = make_shape(q1, k1, q2, k2)
    return int(load().skl_forward_splitk_workspace_size(ctypes.byref(s), int(num_splits)))


def skl_forward_splitk(q1, k1, q2, k2, scale1=None, scale2=None, causal: bool = False,
                       num_splits: Optional[int] = None, ws=None):
    """Split-K partial statistics; returns (ws, num_splits) for skl_reduce."""
    import torch

    _check_device(q1, k1, q2, k2)
    s = make_shape(q1, k1, q2, k2)
    s1, s2 = _scales(q1, q2, scale1, scale2)
    if num_splits is None:
        num_splits = skl_recommended_splits(q1, k1, q2, k2, causal)
    need = int(load().skl_forward_splitk_workspace_size(ctypes.byref(s), int(num_splits)))
    if ws is None:
        ws = torch.empty(max(need, 4) // 4, dtype=torch.float32, device=q1.device)
    _check(load().skl_forward_splitk(ctypes.byref(s), _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), s1, s2,
                                     int(causal), int(num_splits), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(q1)))
    return ws, int(num_splits)


def skl_forward_splitk_noalloc(q1, k1, q2, k2, scale1=None, scale2=None, causal: bool = False,
                               num_splits: Optional[int] = None, out=None):
    """(kl, lse1, lse2) through split-K + reduce with the partials in the
    library's static scratch array (no workspace).  ``out`` may hold three
    preallocated contiguous fp32 [B, H, N_Q] tensors, so that the call itself
    allocates nothing."""
    import torch

    _check_device(q1, k1, q2, k2)
    s = make_shape(q1, k1, q2, k2)
    s1, s2 = _scales(q1, q2, scale1, scale2)
    if num_splits is None:
        num_splits = skl_recommended_splits(q1, k1, q2, k2, causal)
    if out is None:
        out = [torch.empty((s.B, s.H, s.NQ), dtype=torch.float32, device=q1.device) for _ in range(3)]
    for t, n in zip(out, ("kl", "lse1", "lse2")):
        _rowvec(t, s.B, s.H, s.NQ, n)
    _check(load().skl_forward_splitk_noalloc(ctypes.byref(s), _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), s1, s2,
                                             int(causal), int(num_splits), _ptr(out[0]), _ptr(out[1]),
                                             _ptr(out[2]), _stream(q1)))
    return tuple(out)


def skl_noalloc_scratch_bytes() -> int:
    return int(load().skl_noalloc_scratch_bytes())


def skl_reduce(ws, num_splits: int, B: int, H: int, NQ: int):
    """Merge split-K partials into (kl, lse1, lse2)."""
    import torch

    _check_device(ws)
    s = SklShape()
    s.B, s.H, s.NQ, s.NK, s.d1, s.d2, s.dtype, s.reserved = B, H, NQ, 0, 0, 0, SKL_F32, 0
    out = [torch.empty((B, H, NQ), dtype=torch.float32, device=ws.device) for _ in range(3)]
    _check(load().skl_reduce(ctypes.byref(s), int(num_splits), _ptr(ws), ws.numel() * ws.element_size(),
                             _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _stream(ws)))
    return tuple(out)


def _algo(algo) -> int:
    if isinstance(algo, str):
        if algo not in _ALGOS:
            raise SklError(1, f"unknown backward algorithm {algo!r} (split, fused_atomic)")
        return _ALGOS[algo]
    return int(algo)


def skl_backward_workspace_size(q1, k1, q2, k2, teacher: bool, algo="split") -> int:
    s = make_shape(q1, k1, q2, k2)
    return int(load().skl_backward_workspace_size(ctypes.byref(s), int(bool(teacher)), _algo(algo)))


def _disjoint_layout(strides, B, H, N, d) -> bool:
    """Host check of the library's rule for gradient layouts: taking the
    (b, h, n) axes of size > 1 in order of increasing stride, each stride must
    reach past the span of the axes inside it (the d axis spans d elements)."""
    span = d
    for size, st in sorted(zip((B, H, N), strides), key=lambda a: a[1]):
        if size <= 1:
            continue
        if st < span:
            return False
        span += st * (size - 1)
    return True


def _own_layout(t):
    """t itself if every element has its own address, else a contiguous copy
    (e.g. a K broadcast over heads with expand())."""
    B, H, N, d = t.shape
    return t if _disjoint_layout(_bhn_strides(t), B, H, N, d) else t.contiguous()


def _grad_like(t):
    import torch

    return torch.empty_strided(tuple(t.shape), t.stride(), dtype=t.dtype, device=t.device)


def _ws_for(s, teacher, algo, ws, device):
    import torch

    need = int(load().skl_backward_workspace_size(ctypes.byref(s), int(teacher), algo))
    if need and ws is None:
        ws = torch.empty(need // 4, dtype=torch.float32, device=device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    return ws, nbytes


def skl_backward_student(q1, k1, q2, k2, lse1, lse2, dkl, scale1=None, scale2=None,
                         causal: bool = False, algo="split", ws=None) -> Tuple:
    """(dq2, dk2) for 'optimise P2'; same dtype and strides as q2, k2."""
    _check_device(q1, k1, q2, k2, lse1, lse2, dkl)
    s = make_shape(q1, k1, q2, k2)
    s1, s2 = _scales(q1, q2, scale1, scale2)
    for t, n in ((lse1, "lse1"), (lse2, "lse2"), (dkl, "dkl")):
        _rowvec(t, s.B, s.H, s.NQ, n)
    a = _algo(algo)
    dq2, dk2 = _grad_like(q2), _grad_like(k2)
    ws, nbytes = _ws_for(s, 0, a, ws, q1.device)
    _check(load().skl_backward_student(ctypes.byref(s), _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), s1, s2,
                                       int(causal), _ptr(lse1), _ptr(lse2), _ptr(dkl), _ptr(dq2), _ptr(dk2),
                                       a, _ptr(ws), nbytes, _stream(q1)))
    return dq2, dk2


def skl_backward_teacher(q1, k1, q2, k2, lse1, lse2, kl, dkl, scale1=None, scale2=None,
                         causal: bool = False, algo="split", ws=None) -> Tuple:
    """(dq1, dk1) for 'optimise P1'; same dtype and strides as q1, k1."""
    _check_device(q1, k1, q2, k2, lse1, lse2, kl, dkl)
    s = make_shape(q1, k1, q2, k2)
    s1, s2 = _scales(q1, q2, scale1, scale2)
    for t, n in ((lse1, "lse1"), (lse2, "lse2"), (kl, "kl"), (dkl, "dkl")):
        _rowvec(t, s.B, s.H, s.NQ, n)
    a = _algo(algo)
    dq1, dk1 = _grad_like(q1), _grad_like(k1)
    ws, nbytes = _ws_for(s, 1, a, ws, q1.device)
    _check(load().skl_backward_teacher(ctypes.byref(s), _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), s1, s2,
                                       int(causal), _ptr(lse1), _ptr(lse2), _ptr(kl), _ptr(dkl), _ptr(dq1),
                                       _ptr(dk1), a, _ptr(ws), nbytes, _stream(q1)))
    return dq1, dk1


def skl_backward_joint_workspace_size(q1, k1, q2, k2) -> int:
    s = make_shape(q1, k1, q2, k2)
    return int(load().skl_backward_joint_workspace_size(ctypes.byref(s)))


def skl_backward_joint(q1, k1, q2, k2, lse1, lse2, kl, dkl, scale1=None, scale2=None,
                       causal: bool = False, ws=None) -> Tuple:
    """(dq1, dk1, dq2, dk2): both settings in one pass; dtype and strides of
    q1, k1, q2, k2."""
    import torch

    _check_device(q1, k1, q2, k2, lse1, lse2, kl, dkl)
    s = make_shape(q1, k1, q2, k2)
    s1, s2 = _scales(q1, q2, scale1, scale2)
    for t, n in ((lse1, "lse1"), (lse2, "lse2"), (kl, "kl"), (dkl, "dkl")):
        _rowvec(t, s.B, s.H, s.NQ, n)
    dq1, dk1, dq2, dk2 = _grad_like(q1), _grad_like(k1), _grad_like(q2), _grad_like(k2)
    need = int(load().skl_backward_joint_workspace_size(ctypes.byref(s)))
    if need and ws is None:
        ws = torch.empty(need // 4, dtype=torch.float32, device=q1.device)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().skl_backward_joint(ctypes.byref(s), _ptr(q1), _ptr(k1), _ptr(q2), _ptr(k2), s1, s2,
                                     int(causal), _ptr(lse1), _ptr(lse2), _ptr(kl), _ptr(dkl), _ptr(dq1),
                                     _ptr(dk1), _ptr(dq2), _ptr(dk2), _ptr(ws), nbytes, _stream(q1)))
    return dq1, dk1, dq2, dk2


def skl_recommended_splits(q1, k1, q2, k2, causal: bool = False, num_cus: Optional[int] = None) -> int:
    if num_cus is None:
        import torch

        num_cus = torch.cuda.get_device_properties(q1.device).multi_processor_count
    s = make_shape(q1, k1, q2, k2)
    return int(load().skl_recommended_splits(ctypes.byref(s), int(bool(causal)), int(num_cus)))


# ---------------------------------------------------------------------------
# Autograd wrapper: per-row KL(P1 || P2) as a differentiable torch op.  P1
# does not depend on (Q2, K2) and P2 does not depend on (Q1, K1), so the
# student call ("optimise P2") gives exactly dKL/d(Q2, K2) and the teacher
# call ("optimise P1") exactly dKL/d(Q1, K1); backward launches only the
# settings whose inputs require a gradient (a frozen teacher costs one).  When
# both do, the default ("auto") makes one joint call, which computes both
# settings from one recompute and measures faster on MI355X than the two split
# calls; algo="split" forces the two split calls.
# ---------------------------------------------------------------------------

def _autograd_function():
    import torch

    class AttentionKL(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q1, k1, q2, k2, scale1, scale2, causal, algo):
            kl, lse1, lse2 = skl_forward(q1, k1, q2, k2, scale1, scale2, causal)
            ctx.save_for_backward(q1, k1, q2, k2, kl, lse1, lse2)
            ctx.args = (scale1, scale2, causal, algo)
            ctx.mark_non_differentiable(lse1, lse2)
            return kl, lse1, lse2

        @staticmethod
        def backward(ctx, g, _g_lse1, _g_lse2):
            q1, k1, q2, k2, kl, lse1, lse2 = ctx.saved_tensors
            scale1, scale2, causal, algo = ctx.args
            g = g.float().contiguous()
            # Gradients take their input's strides; an input that repeats
            # elements (broadcast over heads or batches) is copied first, and
            # autograd sums the copy's gradient back over the broadcast axes.
            q1, k1, q2, k2 = (_own_layout(x) for x in (q1, k1, q2, k2))
            dq1 = dk1 = dq2 = dk2 = None
            need_s = ctx.needs_input_grad[2] or ctx.needs_input_grad[3]
            need_t = ctx.needs_input_grad[0] or ctx.needs_input_grad[1]
            if algo in ("joint", "auto"):
                if need_s and need_t:
                    dq1, dk1, dq2, dk2 = skl_backward_joint(q1, k1, q2, k2, lse1, lse2, kl, g, scale1, scale2,
                                                            causal)
                    return dq1, dk1, dq2, dk2, None, None, None, None
                algo = "split"
            if need_s:
                dq2, dk2 = skl_backward_student(q1, k1, q2, k2, lse1, lse2, g, scale1, scale2, causal, algo=algo)
            if need_t:
                dq1, dk1 = skl_backward_teacher(q1, k1, q2, k2, lse1, lse2, kl, g, scale1, scale2, causal,
                                                algo=algo)
            return dq1, dk1, dq2, dk2, None, None, None, None

    return AttentionKL


_ATTENTION_KL = None


def attention_kl(q1, k1, q2, k2, scale1=None, scale2=None, causal: bool = False, algo="auto"):
    """Differentiable per-row KL(P1 || P2), P_k = softmax(scale_k Q_k K_k^T).

    Returns (kl, lse1, lse2); kl [B, H, N_Q] fp32 carries gradients to every
    input that requires one (the LSEs are auxiliary and not differentiable).
    Scales default to 1/sqrt(d_k).  algo: "auto" (default: the joint kernels
    when both settings need gradients -- one recompute for both, the measured
    fastest -- else the split kernels), "split", "fused_atomic", or "joint"
    (the same as "auto")."""
    if algo not in ("auto", "split", "fused_atomic", "joint"):
        raise SklError(1, f"unknown backward algorithm {algo!r} (auto, split, fused_atomic, joint)")
    global _ATTENTION_KL
    if _ATTENTION_KL is None:
        _ATTENTION_KL = _autograd_function()
    s1, s2 = _scales(q1, q2, scale1, scale2)
    return _ATTENTION_KL.apply(q1, k1, q2, k2, s1, s2, bool(causal), algo)


__all__ += ["attention_kl"]
