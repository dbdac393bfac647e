"""C-ABI checks that need no GPU: the built library loads, exports every
function include/streamkl.h declares, and rejects bad arguments on the host
(before anything is enqueued) with the documented status codes."""
import ctypes
import os
import re

import pytest

import attention_kl_divergence_skl_amd as skl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "streamkl.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(skl_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(skl.LIB_PATH):
        pytest.fail("libstreamkl.so is not built (python -m attention_kl_divergence_skl_amd.build)")
    return skl.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("skl_forward", "skl_forward_splitk", "skl_reduce", "skl_backward_student",
              "skl_backward_teacher", "skl_forward_splitk_workspace_size", "skl_backward_workspace_size"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_shape_struct_matches_header_layout():
    # int64 x4, int32 x4, then four int64[3] stride triples.
    assert ctypes.sizeof(skl.SklShape) == 4 * 8 + 4 * 4 + 12 * 8
    assert skl.SklShape.sq1.offset == 48


def _shape(B=1, H=2, NQ=256, NK=256, d1=128, d2=128, dtype=0):
    s = skl.SklShape()
    s.B, s.H, s.NQ, s.NK, s.d1, s.d2, s.dtype, s.reserved = B, H, NQ, NK, d1, d2, dtype, 0
    for name, (n, d) in (("sq1", (NQ, d1)), ("sk1", (NK, d1)), ("sq2", (NQ, d2)), ("sk2", (NK, d2))):
        getattr(s, name)[:] = (H * n * d, n * d, d)
    return s


# Fake, never-dereferenced device addresses: validation fails before any use.
A = 0x10000
P = [A, A + 0x1000, A + 0x2000, A + 0x3000]


def _fwd(lib, s, scale1=0.1, scale2=0.1, causal=0, ptrs=None, outs=(A + 0x4000, A + 0x5000, A + 0x6000)):
    p = P if ptrs is None else ptrs
    return lib.skl_forward(ctypes.byref(s), *p, scale1, scale2, causal, *outs, None)


@pytest.mark.parametrize("mut,expect", [
    (lambda s: setattr(s, "d1", 96), UNSUPPORTED),
    (lambda s: setattr(s, "d2", 256), UNSUPPORTED),
    (lambda s: setattr(s, "dtype", 7), UNSUPPORTED),
    (lambda s: setattr(s, "B", -1), INVALID),
    (lambda s: setattr(s, "reserved", 1), INVALID),
    (lambda s: s.sq1.__setitem__(2, 100), UNSUPPORTED),   # n stride not a multiple of 8 bf16 elements
    (lambda s: s.sk2.__setitem__(0, -8), INVALID),
    (lambda s: s.sq2.__setitem__(2, 1 << 24), UNSUPPORTED),   # 64 rows of this stride overflow 32-bit offsets
    (lambda s: setattr(s, "NK", 1 << 30), UNSUPPORTED),       # row indices are 32-bit in the kernels
    (lambda s: setattr(s, "NQ", 1 << 30), UNSUPPORTED),
])
def test_forward_rejects_bad_shapes(lib, mut, expect):
    s = _shape()
    mut(s)
    assert _fwd(lib, s) == expect
    assert lib.skl_last_error().decode()


def test_forward_rejects_bad_scalars_and_pointers(lib):
    s = _shape()
    assert _fwd(lib, s, scale1=0.0) == INVALID
    assert _fwd(lib, s, scale2=float("nan")) == INVALID
    assert _fwd(lib, s, scale1=-1.0) == INVALID
    assert _fwd(lib, s, ptrs=[A, None, A, A]) == INVALID
    assert _fwd(lib, s, ptrs=[A + 2, A, A, A]) == UNSUPPORTED   # misaligned q1
    assert _fwd(lib, s, outs=(None, A, A)) == INVALID
    c = _shape(NQ=300, NK=200)
    assert _fwd(lib, c, causal=1) == INVALID                      # causal with N_Q > N_K
    z = _shape(NQ=4, NK=0)
    assert _fwd(lib, z) == INVALID                                 # empty softmax


def test_empty_problems_enqueue_nothing(lib):
    for s in (_shape(B=0), _shape(H=0), _shape(NQ=0, NK=0), _shape(NQ=0)):
        assert _fwd(lib, s, ptrs=[None] * 4, outs=(None, None, None)) == OK


def test_workspace_sizes(lib):
    s = _shape(B=2, H=3, NQ=100, NK=50, d1=128, d2=64)
    assert lib.skl_forward_splitk_workspace_size(ctypes.byref(s), 4) == 5 * 2 * 3 * 4 * 100 * 4
    assert lib.skl_backward_workspace_size(ctypes.byref(s), 0, 1) == 2 * 3 * 100 * 64 * 4
    assert lib.skl_backward_workspace_size(ctypes.byref(s), 1, 1) == 2 * 3 * 100 * 128 * 4
    assert lib.skl_backward_workspace_size(ctypes.byref(s), 0, 0) == 0   # split: no workspace
    assert lib.skl_forward_splitk_workspace_size(ctypes.byref(s), 0) == 0


def test_split_and_backward_validation(lib):
    s = _shape()
    need = lib.skl_forward_splitk_workspace_size(ctypes.byref(s), 2)
    st = lib.skl_forward_splitk(ctypes.byref(s), *P, 0.1, 0.1, 0, 2, A, need - 4, None)
    assert st == WS_SMALL
    st = lib.skl_forward_splitk(ctypes.byref(s), *P, 0.1, 0.1, 0, 0, A, need, None)
    assert st == INVALID
    st = lib.skl_reduce(ctypes.byref(s), 2, A, need - 1, A, A, A, None)
    assert st == WS_SMALL
    wsb = lib.skl_backward_workspace_size(ctypes.byref(s), 0, 1)
    st = lib.skl_backward_student(ctypes.byref(s), *P, 0.1, 0.1, 0, A, A, A, A, A, 1, A, wsb - 16, None)
    assert st == WS_SMALL
    st = lib.skl_backward_teacher(ctypes.byref(s), *P, 0.1, 0.1, 0, A, A, None, A, A, A, 0, None, 0, None)
    assert st == INVALID   # kl is required by the teacher setting
    st = lib.skl_backward_student(ctypes.byref(s), *P, 0.1, 0.1, 0, A, A, A, A + 8, A, 0, None, 0, None)
    assert st == UNSUPPORTED   # misaligned dq2
    st = lib.skl_backward_student(ctypes.byref(s), *P, 0.1, 0.1, 0, A, A, A, A, A, 7, None, 0, None)
    assert st == INVALID   # unknown algorithm
    st = lib.skl_backward_student(ctypes.byref(s), *P, 0.1, 0.1, 0, A, A, A, A, A, 1, None, wsb, None)
    assert st == INVALID   # the fused algorithm needs its workspace


def test_kernel_event_hook_validation(lib):
    arr = (ctypes.c_void_p * 5)()
    assert lib.skl_set_kernel_events(arr, 5) == INVALID
    assert lib.skl_set_kernel_events(None, 2) == INVALID
    assert lib.skl_set_kernel_events(None, 0) == OK


def test_status_strings_and_version(lib):
    assert lib.skl_status_string(0) == b"SKL_OK"
    assert lib.skl_status_string(3) == b"SKL_ERR_WORKSPACE_TOO_SMALL"
    assert lib.skl_version() >= 100


def test_recommended_splits(lib):
    big = _shape(B=1, H=32, NQ=65536, NK=65536)
    assert lib.skl_recommended_splits(ctypes.byref(big), 1, 256) == 1
    small = _shape(B=1, H=1, NQ=256, NK=16384)
    k = lib.skl_recommended_splits(ctypes.byref(small), 0, 256)
    assert 2 <= k <= 64
    tiny = _shape(B=1, H=1, NQ=128, NK=128)
    assert lib.skl_recommended_splits(ctypes.byref(tiny), 0, 256) == 1


def test_joint_backward_validation(lib):
    s = _shape()
    st = lib.skl_backward_joint(ctypes.byref(s), *P, 0.1, 0.1, 0, A, A, None, A, A, A, A, A, None, 0, None)
    assert st == INVALID   # kl is required
    st = lib.skl_backward_joint(ctypes.byref(s), *P, 0.1, 0.1, 0, A, A, A, A, A, A, None, A, None, 0, None)
    assert st == INVALID   # every gradient output is required
    st = lib.skl_backward_joint(ctypes.byref(s), *P, 0.1, 0.1, 2, A, A, A, A, A, A, A + 4, A, None, 0, None)
    assert st in (INVALID, UNSUPPORTED)


def _student(lib, s, algo=0):
    return lib.skl_backward_student(ctypes.byref(s), *P, 0.1, 0.1, 0, A, A, A, A, A, algo, None, 0, None)


def _teacher(lib, s, algo=0):
    return lib.skl_backward_teacher(ctypes.byref(s), *P, 0.1, 0.1, 0, A, A, A, A, A, A, algo, None, 0, None)


def _joint(lib, s):
    return lib.skl_backward_joint(ctypes.byref(s), *P, 0.1, 0.1, 0, A, A, A, A, A, A, A, A, None, 0, None)


@pytest.mark.parametrize("tensor,axis,value", [
    ("sk2", 1, 0),          # K2 broadcast over heads (expand)
    ("sq2", 0, 0),          # Q2 broadcast over the batch (B = 2 below)
    ("sk2", 2, 64),         # rows overlap (stride below the head dim 128)
    ("sq2", 1, 256 * 64),   # heads interleaved into each other's rows
])
def test_backward_rejects_gradient_layouts_that_repeat_elements(lib, tensor, axis, value):
    s = _shape(B=2)
    getattr(s, tensor)[axis] = value
    assert _student(lib, s) == UNSUPPORTED
    assert "stride" in lib.skl_last_error().decode()
    assert _joint(lib, s) == UNSUPPORTED


def test_backward_accepts_bnhd_and_size_one_axes(lib):
    from attention_kl_divergence_skl_amd import _disjoint_layout
    # [B, N, H, d] storage viewed as [B, H, N, d].
    assert _disjoint_layout((256 * 4 * 128, 128, 4 * 128), 2, 4, 256, 128)
    # A size-1 axis may have any stride, 0 included.
    assert _disjoint_layout((0, 256 * 128, 128), 1, 3, 256, 128)
    assert not _disjoint_layout((256 * 128, 0, 128), 1, 3, 256, 128)
    assert not _disjoint_layout((256 * 128, 256 * 128, 64), 1, 1, 256, 128)


def test_dispatch_size_limit(lib):
    # 2^20 heads x 16 query tiles = 2^24 workgroups > (2^32 - 1) / 256.
    big = _shape(B=1, H=1 << 20, NQ=2048, NK=2048)
    assert _fwd(lib, big) == UNSUPPORTED
    assert "dispatch limit" in lib.skl_last_error().decode()
    assert _student(lib, big) == UNSUPPORTED
    assert _teacher(lib, big, algo=1) == UNSUPPORTED
    assert _joint(lib, big) == UNSUPPORTED
    # Split-K: 2^16 heads x 1 query tile x 256 splits.
    sk = _shape(B=1, H=1 << 16, NQ=128, NK=65536)
    need = lib.skl_forward_splitk_workspace_size(ctypes.byref(sk), 256)
    st = lib.skl_forward_splitk(ctypes.byref(sk), *P, 0.1, 0.1, 0, 256, A, need, None)
    assert st == UNSUPPORTED
    assert "dispatch limit" in lib.skl_last_error().decode()


def test_noalloc_rejects_partials_beyond_the_static_array(lib):
    assert lib.skl_noalloc_scratch_bytes() == 32 << 20
    s = _shape(B=1, H=64, NQ=4096, NK=8192)   # 20 * 64 * 4096 * 8 bytes = 40 MiB of partials
    st = lib.skl_forward_splitk_noalloc(ctypes.byref(s), *P, 0.1, 0.1, 1, 8, A, A, A, None)
    assert st == UNSUPPORTED
    assert "static scratch" in lib.skl_last_error().decode()
