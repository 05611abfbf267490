"""Host-side tests of the C ABI (no GPU needed).

Loads libstreamkl.so, checks that it exports every function include/streamkl.h
declares, and drives the validation paths: each call below carries an
argument error that the library must reject on the host, before any HIP call
or launch.  No call here reaches a kernel.
"""
import ctypes
import os
import re

import pytest

from attention_kl_divergence_online_amd import _lib
from attention_kl_divergence_online_amd._lib import Problem

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "streamkl.h")
CSRC = os.path.join(ROOT, "attention_kl_divergence_online_amd", "csrc")

# Fake, 16-byte aligned device addresses: never dereferenced, because every
# call that uses them fails validation on another argument first.
A = 0x10000
MIS = 0x10008  # misaligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from attention_kl_divergence_online_amd import build
        build.build()
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(streamkl_\w+)\s*\(", text)


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert names, "header parse found no functions"
    assert tuple(names) == _lib.EXPORTS
    for n in names:
        assert hasattr(L, n), n


def test_library_allocates_no_device_memory():
    # The library owns no device buffers: callers pass every buffer in.
    for f in os.listdir(CSRC):
        src = open(os.path.join(CSRC, f)).read()
        assert not re.search(r"\bhip(Malloc|Free|MallocAsync|HostMalloc)\w*\s*\(", src), f


def test_status_strings(L):
    assert _lib.status_string(0) == "ok"
    for s in range(1, 7):
        assert _lib.status_string(s) not in ("ok", "unknown status")
    assert _lib.status_string(99) == "unknown status"
    assert L.streamkl_version() >= 100


def P(**kw):
    base = dict(B=1, H=2, NQ=8, NK=8, D=64, scale=0.125, causal=0, dtype=_lib.STREAMKL_BF16)
    base.update(kw)
    return Problem(**base)


def fwd(L, p, q1=A, k1=A, q2=A, k2=A, kl=A, l1=A, l2=A):
    return L.streamkl_fwd(ctypes.byref(p) if p is not None else None, q1, k1, q2, k2, kl, l1, l2, None)


def test_forward_validation(L):
    assert L.streamkl_fwd(None, A, A, A, A, A, A, A, None) == _lib.STREAMKL_ERR_NULL
    assert fwd(L, P(dtype=7)) == _lib.STREAMKL_ERR_DTYPE
    assert fwd(L, P(D=96)) == _lib.STREAMKL_ERR_SHAPE
    assert fwd(L, P(NQ=-1)) == _lib.STREAMKL_ERR_SHAPE
    assert fwd(L, P(NK=0)) == _lib.STREAMKL_ERR_SHAPE
    assert fwd(L, P(causal=1, NQ=9, NK=8)) == _lib.STREAMKL_ERR_SHAPE
    assert fwd(L, P(NK=1 << 25, D=64)) == _lib.STREAMKL_ERR_SHAPE  # per-head tensor >= 2^31
    assert fwd(L, P(scale=float("nan"))) == _lib.STREAMKL_ERR_SHAPE
    assert fwd(L, P(), q1=None) == _lib.STREAMKL_ERR_NULL
    assert fwd(L, P(), k2=None) == _lib.STREAMKL_ERR_NULL
    assert fwd(L, P(), kl=None) == _lib.STREAMKL_ERR_NULL
    assert fwd(L, P(), q2=MIS) == _lib.STREAMKL_ERR_ALIGN
    assert fwd(L, P(), l2=MIS) == _lib.STREAMKL_ERR_ALIGN


def test_fp8_dtype_is_accepted(L):
    # fp8 e4m3 inputs pass every entry point's checks (the calls then stop at
    # the first null pointer, before any launch), and the workspace queries
    # size them like bf16 problems without the bf16 chunk maxima.
    f8 = _lib.STREAMKL_FP8_E4M3
    assert fwd(L, P(dtype=f8), q1=None) == _lib.STREAMKL_ERR_NULL
    assert fwd(L, P(dtype=f8, D=128), q2=MIS) == _lib.STREAMKL_ERR_ALIGN
    assert fwd(L, P(dtype=f8, B=0), q1=None, kl=None) == _lib.STREAMKL_OK
    p = P(dtype=f8)
    assert L.streamkl_fwd_splitk_workspace_size(ctypes.byref(p), 1) > 0
    ws8 = L.streamkl_bwd_workspace_size(ctypes.byref(p))
    assert 0 < ws8 < L.streamkl_bwd_workspace_size(ctypes.byref(P()))
    assert L.streamkl_bwd_workspace_size_min(ctypes.byref(p)) == ws8
    assert L.streamkl_bwd(ctypes.byref(p), None, A, A, A, A, A, A, A, A, A, A, A, A, 1 << 20,
                          None) == _lib.STREAMKL_ERR_NULL
    assert L.streamkl_bwd_prepare(ctypes.byref(p), A, A, A, A, None, A, 1 << 20, None) == _lib.STREAMKL_ERR_NULL
    for name in ("streamkl_bwd_dk", "streamkl_bwd_dq"):
        fn = getattr(L, name)
        assert fn(ctypes.byref(p), A, A, A, A, None, A, A, A, A, A, A, 1 << 20, None) == _lib.STREAMKL_ERR_NULL, name


def test_grid_limit_is_rejected_on_the_host(L):
    # 2^30 heads of 1024 queries: every size is legal on its own, but the forward
    # grid (4 query tiles x 512 threads per head) passes 2^32 work-items.
    big = P(B=1 << 20, H=1 << 10, NQ=1024, NK=1024)
    assert fwd(L, big) == _lib.STREAMKL_ERR_SHAPE
    assert L.streamkl_bwd_workspace_size(ctypes.byref(big)) == 0
    # Split-K multiplies the forward grid by the split count.
    p = P(B=1, H=1 << 14, NQ=1024, NK=1 << 20)
    assert L.streamkl_fwd_splitk_workspace_size(ctypes.byref(p), 1) > 0
    assert L.streamkl_fwd_splitk_workspace_size(ctypes.byref(p), 1 << 14) == 0
    assert L.streamkl_fwd_splitk(ctypes.byref(p), A, A, A, A, A, A, A, 1 << 14, A, 1 << 40,
                                 None) == _lib.STREAMKL_ERR_SHAPE


def test_fp8_grid_counts_its_twelve_wave_tiles(L):
    # fp8's main forward shape runs 768 work-items per 384-query tile, more per
    # query than bf16's 512 per 256: 2 * 10^6 heads of 1024 queries fit the
    # 2^32 work-item limit in bf16 (4.10e9) but not in fp8 (4.61e9).
    p = P(B=2000, H=1000, NQ=1024, NK=1024, D=128)
    assert fwd(L, p, q1=None) == _lib.STREAMKL_ERR_NULL  # passes the host checks
    assert fwd(L, P(B=2000, H=1000, NQ=1024, NK=1024, D=128, dtype=_lib.STREAMKL_FP8_E4M3)) == \
        _lib.STREAMKL_ERR_SHAPE


def test_empty_problems_are_no_ops(L):
    # Nothing to compute: success without touching any pointer.
    assert fwd(L, P(B=0), q1=None, kl=None) == _lib.STREAMKL_OK
    assert fwd(L, P(NQ=0), q1=None, kl=None) == _lib.STREAMKL_OK
    assert fwd(L, P(H=0, NK=0), q1=None) == _lib.STREAMKL_OK


def test_splitk_validation(L):
    p = P(NK=200)  # 4 key tiles of 64
    assert L.streamkl_fwd_splitk_workspace_size(ctypes.byref(p), 4) == 5 * 4 * 2 * 8 * 4
    assert L.streamkl_fwd_splitk_workspace_size(ctypes.byref(p), 5) == 0
    assert L.streamkl_fwd_splitk_workspace_size(ctypes.byref(p), 0) == 0
    args = (A, A, A, A, A, A, A)
    assert L.streamkl_fwd_splitk(ctypes.byref(p), *args, 0, A, 1 << 20, None) == _lib.STREAMKL_ERR_SHAPE
    assert L.streamkl_fwd_splitk(ctypes.byref(p), *args, 5, A, 1 << 20, None) == _lib.STREAMKL_ERR_SHAPE
    assert L.streamkl_fwd_splitk(ctypes.byref(p), *args, 3, None, 0, None) == _lib.STREAMKL_ERR_WORKSPACE
    assert L.streamkl_fwd_splitk(ctypes.byref(p), *args, 3, A, 10, None) == _lib.STREAMKL_ERR_WORKSPACE
    assert L.streamkl_fwd_splitk(ctypes.byref(p), *args, 3, MIS, 1 << 20, None) == _lib.STREAMKL_ERR_ALIGN
    assert L.streamkl_fwd_splitk(ctypes.byref(p), None, A, A, A, A, A, A, 3, A, 1 << 20,
                                 None) == _lib.STREAMKL_ERR_NULL


def test_noalloc_splitk_validation(L):
    # Host-side rejections of the allocation-free split-K forward, before any
    # HIP call: the argument errors of streamkl_fwd_splitk, and a problem whose
    # partial states would not fit the library's scratch array.
    p = P(NK=200)
    args = (A, A, A, A, A, A, A)
    assert L.streamkl_fwd_splitk_noalloc(ctypes.byref(p), *args, 0, None) == _lib.STREAMKL_ERR_SHAPE
    assert L.streamkl_fwd_splitk_noalloc(ctypes.byref(p), *args, 5, None) == _lib.STREAMKL_ERR_SHAPE
    assert L.streamkl_fwd_splitk_noalloc(ctypes.byref(p), None, A, A, A, A, A, A, 3,
                                         None) == _lib.STREAMKL_ERR_NULL
    assert L.streamkl_fwd_splitk_noalloc(ctypes.byref(p), A, A, A, A, MIS, A, A, 3,
                                         None) == _lib.STREAMKL_ERR_ALIGN
    big = P(B=1, H=32, NQ=1024, NK=8192)  # 128 splits: 5 * 128 * 32 * 1024 * 4 B = 80 MiB
    need = L.streamkl_fwd_splitk_workspace_size(ctypes.byref(big), 128)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert L.streamkl_fwd_splitk_noalloc(ctypes.byref(big), *args, 128, None) == _lib.STREAMKL_ERR_WORKSPACE
    fits = L.streamkl_fwd_splitk_workspace_size(ctypes.byref(big), 64)
    assert 0 < fits <= _lib.NOALLOC_SCRATCH_BYTES
    assert L.streamkl_fwd_splitk_noalloc(ctypes.byref(P(H=0)), *args, 1, None) == _lib.STREAMKL_OK


def test_noalloc_scratch_is_a_file_scope_device_array():
    # The scratch is one static device array in the split-K source, reached in
    # host code only through the address hipGetSymbolAddress returns.
    src = open(os.path.join(CSRC, "fwd.hip")).read()
    assert re.search(r"static __device__ __align__\(256\) float scratch\[", src)
    assert "hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch))" in src
    code = re.sub(r"//[^\n]*", "", src)
    uses = re.findall(r"\bscratch\b", code)
    assert len(uses) == 2, "scratch is named only where declared and in the address lookup"


def bwd(L, p, dq1=A, dk1=A, dq2=A, dk2=A, ws=A, wsb=1 << 20, g=A, kl=A):
    return L.streamkl_bwd(ctypes.byref(p), A, A, A, A, kl, A, A, g, dq1, dk1, dq2, dk2, ws, wsb, None)


def dq_splits(B, H, NQ, NK):
    # The header's rule: fewer than 256 query tiles of 128 rows in all split the
    # keys into S chunks of whole 64-key tiles.
    tiles = B * H * ((NQ + 127) // 128)
    ktiles = (NK + 63) // 64
    if NQ == 0 or NK == 0 or tiles >= 256:
        return 1
    sp = min((256 + tiles - 1) // tiles, 64, ktiles)
    if sp <= 1:
        return 1
    per = (ktiles + sp - 1) // sp
    return (ktiles + per - 1) // per


def bwd_workspace(B, H, NQ, NK, D, split=True, bf16=True):
    # sigma of every head and the four operand scales of every head (256-byte
    # slots), for bf16 inputs the chunk maxima (16 per head and tensor), then,
    # with `split`, the split query pass's partial dQ1, dQ2 (fp32).
    up = lambda n, a: (n + a - 1) // a * a
    bh = B * H
    S = dq_splits(B, H, NQ, NK) if bf16 else 1
    dqp = S * 2 * bh * NQ * D * 4 if (split and S > 1) else 0
    part = up(bh * 4 * 16 * 4, 256) if bf16 else 0
    return up(max(16, 4 * bh), 256) + up(max(16, 16 * bh), 256) + part + up(dqp, 256)


def fused_workspace(B, H, NQ, NK, D):
    # The fused pass (bf16, at most 128 queries): C key chunks of whole 32-key
    # blocks aiming at 2048 workgroups (512 above 32 queries), a dQ partial
    # per chunk when there are several.
    up = lambda n, a: (n + a - 1) // a * a
    units, blocks = B * H, (NK + 31) // 32
    target = 2048 if NQ <= 32 else 512
    sp = max(1, min((target + units - 1) // units, 64, blocks))
    per = (blocks + sp - 1) // sp
    C = (blocks + per - 1) // per
    part = C * 2 * units * NQ * D * 4 if C > 1 else 0
    return up(max(part, 16), 256)


def test_backward_validation(L):
    p = P()
    f32 = _lib.STREAMKL_FP32
    assert L.streamkl_bwd_workspace_size(ctypes.byref(P(dtype=f32))) == 512
    assert L.streamkl_bwd_workspace_size(ctypes.byref(P(B=3, H=7, dtype=f32))) == 768
    assert L.streamkl_bwd_workspace_size(ctypes.byref(p)) == bwd_workspace(1, 2, 8, 8, 64)
    # At most 128 queries: the larger of the split passes' and the fused pass's needs.
    assert L.streamkl_bwd_workspace_size(ctypes.byref(P(B=3, H=7, NQ=65, NK=200, D=128))) == \
        max(bwd_workspace(3, 7, 65, 200, 128), fused_workspace(3, 7, 65, 200, 128)) == fused_workspace(3, 7, 65, 200, 128)
    assert L.streamkl_bwd_workspace_size(ctypes.byref(P(B=3, H=7, NQ=129, NK=200, D=128))) == \
        bwd_workspace(3, 7, 129, 200, 128)
    assert L.streamkl_bwd_workspace_size(ctypes.byref(P(D=32))) == 0
    # Minimum: everything but the split query pass's partials (that pass then runs unsplit).
    assert L.streamkl_bwd_workspace_size_min(ctypes.byref(P(B=3, H=7, NQ=65, NK=200, D=128))) == \
        bwd_workspace(3, 7, 65, 200, 128, split=False)
    assert bwd_workspace(3, 7, 65, 200, 128, split=False) < bwd_workspace(3, 7, 65, 200, 128)
    assert L.streamkl_bwd_workspace_size_min(ctypes.byref(P(B=3, H=7, dtype=f32))) == 768
    # O(B * H) at the 64K causal workload: 32 heads, no split, a few KiB.
    big = P(B=1, H=32, NQ=65536, NK=65536, D=128, causal=1)
    assert L.streamkl_bwd_workspace_size(ctypes.byref(big)) == bwd_workspace(1, 32, 65536, 65536, 128) <= 16384
    # Below the minimum the combined call refuses; between minimum and full it accepts (not run here).
    pm = P(B=4, H=8)
    mn = L.streamkl_bwd_workspace_size_min(ctypes.byref(pm))
    assert bwd(L, pm, wsb=mn - 1) == _lib.STREAMKL_ERR_WORKSPACE
    assert bwd(L, p, dq1=None) == _lib.STREAMKL_ERR_NULL       # half pair
    assert bwd(L, p, dk2=None) == _lib.STREAMKL_ERR_NULL
    assert bwd(L, p, ws=None) == _lib.STREAMKL_ERR_WORKSPACE
    assert bwd(L, P(B=4, H=8), wsb=64) == _lib.STREAMKL_ERR_WORKSPACE
    assert bwd(L, p, g=None) == _lib.STREAMKL_ERR_NULL
    assert bwd(L, p, kl=MIS) == _lib.STREAMKL_ERR_ALIGN
    assert bwd(L, p, dk1=MIS) == _lib.STREAMKL_ERR_ALIGN
    assert bwd(L, P(D=100)) == _lib.STREAMKL_ERR_SHAPE
    # Both pairs skipped: nothing to do.
    assert bwd(L, p, dq1=None, dk1=None, dq2=None, dk2=None, ws=None) == _lib.STREAMKL_OK


def test_backward_step_validation(L):
    p = P()
    prep = lambda g=A, ws=A, wsb=1 << 20, pp=p, q1=A, k2=A: L.streamkl_bwd_prepare(ctypes.byref(pp), q1, A, A, k2,
                                                                                   g, ws, wsb, None)
    assert prep(g=None) == _lib.STREAMKL_ERR_NULL
    assert prep(q1=None) == _lib.STREAMKL_ERR_NULL
    assert prep(k2=MIS) == _lib.STREAMKL_ERR_ALIGN
    assert prep(ws=None) == _lib.STREAMKL_ERR_WORKSPACE
    assert prep(wsb=4) == _lib.STREAMKL_ERR_WORKSPACE
    assert prep(ws=MIS) == _lib.STREAMKL_ERR_ALIGN
    assert prep(g=MIS) == _lib.STREAMKL_ERR_ALIGN
    assert prep(g=None, pp=P(NQ=0)) == _lib.STREAMKL_OK
    for name in ("streamkl_bwd_dk", "streamkl_bwd_dq"):
        fn = getattr(L, name)
        call = lambda a=A, b=A, ws=A, wsb=1 << 20, kl=A: fn(ctypes.byref(p), A, A, A, A, kl, A, A, A, a, b,
                                                             ws, wsb, None)
        assert call(ws=None) == _lib.STREAMKL_ERR_WORKSPACE, name
        assert call(wsb=8) == _lib.STREAMKL_ERR_WORKSPACE, name
        assert call(a=MIS) == _lib.STREAMKL_ERR_ALIGN, name
        assert call(kl=None) == _lib.STREAMKL_ERR_NULL, name
        assert call(a=None, b=None, ws=None) == _lib.STREAMKL_OK, name
        assert fn(ctypes.byref(P(dtype=5)), A, A, A, A, A, A, A, A, A, A, A, 64, None) == _lib.STREAMKL_ERR_DTYPE


class VP:
    """streamkl_varlen_problem with its host offset arrays kept alive."""

    def __init__(self, cu_q, cu_k, H=2, D=64, causal=0, dtype=_lib.STREAMKL_BF16, null_cu=False):
        self.cq = (ctypes.c_int32 * len(cu_q))(*cu_q)
        self.ck = (ctypes.c_int32 * len(cu_k))(*cu_k)
        self.p = _lib.VarlenProblem(len(cu_q) - 1, H, D, None if null_cu else ctypes.addressof(self.cq),
                                    ctypes.addressof(self.ck), 0.125, causal, dtype)

    def ref(self):
        return ctypes.byref(self.p)


def vfwd(L, v, q1=A, kl=A):
    return L.streamkl_fwd_varlen(v.ref(), q1, A, A, A, kl, A, A, None)


def vbwd(L, v, ws=A, wsb=1 << 30, dq1=A, dk1=A, g=A, q2=A):
    return L.streamkl_bwd_varlen(v.ref(), A, A, q2, A, A, A, A, g, dq1, dk1, A, A, ws, wsb, None)


def test_varlen_validation(L):
    assert L.streamkl_fwd_varlen(None, A, A, A, A, A, A, A, None) == _lib.STREAMKL_ERR_NULL
    assert vfwd(L, VP([0, 5], [0, 5], null_cu=True)) == _lib.STREAMKL_ERR_NULL
    assert vfwd(L, VP([1, 5], [0, 5])) == _lib.STREAMKL_ERR_SHAPE              # first offset not 0
    assert vfwd(L, VP([0, 5, 3], [0, 5, 9])) == _lib.STREAMKL_ERR_SHAPE        # decreasing
    assert vfwd(L, VP([0, 5, 9], [0, 5, 5])) == _lib.STREAMKL_ERR_SHAPE        # queries without keys
    assert vfwd(L, VP([0, 5, 9], [0, 5, 8], causal=1)) == _lib.STREAMKL_ERR_SHAPE  # 4 queries > 3 keys
    assert vfwd(L, VP([0, 5], [0, 5], D=96)) == _lib.STREAMKL_ERR_SHAPE
    assert vfwd(L, VP([0, 5], [0, 5], dtype=9)) == _lib.STREAMKL_ERR_DTYPE
    assert vfwd(L, VP([0, 5], [0, 5], dtype=_lib.STREAMKL_FP8_E4M3), q1=None) == _lib.STREAMKL_ERR_NULL
    assert vbwd(L, VP([0, 5], [0, 5], dtype=_lib.STREAMKL_FP8_E4M3), g=None) == _lib.STREAMKL_ERR_NULL
    assert vfwd(L, VP([0, 5], [0, 5]), q1=None) == _lib.STREAMKL_ERR_NULL
    assert vfwd(L, VP([0, 5], [0, 5]), q1=MIS) == _lib.STREAMKL_ERR_ALIGN
    assert vfwd(L, VP([0, 5], [0, 5]), kl=MIS) == _lib.STREAMKL_ERR_ALIGN
    # Nothing to compute: no sequences, no heads, or no query rows at all.
    assert vfwd(L, VP([0], [0]), q1=None, kl=None) == _lib.STREAMKL_OK
    assert vfwd(L, VP([0, 5], [0, 5], H=0), q1=None, kl=None) == _lib.STREAMKL_OK
    assert vfwd(L, VP([0, 0, 0], [0, 4, 9]), q1=None, kl=None) == _lib.STREAMKL_OK


def varlen_bf16_workspace(B, H, D, runs):
    # sigma, operand scales and chunk maxima of every (sequence, head), laid out
    # as for a problem of B * H heads, or, if larger, the largest workspace of
    # a run that runs on its own.  All runs join the segmented passes when the
    # batch has at least 256 query tiles of 128 rows; otherwise those whose own
    # query pass would split its keys run alone.
    fills = sum(b * H * ((nq + 127) // 128) for b, nq, nk in runs) >= 256
    need = bwd_workspace(B, H, 0, 0, D, split=False)
    for b, nq, nk in runs:
        if not fills and dq_splits(b, H, nq, nk) > 1:
            need = max(need, bwd_workspace(b, H, nq, nk, D))
    return need


def test_varlen_backward_validation(L):
    # Runs of equal lengths: (3,3) x2, (64,200), (0,7), (65,65).  The (3,3) run joins
    # the segmented passes; (64,200) and (65,65) split their query pass's keys
    # and run on their own.
    cu_q = [0, 3, 6, 70, 70, 135]
    cu_k = [0, 3, 6, 206, 213, 278]
    v = VP(cu_q, cu_k, H=3, D=128)
    need = L.streamkl_bwd_varlen_workspace_size(v.ref())
    runs = [(2, 3, 3), (1, 64, 200), (1, 65, 65)]
    assert [dq_splits(b, 3, nq, nk) > 1 for b, nq, nk in runs] == [False, True, True]
    assert need == varlen_bf16_workspace(5, 3, 128, runs)
    # A batch of 448 query tiles: every run joins, although the (300, 300) run
    # alone would split.
    v2 = VP([0, 300, 600, 1600], [0, 300, 600, 1600], H=32, D=64)
    runs2 = [(2, 300, 300), (1, 1000, 1000)]
    assert dq_splits(2, 32, 300, 300) > 1
    assert L.streamkl_bwd_varlen_workspace_size(v2.ref()) == varlen_bf16_workspace(3, 32, 64, runs2)
    f32 = VP(cu_q, cu_k, H=3, D=128, dtype=_lib.STREAMKL_FP32)
    # fp32: sigma and the (unit) operand scales of all 5 x 3 (sequence, head) pairs.
    assert L.streamkl_bwd_varlen_workspace_size(f32.ref()) == 512
    assert L.streamkl_bwd_varlen_workspace_size(VP([2, 3], [0, 3]).ref()) == 0
    assert vbwd(L, v, wsb=need - 1) == _lib.STREAMKL_ERR_WORKSPACE
    assert vbwd(L, v, ws=None) == _lib.STREAMKL_ERR_WORKSPACE
    assert vbwd(L, v, ws=MIS) == _lib.STREAMKL_ERR_ALIGN
    assert vbwd(L, v, dq1=None) == _lib.STREAMKL_ERR_NULL     # half pair
    assert vbwd(L, v, g=None) == _lib.STREAMKL_ERR_NULL
    assert vbwd(L, v, q2=MIS) == _lib.STREAMKL_ERR_ALIGN
    assert vbwd(L, v, dk1=MIS) == _lib.STREAMKL_ERR_ALIGN
    assert vbwd(L, VP([0, 4], [0, 3], causal=1)) == _lib.STREAMKL_ERR_SHAPE
    # Both pairs skipped: nothing to do.
    assert L.streamkl_bwd_varlen(v.ref(), A, A, A, A, A, A, A, A, None, None, None, None, None, 0,
                                 None) == _lib.STREAMKL_OK


def test_mfma_probe_rejects_bad_arguments(L):
    # Each call fails validation on the host; none launches the probe.
    probe = L.streamkl_probe_mfma_bf16
    assert probe(0, 1, A, None) == 2          # no iterations
    assert probe(1 << 25, 1, A, None) == 2    # too many iterations
    assert probe(1, 0, A, None) == 2          # no workgroups
    assert probe(1, (1 << 20) + 1, A, None) == 2
    assert probe(1, 1, None, None) == 1       # NULL sink
    assert probe(1, 1, MIS, None) == 4        # misaligned sink
