"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before enqueueing."""
import ctypes
import os
import re

import pytest

from chunked_top_kl_head_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("kd_topk_kl.h", "kd_topk_select.h")]

# fake but well-aligned device addresses: validation never dereferences them
P16 = ctypes.c_void_p(0x100000)
P16b = ctypes.c_void_p(0x200000)
P4 = ctypes.c_void_p(0x300004)
MIS = ctypes.c_void_p(0x400002)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from chunked_top_kl_head_amd import build
        build.build()
    return B.load_library()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:kd_status|size_t|int64_t|const char\*)\s+(kd_\w+)\s*\(", text, re.M)))


def test_every_header_in_include_is_checked():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == sorted(os.path.basename(h) for h in HEADERS)


def test_header_declarations_match_binding():
    assert declared_functions() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def prob(T=64, d=64, V=1000, K=10, chunk=0, dtype=B.KD_BF16, tau=1.0):
    return B.KdProblem(T, d, V, K, chunk, dtype, tau)


def ws_size(lib, p, op):
    n = ctypes.c_size_t(0)
    st = lib.kd_topk_kl_workspace_size(ctypes.byref(p), op, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), B.KD_ERR_SHAPE), (dict(d=0), B.KD_ERR_SHAPE), (dict(V=0), B.KD_ERR_SHAPE),
    (dict(K=0), B.KD_ERR_SHAPE), (dict(K=1001), B.KD_ERR_SHAPE), (dict(chunk=-2), B.KD_ERR_SHAPE),
    (dict(tau=0.0), B.KD_ERR_VALUE), (dict(tau=-1.0), B.KD_ERR_VALUE), (dict(tau=float("nan")), B.KD_ERR_VALUE),
    (dict(tau=float("inf")), B.KD_ERR_VALUE), (dict(dtype=7), B.KD_ERR_UNSUPPORTED),
    (dict(d=60), B.KD_ERR_UNSUPPORTED), (dict(K=1025, V=5000), B.KD_ERR_UNSUPPORTED),
    (dict(V=(1 << 21) + 1), B.KD_ERR_UNSUPPORTED), (dict(T=1 << 31), B.KD_ERR_UNSUPPORTED),
    (dict(chunk=(1 << 20) + 1), B.KD_ERR_UNSUPPORTED),
])
def test_problem_validation(lib, kw, status):
    st, _ = ws_size(lib, prob(**kw), B.KD_OP_FUSED)
    assert st == status


def test_size_limit_rejected(lib):
    # W beyond the 2^31-byte operand limit
    st, _ = ws_size(lib, prob(d=8192, V=200000, K=10, dtype=B.KD_F32), B.KD_OP_FUSED)
    assert st == B.KD_ERR_UNSUPPORTED


def test_workspace_independent_of_T(lib):
    sizes = set()
    for T in (1, 4096, 32768, 262144):
        st, n = ws_size(lib, prob(T=T, d=2880, V=201088, K=100, chunk=2048), B.KD_OP_FUSED)
        assert st == B.KD_OK
        sizes.add(n)
    assert len(sizes) == 1
    (n,) = sizes
    # G chunk (C x V_pad bf16) dominates; far below the T x V logits
    assert 2048 * 201216 * 2 <= n < 2 * 2048 * 201216 * 2 + 64 * 2**20


def test_workspace_by_op(lib):
    p = prob(T=1000, d=256, V=4096, K=16, chunk=128)
    f = ws_size(lib, p, B.KD_OP_FORWARD)[1]
    b = ws_size(lib, p, B.KD_OP_BACKWARD)[1]
    u = ws_size(lib, p, B.KD_OP_FUSED)[1]
    assert 0 < f < u and 0 < b <= u
    assert ws_size(lib, p, 9)[0] == B.KD_ERR_VALUE
    assert lib.kd_topk_kl_workspace_size(ctypes.byref(p), 0, None) == B.KD_ERR_NULL
    assert lib.kd_topk_kl_workspace_size(None, 0, ctypes.byref(ctypes.c_size_t())) == B.KD_ERR_NULL


def test_default_chunk(lib):
    assert lib.kd_topk_kl_default_chunk(ctypes.byref(prob(d=2880, V=201088, K=100))) == 8192
    assert lib.kd_topk_kl_default_chunk(ctypes.byref(prob(K=0))) == 0
    # bf16 operands are addressed through rebased descriptors: no size cap
    assert lib.kd_topk_kl_default_chunk(ctypes.byref(prob(d=2880, V=2000000, K=100))) == 8192
    # fp32 operands keep 32-bit offsets: the chunk shrinks
    c = lib.kd_topk_kl_default_chunk(ctypes.byref(prob(d=64, V=500000, K=100, dtype=B.KD_F32)))
    assert 256 <= c < 8192 and c % 256 == 0


def test_large_bf16_chunk_accepted(lib):
    # chunk x V_pad x 2 bytes well beyond 2^31
    st, n = ws_size(lib, prob(T=65536, d=2880, V=201088, K=100, chunk=16384), B.KD_OP_FUSED)
    assert st == B.KD_OK and n >= 16384 * 201216 * 2


def call_fwd(lib, p, H=P16, W=P16b, idx=P4, lg=P4, ig=None, loss=P4, lse=P4, rl=None, ws=P16, wsb=1 << 40):
    return lib.kd_topk_kl_forward(ctypes.byref(p), H, W, idx, lg, ig, loss, lse, rl, ws, wsb, None)


def call_bwd(lib, p, H=P16, W=P16b, idx=P4, lg=P4, ig=None, lse=P4, g=None, gH=P16, gW=P16b, ws=P16, wsb=1 << 40):
    return lib.kd_topk_kl_backward(ctypes.byref(p), H, W, idx, lg, ig, lse, g, gH, gW, ws, wsb, None)


def call_fused(lib, p, H=P16, W=P16b, idx=P4, lg=P4, ig=None, g=None, loss=P4, lse=None, rl=None, gH=P16, gW=P16b,
               ws=P16, wsb=1 << 40):
    return lib.kd_topk_kl_fused(ctypes.byref(p), H, W, idx, lg, ig, g, loss, lse, rl, gH, gW, ws, wsb, None)


def call_noalloc(lib, p, H=P16, W=P16b, idx=P4, lg=P4, ig=None, g=None, loss=P4, lse=None, rl=None, gH=P16,
                 gW=P16b):
    return lib.kd_topk_kl_fused_noalloc(ctypes.byref(p), H, W, idx, lg, ig, g, loss, lse, rl, gH, gW, None)


def test_noalloc_argument_errors(lib):
    """Checked before the scratch is looked up, so no GPU is needed."""
    big = prob(T=20000, d=2880, V=201088, K=100, chunk=8192)     # 3.3 GB of workspace at this chunk
    assert call_noalloc(lib, big) == B.KD_ERR_WORKSPACE
    assert lib.kd_topk_kl_fused_noalloc(None, P16, P16b, P4, P4, None, None, P4, None, None, P16, P16b,
                                        None) == B.KD_ERR_NULL
    assert call_noalloc(lib, prob(K=0)) == B.KD_ERR_SHAPE
    assert call_noalloc(lib, prob(tau=0.0)) == B.KD_ERR_VALUE
    assert call_noalloc(lib, prob(), H=None) == B.KD_ERR_NULL
    assert call_noalloc(lib, prob(), loss=None) == B.KD_ERR_NULL
    assert call_noalloc(lib, prob(), gW=None) == B.KD_ERR_NULL
    assert call_noalloc(lib, prob(), H=P4) == B.KD_ERR_ALIGN
    assert call_noalloc(lib, prob(), gH=P4) == B.KD_ERR_ALIGN
    assert call_noalloc(lib, prob(), lse=MIS) == B.KD_ERR_ALIGN


def test_forward_argument_errors(lib):
    p = prob()
    assert call_fwd(lib, p, H=None) == B.KD_ERR_NULL
    assert call_fwd(lib, p, W=None) == B.KD_ERR_NULL
    assert call_fwd(lib, p, idx=None) == B.KD_ERR_NULL
    assert call_fwd(lib, p, lg=None) == B.KD_ERR_NULL
    assert call_fwd(lib, p, loss=None) == B.KD_ERR_NULL
    assert call_fwd(lib, p, lse=None) == B.KD_ERR_NULL
    assert call_fwd(lib, p, ws=None) == B.KD_ERR_NULL
    assert call_fwd(lib, p, H=MIS) == B.KD_ERR_ALIGN
    assert call_fwd(lib, p, W=P4) == B.KD_ERR_ALIGN
    assert call_fwd(lib, p, idx=MIS) == B.KD_ERR_ALIGN
    assert call_fwd(lib, p, lse=MIS) == B.KD_ERR_ALIGN
    assert call_fwd(lib, p, wsb=16) == B.KD_ERR_WORKSPACE
    assert call_fwd(lib, prob(K=2000)) == B.KD_ERR_SHAPE
    assert lib.kd_topk_kl_forward(None, P16, P16b, P4, P4, None, P4, P4, None, P16, 1 << 40, None) == B.KD_ERR_NULL


def test_backward_argument_errors(lib):
    p = prob()
    assert call_bwd(lib, p, lse=None) == B.KD_ERR_NULL
    assert call_bwd(lib, p, gH=None) == B.KD_ERR_NULL
    assert call_bwd(lib, p, gW=None) == B.KD_ERR_NULL
    assert call_bwd(lib, p, gH=P4) == B.KD_ERR_ALIGN
    assert call_bwd(lib, p, gW=P4) == B.KD_ERR_ALIGN
    assert call_bwd(lib, p, g=MIS) == B.KD_ERR_ALIGN
    assert call_bwd(lib, p, wsb=0) == B.KD_ERR_WORKSPACE
    assert call_bwd(lib, prob(tau=0.0)) == B.KD_ERR_VALUE


def test_fused_argument_errors(lib):
    p = prob()
    assert call_fused(lib, p, loss=None) == B.KD_ERR_NULL
    assert call_fused(lib, p, gW=None) == B.KD_ERR_NULL
    assert call_fused(lib, p, gH=None) == B.KD_ERR_NULL
    assert call_fused(lib, p, lse=MIS) == B.KD_ERR_ALIGN
    assert call_fused(lib, p, rl=MIS) == B.KD_ERR_ALIGN
    assert call_fused(lib, p, ws=P4) == B.KD_ERR_ALIGN
    assert call_fused(lib, p, wsb=100) == B.KD_ERR_WORKSPACE
    assert call_fused(lib, prob(d=12)) == B.KD_ERR_UNSUPPORTED


def test_validate_argument_errors(lib):
    p = prob()
    assert lib.kd_topk_kl_validate(ctypes.byref(p), P4, P4, None, None, None) == B.KD_ERR_NULL
    assert lib.kd_topk_kl_validate(ctypes.byref(p), None, P4, None, P16, None) == B.KD_ERR_NULL
    assert lib.kd_topk_kl_validate(ctypes.byref(p), P4, P4, None, P4, None) == B.KD_ERR_ALIGN


def test_problem_struct_layout():
    # int64 T, d, V, K, chunk; int32 dtype; float temperature; int32 flags, reserved
    assert ctypes.sizeof(B.KdProblem) == 56
    assert B.KdProblem.flags.offset == 48 and B.KdProblem.reserved.offset == 52


@pytest.mark.parametrize("flags,reserved,status", [
    (B.KD_FLAG_ACCUMULATE_GRAD_W, 0, B.KD_OK), (B.KD_FLAG_LOGIT_BF16, 0, B.KD_OK),
    (B.KD_FLAG_ACCUMULATE_GRAD_W | B.KD_FLAG_LOGIT_BF16, 0, B.KD_OK),
    (4, 0, B.KD_ERR_VALUE), (1 << 30, 0, B.KD_ERR_VALUE), (0, 1, B.KD_ERR_VALUE),
])
def test_flags_validation(lib, flags, reserved, status):
    p = prob()
    p.flags, p.reserved = flags, reserved
    assert ws_size(lib, p, B.KD_OP_FUSED)[0] == status


def test_bf16_logit_alignment(lib):
    p = prob()
    p.flags = B.KD_FLAG_LOGIT_BF16
    odd = ctypes.c_void_p(0x500001)
    assert call_fwd(lib, p, lg=odd) == B.KD_ERR_ALIGN
    assert call_bwd(lib, p, lg=odd) == B.KD_ERR_ALIGN
    assert call_fused(lib, p, lg=odd) == B.KD_ERR_ALIGN
    assert lib.kd_topk_kl_validate(ctypes.byref(p), P4, odd, None, P16, None) == B.KD_ERR_ALIGN
    # a 2-byte aligned fp32 cache is rejected
    assert call_fwd(lib, prob(), lg=MIS) == B.KD_ERR_ALIGN


def test_scale_grads_argument_errors(lib):
    p = prob()          # grad_H 64 x 64 bf16 (8 KiB), grad_W 1000 x 64 fp32 (250 KiB)
    F32, BF = B.KD_F32, B.KD_BF16
    sg = lib.kd_topk_kl_scale_grads
    P16c = ctypes.c_void_p(0x300000)
    P16d = ctypes.c_void_p(0x400000)
    # one of a pair missing
    assert sg(ctypes.byref(p), P4, P16, P16b, None, P16d, F32, None) == B.KD_ERR_NULL
    assert sg(ctypes.byref(p), P4, P16, P16b, P16c, None, F32, None) == B.KD_ERR_NULL
    assert sg(ctypes.byref(p), None, None, P16b, None, None, F32, None) == B.KD_ERR_NULL
    # alignment
    assert sg(ctypes.byref(p), MIS, P16, P16b, P16c, P16d, F32, None) == B.KD_ERR_ALIGN
    assert sg(ctypes.byref(p), P4, P4, P16b, P16c, P16d, F32, None) == B.KD_ERR_ALIGN
    assert sg(ctypes.byref(p), P4, P16, P4, P16c, P16d, F32, None) == B.KD_ERR_ALIGN
    assert sg(ctypes.byref(p), P4, P16, P16b, P4, P16d, F32, None) == B.KD_ERR_ALIGN
    assert sg(ctypes.byref(p), P4, P16, P16b, P16c, P4, BF, None) == B.KD_ERR_ALIGN
    # problem checks and the output type
    assert sg(ctypes.byref(prob(tau=0.0)), P4, P16, P16b, P16c, P16d, F32, None) == B.KD_ERR_VALUE
    assert sg(None, P4, P16, P16b, P16c, P16d, F32, None) == B.KD_ERR_NULL
    assert sg(ctypes.byref(p), P4, P16, P16b, P16c, P16d, 7, None) == B.KD_ERR_UNSUPPORTED
    # outputs that partly overlap their inputs (in place is the same pointer, same type)
    assert sg(ctypes.byref(p), P4, P16, None, ctypes.c_void_p(0x100000 + 4096), None, F32, None) == B.KD_ERR_VALUE
    assert sg(ctypes.byref(p), P4, None, P16b, None, P16b, BF, None) == B.KD_ERR_VALUE
    assert sg(ctypes.byref(p), P4, None, P16b, None, ctypes.c_void_p(0x200000 + 65536), F32, None) == \
        B.KD_ERR_VALUE


@pytest.mark.parametrize("name,splits", [("gptoss20b", 2), ("llama3b", 5)])
def test_fused_workspace_layout(lib, name, splits):
    """The fused workspace of a standard workload is the sum of the regions the
    layout documents, with the grad_H contraction split over the vocabulary
    `splits` ways (fewer than 512 output tiles: 12 x 32 = 384 at the
    GPT-OSS-like shape, 12 x 4 = 48 at the Llama-like one) -- pinned so that
    the documented layout and the code cannot drift apart."""
    from chunked_top_kl_head_amd import synth
    w = synth.WORKLOADS[name]
    C, d, V, K = w.chunk, w.d, w.V, w.K
    V_pad = (V + 255) // 256 * 256
    a = lambda x: (x + 255) // 256 * 256
    regions = [256,                                   # header (loss accumulator, N, s)
               a(4 * C),                              # chunk row losses
               a(8 * C * (V_pad // 128)),             # (reference, sum) per 128-id block
               a(2 * C * V_pad),                      # G, bf16, blocked
               a(4 * splits * C * d),                 # grad_H partials
               a(8 * C * K),                          # cached-entry list
               a(4 * C * K),                          # cached-id logits
               a(4 * C), a(4 * C), a(C),              # references, row factors, dirty flags
               a(2 * C * d)]                          # row-scaled H_c
    st, n = ws_size(lib, prob(T=w.T, d=d, V=V, K=K, chunk=C), B.KD_OP_FUSED)
    assert st == B.KD_OK and n == sum(regions)


def test_status_strings(lib):
    for s in range(9):
        msg = lib.kd_status_string(s).decode()
        assert msg and msg != "unknown status"
    assert lib.kd_status_string(99).decode() == "unknown status"


def sel(T=4, V=1000, K=10, ld=None, dtype=B.KD_BF16, reserved=0):
    return B.KdSelectProblem(T, V, K, V if ld is None else ld, dtype, reserved)


def test_select_struct_layout():
    assert ctypes.sizeof(B.KdSelectProblem) == 40


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), B.KD_ERR_SHAPE), (dict(V=0), B.KD_ERR_SHAPE), (dict(K=0), B.KD_ERR_SHAPE),
    (dict(K=1001), B.KD_ERR_SHAPE), (dict(ld=999), B.KD_ERR_SHAPE), (dict(reserved=3), B.KD_ERR_VALUE),
    (dict(dtype=5), B.KD_ERR_UNSUPPORTED), (dict(V=5000, K=1025), B.KD_ERR_UNSUPPORTED),
    (dict(V=1 << 31, K=10), B.KD_ERR_UNSUPPORTED),
])
def test_select_validation(lib, kw, status):
    assert lib.kd_topk_select(ctypes.byref(sel(**kw)), P16, P4, P4, None) == status


def test_select_argument_errors(lib):
    p = sel()
    assert lib.kd_topk_select(None, P16, P4, P4, None) == B.KD_ERR_NULL
    assert lib.kd_topk_select(ctypes.byref(p), None, P4, P4, None) == B.KD_ERR_NULL
    assert lib.kd_topk_select(ctypes.byref(p), P16, None, P4, None) == B.KD_ERR_NULL
    assert lib.kd_topk_select(ctypes.byref(p), P16, P4, None, None) == B.KD_ERR_NULL
    assert lib.kd_topk_select(ctypes.byref(p), ctypes.c_void_p(0x100001), P4, P4, None) == B.KD_ERR_ALIGN
    assert lib.kd_topk_select(ctypes.byref(sel(dtype=B.KD_F32)), MIS, P4, P4, None) == B.KD_ERR_ALIGN
    assert lib.kd_topk_select(ctypes.byref(p), P16, MIS, P4, None) == B.KD_ERR_ALIGN
    assert lib.kd_topk_select(ctypes.byref(p), P16, P4, MIS, None) == B.KD_ERR_ALIGN
    # no rows: nothing to do, nothing dereferenced
    assert lib.kd_topk_select(ctypes.byref(sel(T=0)), None, None, None, None) == B.KD_OK


def teacher(T=64, d=64, V=1000, K=10, chunk=0, dtype=B.KD_BF16, reserved=0):
    return B.KdTeacherProblem(T, d, V, K, chunk, dtype, reserved)


def teacher_ws(lib, p):
    n = ctypes.c_size_t(0)
    return lib.kd_teacher_topk_workspace_size(ctypes.byref(p), ctypes.byref(n)), n.value


def test_teacher_struct_layout():
    assert ctypes.sizeof(B.KdTeacherProblem) == 48


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), B.KD_ERR_SHAPE), (dict(d=0), B.KD_ERR_SHAPE), (dict(V=0), B.KD_ERR_SHAPE),
    (dict(K=0), B.KD_ERR_SHAPE), (dict(K=1001), B.KD_ERR_SHAPE), (dict(chunk=-1), B.KD_ERR_SHAPE),
    (dict(reserved=1), B.KD_ERR_VALUE), (dict(dtype=9), B.KD_ERR_UNSUPPORTED), (dict(d=60), B.KD_ERR_UNSUPPORTED),
    (dict(V=5000, K=1025), B.KD_ERR_UNSUPPORTED), (dict(V=(1 << 21) + 1), B.KD_ERR_UNSUPPORTED),
    (dict(T=1 << 31), B.KD_ERR_UNSUPPORTED), (dict(chunk=(1 << 20) + 1), B.KD_ERR_UNSUPPORTED),
    (dict(d=8192, V=200000, dtype=B.KD_F32), B.KD_ERR_UNSUPPORTED),
])
def test_teacher_validation(lib, kw, status):
    assert teacher_ws(lib, teacher(**kw))[0] == status
    assert lib.kd_teacher_topk(ctypes.byref(teacher(**kw)), P16, P16b, P4, P4, P16, 1 << 40, None) == status


def test_teacher_workspace_independent_of_T(lib):
    # one chunk of fp32 logits, rows padded to a multiple of 4 values
    st1, n1 = teacher_ws(lib, teacher(T=10, V=1001, chunk=512))
    st2, n2 = teacher_ws(lib, teacher(T=100000, V=1001, chunk=512))
    assert st1 == st2 == B.KD_OK and n1 == n2 and n1 >= 512 * 1004 * 4
    assert teacher_ws(lib, teacher(V=1001))[1] >= 4096 * 1004 * 4   # default chunk 4096


def test_teacher_argument_errors(lib):
    p = teacher()
    st, n = teacher_ws(lib, p)
    assert st == B.KD_OK
    assert lib.kd_teacher_topk_workspace_size(ctypes.byref(p), None) == B.KD_ERR_NULL
    assert lib.kd_teacher_topk(None, P16, P16b, P4, P4, P16, n, None) == B.KD_ERR_NULL
    assert lib.kd_teacher_topk(ctypes.byref(p), None, P16b, P4, P4, P16, n, None) == B.KD_ERR_NULL
    assert lib.kd_teacher_topk(ctypes.byref(p), P16, None, P4, P4, P16, n, None) == B.KD_ERR_NULL
    assert lib.kd_teacher_topk(ctypes.byref(p), P16, P16b, None, P4, P16, n, None) == B.KD_ERR_NULL
    assert lib.kd_teacher_topk(ctypes.byref(p), P16, P16b, P4, None, P16, n, None) == B.KD_ERR_NULL
    assert lib.kd_teacher_topk(ctypes.byref(p), P16, P16b, P4, P4, None, n, None) == B.KD_ERR_NULL
    assert lib.kd_teacher_topk(ctypes.byref(p), MIS, P16b, P4, P4, P16, n, None) == B.KD_ERR_ALIGN
    assert lib.kd_teacher_topk(ctypes.byref(p), P16, MIS, P4, P4, P16, n, None) == B.KD_ERR_ALIGN
    assert lib.kd_teacher_topk(ctypes.byref(p), P16, P16b, MIS, P4, P16, n, None) == B.KD_ERR_ALIGN
    assert lib.kd_teacher_topk(ctypes.byref(p), P16, P16b, P4, P4, P4, n, None) == B.KD_ERR_ALIGN
    assert lib.kd_teacher_topk(ctypes.byref(p), P16, P16b, P4, P4, P16, n - 1, None) == B.KD_ERR_WORKSPACE
    # no positions: nothing to do, nothing dereferenced
    assert lib.kd_teacher_topk(ctypes.byref(teacher(T=0)), None, None, None, None, None, 0, None) == B.KD_OK


def test_mfma_probe_library_loads_and_checks_arguments():
    """The MFMA-rate probe that bench.py --mfma-ceiling runs: built beside the
    library, exports its launcher, and rejects bad arguments before any launch."""
    from chunked_top_kl_head_amd import build as hip_build

    assert os.path.exists(hip_build.PROBE_LIB), "libkdprobe.so is not built"
    probe = ctypes.CDLL(hip_build.PROBE_LIB)
    f = probe.kd_probe_mfma_launch
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    buf = ctypes.c_void_p(16)   # never dereferenced: every call below is rejected first
    invalid = 1                 # hipErrorInvalidValue
    assert f(4, 256, 1000, buf, buf, None) == invalid      # unknown mode
    assert f(-1, 256, 1000, buf, buf, None) == invalid
    assert f(2, 0, 1000, buf, buf, None) == invalid        # no workgroups
    assert f(2, 256, 1001, buf, buf, None) == invalid      # odd step count
    assert f(0, 256, 0, buf, buf, None) == invalid
    assert f(1, 256, 1000, None, buf, None) == invalid     # missing buffers
    assert f(1, 256, 1000, buf, None, None) == invalid
