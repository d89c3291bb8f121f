"""Host-side checks of the C ABI (no GPU needed: nothing here reaches a kernel).

The library must load, export every function that include/csa_index.h
declares, and reject bad arguments on the host before any HIP call, with the
status codes the header documents.
"""

import ctypes
import os
import re

import pytest

import sparse_attention_indexer_csa_amd as csa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa_index.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, DEVICE = range(5)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return csa.load_library()


def test_library_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(csa.SIGNATURES) == names


def test_abi_version_and_status_strings(lib):
    assert lib.csa_index_abi_version() == 1
    for s in range(5):
        assert lib.csa_status_string(s)
    assert lib.csa_status_string(99) == b"unknown status"


def prob(B=1, S=16, H=4, D=32, W=8, m=4, scale=1.0, plan=0, **strides):
    st = dict(q_sb=H * S * D, q_sh=S * D, q_ss=D, k_sb=W * D, k_sw=D, w_sb=S * H, w_ss=H)
    st.update(strides)
    return csa._Problem(B, S, H, D, W, m, scale, plan, st["q_sb"], st["q_sh"], st["q_ss"], st["k_sb"], st["k_sw"],
                        st["w_sb"], st["w_ss"])


FAKE = 0x10000  # a 256-byte aligned non-null value; never dereferenced by these tests


def ws_size(lib, p, top_k):
    n = ctypes.c_size_t(12345)
    st = lib.csa_index_workspace_size(ctypes.byref(p), top_k, ctypes.byref(n))
    return st, n.value


@pytest.mark.parametrize("fields,status", [
    (dict(B=-1), INVALID), (dict(S=-1), INVALID), (dict(W=-2), INVALID), (dict(H=0), INVALID),
    (dict(D=0), INVALID), (dict(m=0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(scale=float("inf")), INVALID), (dict(plan=3), INVALID), (dict(plan=-1), INVALID),
    (dict(D=48), UNSUPPORTED), (dict(D=256), UNSUPPORTED), (dict(H=129), UNSUPPORTED),
    (dict(q_ss=36), UNSUPPORTED), (dict(k_sw=33), UNSUPPORTED), (dict(q_sh=-32), INVALID),
])
def test_problem_validation(lib, fields, status):
    p = prob(**fields)
    st, _ = ws_size(lib, p, 4)
    assert st == status, lib.csa_last_error()
    assert lib.csa_last_error()
    assert lib.csa_index_resolve_plan(ctypes.byref(p)) == -1


def test_null_problem_and_outputs(lib):
    n = ctypes.c_size_t(0)
    assert lib.csa_index_workspace_size(None, 4, ctypes.byref(n)) == INVALID
    assert lib.csa_index_workspace_size(ctypes.byref(prob()), 4, None) == INVALID
    assert lib.csa_index_resolve_plan(None) == -1


@pytest.mark.parametrize("k,status", [(0, UNSUPPORTED), (-3, UNSUPPORTED), (2049, UNSUPPORTED), (1, OK), (2048, OK)])
def test_top_k_range(lib, k, status):
    st, _ = ws_size(lib, prob(), k)
    assert st == status


def test_plans_and_workspace_sizes(lib):
    # prefill shapes: row tiles, no workspace
    p = prob(B=1, S=16384, H=64, D=128, W=4096)
    assert lib.csa_index_resolve_plan(ctypes.byref(p)) == 1
    assert ws_size(lib, p, 512) == (OK, 0)
    # decode shapes: few rows, long cache -> split rows, workspace = rows*W*4
    p = prob(B=64, S=1, H=64, D=128, W=32768)
    assert lib.csa_index_resolve_plan(ctypes.byref(p)) == 2
    assert ws_size(lib, p, 512) == (OK, 64 * 32768 * 4)
    # forced plans are honoured
    p = prob(B=64, S=1, H=64, D=128, W=32768, plan=1)
    assert lib.csa_index_resolve_plan(ctypes.byref(p)) == 1
    assert ws_size(lib, p, 512) == (OK, 0)
    p = prob(B=1, S=256, H=4, D=32, W=64, plan=2)
    assert lib.csa_index_resolve_plan(ctypes.byref(p)) == 2
    assert ws_size(lib, p, 16) == (OK, 256 * 64 * 4)
    # short rows are not split even when there are few of them
    p = prob(B=1, S=256, H=4, D=32, W=64)
    assert lib.csa_index_resolve_plan(ctypes.byref(p)) == 1
    # the row-tile plan holds entries in 16 bits: W <= 65536
    p = prob(B=1, S=16384, H=64, D=128, W=65536)
    assert lib.csa_index_resolve_plan(ctypes.byref(p)) == 1
    p = prob(B=1, S=16384, H=64, D=128, W=65537)
    assert lib.csa_index_resolve_plan(ctypes.byref(p)) == 2
    p = prob(B=1, S=16384, H=64, D=128, W=65537, plan=1)
    assert lib.csa_index_resolve_plan(ctypes.byref(p)) == -1
    assert ws_size(lib, p, 512)[0] == UNSUPPORTED


def masks(q_offset=None, q_seg=None, k_seg=None):
    return csa._Masks(q_offset, q_seg, k_seg)


def test_select_rejects_bad_pointers_before_any_launch(lib):
    p = prob()
    idx = ctypes.c_void_p(FAKE)
    m = masks()

    def call(q=FAKE, k=FAKE, w=FAKE, msk=m, top_k=4, out=idx, ws=None, wsb=0, pp=p):
        return lib.csa_index_select(ctypes.byref(pp) if pp is not None else None, ctypes.c_void_p(q) if q else None,
                                    ctypes.c_void_p(k) if k else None, ctypes.c_void_p(w) if w else None,
                                    ctypes.byref(msk) if msk is not None else None, top_k, out, None, ws, wsb, None)

    assert call(pp=None) == INVALID
    assert call(q=0) == INVALID
    assert call(k=0) == INVALID
    assert call(w=0) == INVALID
    assert call(q=FAKE + 8) == INVALID  # q not 16-byte aligned
    assert call(k=FAKE + 4) == INVALID
    assert call(w=FAKE + 1) == INVALID
    assert call(out=None) == INVALID
    assert call(out=ctypes.c_void_p(FAKE + 2)) == INVALID
    assert call(top_k=0) == UNSUPPORTED
    assert call(msk=masks(q_seg=FAKE)) == INVALID  # q_seg without k_seg
    assert call(msk=masks(k_seg=FAKE)) == INVALID
    assert call(msk=masks(q_offset=FAKE + 2)) == INVALID
    # split plan without the workspace it needs
    ps = prob(plan=2)
    assert call(pp=ps) == WORKSPACE
    assert call(pp=ps, ws=ctypes.c_void_p(FAKE), wsb=16 * 8 * 4 - 1) == WORKSPACE
    assert call(pp=ps, ws=ctypes.c_void_p(FAKE + 16), wsb=16 * 8 * 4) == INVALID  # workspace alignment
    # empty problems succeed without touching the device
    assert call(pp=prob(S=0)) == OK
    assert call(pp=prob(B=0), q=0, k=0, w=0) == OK


def test_score_rejects_bad_pointers(lib):
    p = prob()
    m = masks()

    def call(q=FAKE, k=FAKE, w=FAKE, out=FAKE, pp=p):
        return lib.csa_index_score(ctypes.byref(pp), ctypes.c_void_p(q) if q else None,
                                   ctypes.c_void_p(k) if k else None, ctypes.c_void_p(w) if w else None,
                                   ctypes.byref(m), ctypes.c_void_p(out) if out else None, None)

    assert call(out=0) == INVALID
    assert call(out=FAKE + 1) == INVALID
    assert call(q=FAKE + 2) == INVALID
    assert call(pp=prob(W=0), k=0, out=0) == OK  # nothing to write
    assert call(pp=prob(D=40)) == UNSUPPORTED


def test_topk_validation(lib):
    def call(rows=4, W=8, k=2, s=FAKE, out=FAKE):
        return lib.csa_index_topk(rows, W, k, ctypes.c_void_p(s) if s else None,
                                  ctypes.c_void_p(out) if out else None, None, 0, None)

    assert call(rows=-1) == INVALID
    assert call(W=-1) == INVALID
    assert call(k=0) == UNSUPPORTED
    assert call(k=4096) == UNSUPPORTED
    assert call(out=0) == INVALID
    assert call(s=0) == INVALID
    assert call(s=FAKE + 2) == INVALID
    assert call(rows=0) == OK
    n = ctypes.c_size_t(7)
    assert lib.csa_index_topk_workspace_size(10, 100, 5, ctypes.byref(n)) == OK and n.value == 0
    assert lib.csa_index_topk_workspace_size(10, 100, 0, ctypes.byref(n)) == UNSUPPORTED


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 16, 32, dtype=torch.bfloat16)
    k = torch.zeros(1, 8, 32, dtype=torch.bfloat16)
    w = torch.zeros(1, 16, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        csa.select(q, k, w, 4, 4)
    with pytest.raises(ValueError):
        csa.topk(torch.zeros(2, 8), 2)


def test_backward_workspace_and_validation(lib):
    """The backward checks every pointer and the workspace on the host; an
    empty batch succeeds without a launch."""
    n = ctypes.c_size_t(0)
    p = prob(B=2, S=600, H=4, D=32, W=40)
    assert lib.csa_index_backward_workspace_size(ctypes.byref(p), ctypes.byref(n)) == OK
    # B * ceil(S/256) row chunks * W * D fp32 partials (30720 bytes, a multiple
    # of 256), then B * S * ceil(W/32) * H 32-bit logit-sign words
    assert n.value == 2 * 3 * 40 * 32 * 4 + 2 * 600 * 2 * 4 * 4
    assert lib.csa_index_backward_workspace_size(ctypes.byref(prob(D=40)), ctypes.byref(n)) == UNSUPPORTED
    assert lib.csa_index_backward_workspace_size(None, ctypes.byref(n)) == INVALID
    # the plan field is not used by the backward
    assert lib.csa_index_backward_workspace_size(ctypes.byref(prob(W=70000, plan=1)), ctypes.byref(n)) == OK

    p = prob()
    need = 8 * 32 * 4 + 16 * 4 * 4  # one chunk of W=8 entries x D=32, then 16 rows x 4 heads of sign words
    m = masks()

    def call(q=FAKE, k=FAKE, w=FAKE, g=FAKE, dq=FAKE, dk=FAKE, dw=FAKE, ws=FAKE, wsb=need * 2, pp=p):
        v = lambda x: ctypes.c_void_p(x) if x else None
        return lib.csa_index_score_backward(ctypes.byref(pp), v(q), v(k), v(w), ctypes.byref(m), v(g), v(dq),
                                            v(dk), v(dw), v(ws), wsb, None)

    assert call(q=0) == INVALID
    assert call(g=0) == INVALID
    assert call(g=FAKE + 2) == INVALID
    assert call(dq=0) == INVALID
    assert call(dw=0) == INVALID
    assert call(dk=0) == INVALID
    assert call(dk=FAKE + 4) == INVALID  # dk must be 16-byte aligned
    assert call(ws=0) == WORKSPACE
    assert call(wsb=need - 1) == WORKSPACE
    assert call(ws=FAKE + 16) == INVALID
    assert call(pp=prob(D=40)) == UNSUPPORTED
    assert call(pp=prob(H=130)) == UNSUPPORTED
    assert call(pp=prob(B=0), q=0, k=0, w=0, g=0, dq=0, dk=0, dw=0, ws=0, wsb=0) == OK


def test_binding_refuses_short_mask_tensors():
    """Every mask element is read by the kernels, so the binding checks the
    full shapes before anything reaches the library: a k_seg shorter than W
    (or a q_seg shorter than S, a q_offset shorter than B) is refused."""
    import torch
    B, S, W = 2, 16, 8
    seg_q = torch.zeros(B, S, dtype=torch.int32)
    seg_k = torch.zeros(B, W, dtype=torch.int32)
    csa.check_mask_shapes(B, S, W, torch.zeros(B, dtype=torch.int32), seg_q, seg_k)
    with pytest.raises(ValueError, match="k_seg"):
        csa.check_mask_shapes(B, S, W, None, seg_q, torch.zeros(B, W - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="k_seg"):
        csa.check_mask_shapes(B, S, W, None, seg_q, torch.zeros(B, W + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="q_seg"):
        csa.check_mask_shapes(B, S, W, None, torch.zeros(B, S - 1, dtype=torch.int32), seg_k)
    with pytest.raises(ValueError, match="q_offset"):
        csa.check_mask_shapes(B, S, W, torch.zeros(B - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="int32"):
        csa.check_mask_shapes(B, S, W, None, seg_q, seg_k.long())
    with pytest.raises(ValueError, match="together"):
        csa.check_mask_shapes(B, S, W, None, seg_q, None)
    with pytest.raises(ValueError, match="contiguous"):
        csa.check_mask_shapes(B, S, W, None, seg_q, torch.zeros(B, 2 * W, dtype=torch.int32)[:, ::2])


def test_key_stride_below_row_width_is_accepted(lib):
    """Entries may overlap (0 < k_sw < D) or repeat (k_sw = 0, which the
    binding passes for a one-entry cache): only multiples of 8 are required."""
    for k_sw in (0, 8, 16):
        st, _ = ws_size(lib, prob(D=32, k_sw=k_sw), 4)
        assert st == OK, lib.csa_last_error()


def test_noalloc_refuses_oversized_workspace_on_the_host(lib):
    """The no-allocation select checks the problem's workspace against its
    fixed scratch (16 MiB) before touching the device."""
    assert csa.NOALLOC_SCRATCH_BYTES == 16 << 20
    p = prob(B=128, S=1, H=4, D=32, W=40000, plan=2)
    st, need = ws_size(lib, p, 16)
    assert st == OK and need > csa.NOALLOC_SCRATCH_BYTES
    m = masks()
    f = ctypes.c_void_p(FAKE)
    st = lib.csa_index_select_noalloc(ctypes.byref(p), f, f, f, ctypes.byref(m), 16, f, None, None)
    assert st == WORKSPACE
    assert b"scratch" in lib.csa_last_error()
    assert lib.csa_index_select_noalloc(None, f, f, f, ctypes.byref(m), 16, f, None, None) == INVALID
    assert lib.csa_index_select_noalloc(ctypes.byref(prob()), f, f, f, ctypes.byref(m), 0, f, None, None) \
        == UNSUPPORTED


def test_kl_loss_validation(lib):
    """The loss checks its pointers on the host; an empty problem succeeds
    without a launch."""
    m = masks()
    v = lambda x: ctypes.c_void_p(x) if x else None

    def call(q=FAKE, k=FAKE, w=FAKE, t=FAKE, kl=FAKE, g=0, pp=None):
        pp = pp or prob()
        return lib.csa_index_kl_loss(ctypes.byref(pp), v(q), v(k), v(w), ctypes.byref(m), v(t), v(kl), v(g), None)

    assert lib.csa_index_kl_loss(None, v(FAKE), v(FAKE), v(FAKE), ctypes.byref(m), v(FAKE), v(FAKE), None,
                                 None) == INVALID
    assert call(kl=0) == INVALID
    assert call(kl=FAKE + 2) == INVALID
    assert call(t=0) == INVALID
    assert call(t=FAKE + 1) == INVALID
    assert call(g=FAKE + 2) == INVALID
    assert call(q=0) == INVALID
    assert call(pp=prob(D=48)) == UNSUPPORTED
    assert call(pp=prob(S=0), kl=0) == OK
    # the plan field is ignored: a forced row-tile plan beyond its W limit is fine here
    assert call(pp=prob(W=70000, plan=1), kl=0) == INVALID  # still needs kl
