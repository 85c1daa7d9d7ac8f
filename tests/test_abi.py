"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/dflash.h, shares torch's HIP runtime, and rejects bad
arguments before any HIP call (a fully valid call on a GPU-less host fails
with DFLASH_ERR_DEVICE instead of falling back to anything)."""

import ctypes
import os
import re

import pytest
import torch

import block_draft_verification_amd as dfl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dflash.h")
OK, INVALID, UNSUPPORTED, WORKSPACE, LAUNCH, DEVICE = 0, 1, 2, 3, 4, 5

needs_lib = pytest.mark.skipif(not os.path.exists(dfl.LIB_PATH), reason="libdflash.so not built")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int)\s+(dflash_\w+)\s*\(", text, re.M)))


def test_header_declares_the_five_steps():
    names = declared_functions()
    for n in ("dflash_conv2tap", "dflash_head_topk", "dflash_select_path",
              "dflash_verify_greedy", "dflash_verify_sample"):
        assert n in names


@needs_lib
def test_library_exports_every_declared_function():
    L = dfl.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(dfl.EXPORTS)
    assert dfl.status_string(WORKSPACE) == "workspace too small"
    assert L.dflash_version() >> 16 == 1


@needs_lib
def test_single_hip_runtime_in_process():
    dfl.lib()
    maps = open("/proc/self/maps").read()
    paths = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(paths) == 1, paths


# fake, 256-byte aligned, non-overlapping device addresses for validation tests
A = [ctypes.c_void_p((i + 1) << 40) for i in range(16)]
NULL = None


def ws_query(fn, *before, after=(None,)):
    n = ctypes.c_size_t(0)
    st = fn(*before, NULL, ctypes.byref(n), *after)
    return st, n.value


@needs_lib
def test_conv_validation():
    f = dfl.lib().dflash_conv2tap
    assert f(NULL, A[1], A[2], 1, 8, 64, NULL) == INVALID
    assert f(A[0], A[1], A[2], 0, 8, 64, NULL) == INVALID          # n_seq
    assert f(A[0], A[1], A[2], 1, 17, 64, NULL) == INVALID         # T > 16
    assert f(A[0], A[1], A[2], 1, 8, 60, NULL) == INVALID          # D % 8
    assert f(A[0], A[1], A[0], 1, 8, 64, NULL) == INVALID          # y == x
    assert f(A[0], A[1], ctypes.c_void_p((1 << 40) + 8), 1, 8, 64, NULL) == INVALID  # overlap
    assert f(ctypes.c_void_p((1 << 40) + 8), A[1], A[2], 1, 8, 64, NULL) == INVALID  # misaligned
    if not torch.cuda.is_available():
        assert f(A[0], A[1], A[2], 1, 8, 64, NULL) == DEVICE


@needs_lib
def test_conv_proj_validation():
    f = dfl.lib().dflash_conv2tap_proj
    assert f(A[0], NULL, A[2], 1, 8, 64, NULL) == INVALID
    assert f(A[0], A[1], A[2], 0, 8, 64, NULL) == INVALID          # n_seq
    assert f(A[0], A[1], A[2], 1, 0, 64, NULL) == INVALID          # T < 1
    assert f(A[0], A[1], A[2], 1, 17, 64, NULL) == INVALID         # T > 16
    assert f(A[0], A[1], A[2], 1, 8, 32, NULL) == INVALID          # D < 64
    assert f(A[0], A[1], A[2], 1, 8, 96, NULL) == INVALID          # D % 64
    assert f(A[0], A[1], A[0], 1, 8, 64, NULL) == INVALID          # y == x
    assert f(A[0], A[1], A[1], 1, 8, 64, NULL) == INVALID          # y == w_tap
    assert f(A[0], A[1], ctypes.c_void_p((2 << 40) + 4096), 1, 8, 64, NULL) == INVALID  # y inside w_tap
    assert f(A[0], ctypes.c_void_p((2 << 40) + 8), A[2], 1, 8, 64, NULL) == INVALID  # misaligned
    if not torch.cuda.is_available():
        assert f(A[0], A[1], A[2], 1, 8, 64, NULL) == DEVICE


@needs_lib
def test_head_validation_and_workspace():
    f = dfl.lib().dflash_head_topk
    st, need = ws_query(f, A[0], A[1], 7, 5120, 151936, 16, A[2], A[3])
    assert st == OK and need >= 7 * 16 * 8
    st2, need2 = ws_query(f, A[0], A[1], 480, 5120, 262144, 16, A[2], A[3])
    assert st2 == OK and need2 > need
    assert ws_query(f, A[0], A[1], 7, 5120, 151936, 8, A[2], A[3])[0] == UNSUPPORTED
    assert ws_query(f, A[0], A[1], 7, 5120, 15, 16, A[2], A[3])[0] == INVALID     # V < K
    assert ws_query(f, A[0], A[1], 0, 5120, 4096, 16, A[2], A[3])[0] == INVALID
    assert ws_query(f, A[0], A[1], 7, 5121, 4096, 16, A[2], A[3])[0] == INVALID
    assert ws_query(f, A[0], A[1], 7, 65544, 4096, 16, A[2], A[3])[0] == INVALID   # D > 65536
    assert ws_query(f, A[0], A[1], 7, 65536, 4096, 16, A[2], A[3])[0] == OK
    assert ws_query(f, NULL, A[1], 7, 256, 4096, 16, A[2], A[3])[0] == INVALID
    small = ctypes.c_size_t(need - 1)
    assert f(A[0], A[1], 7, 5120, 151936, 16, A[2], A[3], A[4], ctypes.byref(small), NULL) == WORKSPACE
    assert f(A[0], A[1], 7, 5120, 151936, 16, A[2], A[3], A[4], NULL, NULL) == INVALID
    ok = ctypes.c_size_t(need)
    # output aliasing the input hidden states
    assert f(A[0], A[1], 7, 5120, 151936, 16, A[0], A[3], A[4], ctypes.byref(ok), NULL) == INVALID
    if not torch.cuda.is_available():
        assert f(A[0], A[1], 7, 5120, 151936, 16, A[2], A[3], A[4], ctypes.byref(ok), NULL) == DEVICE


@needs_lib
def test_head_noalloc_validation():
    """The allocation-free head checks like dflash_head_topk and rejects sizes
    whose partial lists exceed its 16 MiB static scratch, before any HIP call."""
    L = dfl.lib()
    f = L.dflash_head_topk_noalloc
    assert f(NULL, A[1], 7, 5120, 151936, 16, A[2], A[3], NULL) == INVALID
    assert f(A[0], A[1], 7, 5120, 151936, 8, A[2], A[3], NULL) == UNSUPPORTED
    assert f(A[0], A[1], 7, 5121, 151936, 16, A[2], A[3], NULL) == INVALID
    assert f(A[0], A[1], 7, 5120, 151936, 16, A[0], A[3], NULL) == INVALID       # output aliases h
    # 2^18 rows need 32 MiB of partial lists: rejected on size
    need = ws_query(L.dflash_head_topk, A[0], A[1], 1 << 18, 256, 4096, 16, A[2], A[3])[1]
    assert need > 16 << 20
    assert f(A[0], A[1], 1 << 18, 256, 4096, 16, A[2], A[3], NULL) == WORKSPACE
    # every M up to 65536 fits at V <= 262144
    for M, V in ((65536, 4096), (65536, 262144), (224, 151936), (480, 262144), (7, 151936)):
        assert ws_query(L.dflash_head_topk, A[0], A[1], M, 256, V, 16, A[2], A[3])[1] <= 16 << 20
    if not torch.cuda.is_available():
        assert f(A[0], A[1], 7, 5120, 151936, 16, A[2], A[3], NULL) == DEVICE


@needs_lib
def test_select_validation():
    f = dfl.lib().dflash_select_path
    n = ctypes.c_size_t(0)
    args = lambda B, P, K, V, r, out0=A[4], ws=NULL: (A[0], A[1], A[2], A[3], B, P, K, V, r, out0, A[5], A[6],
                                                      ws, ctypes.byref(n), NULL)
    assert f(*args(1, 7, 8, 4096, 32)) == UNSUPPORTED
    assert f(*args(1, 16, 16, 4096, 32)) == INVALID
    assert f(*args(1, 0, 16, 4096, 32)) == INVALID
    assert f(*args(1, 7, 16, 4096, 30)) == INVALID
    assert f(*args(1, 7, 16, 4096, 512)) == INVALID
    assert f(*args(1, 7, 16, 4096, 32, out0=A[0])) == INVALID
    assert f(*args(4, 7, 16, 4096, 32)) == OK and n.value == 4 * 6 * 16 * 16 * 8
    n.value = 100
    assert f(*args(4, 7, 16, 4096, 32, ws=A[7])) == WORKSPACE
    if not torch.cuda.is_available():
        n.value = 1 << 20
        assert f(*args(2, 7, 16, 4096, 192, ws=A[7])) == DEVICE


@needs_lib
def test_verify_validation():
    g = dfl.lib().dflash_verify_greedy
    s = dfl.lib().dflash_verify_sample
    st, need = ws_query(g, A[0], A[1], 1, 8, 151936, A[2], A[3])
    assert st == OK and need > 0
    assert ws_query(g, A[0], A[1], 1, 1, 100, A[2], A[3])[0] == INVALID     # T < 2
    assert ws_query(g, A[0], A[1], 1, 17, 100, A[2], A[3])[0] == INVALID
    assert ws_query(g, A[0], A[1], 1, 8, 100, A[0], A[3])[0] == INVALID     # out aliases logits
    st, need_s = ws_query(s, A[0], A[1], 8, 8, 151936, 1.0, 0, A[4], A[5], A[2], A[3])
    assert st == OK and need_s > 0
    for bad_tau in (0.0, -1.0, float("inf"), float("nan")):
        assert ws_query(s, A[0], A[1], 8, 8, 100, bad_tau, 0, A[4], A[5], A[2], A[3])[0] == INVALID
    assert ws_query(s, A[0], A[1], 8, 8, 100, 1.0, 0, NULL, A[5], A[2], A[3])[0] == INVALID
    small = ctypes.c_size_t(need_s - 1)
    assert s(A[0], A[1], 8, 8, 151936, 1.0, 0, A[4], A[5], A[2], A[3], A[6], ctypes.byref(small),
             NULL) == WORKSPACE
    if not torch.cuda.is_available():
        ok = ctypes.c_size_t(need)
        assert g(A[0], A[1], 1, 8, 151936, A[2], A[3], A[6], ctypes.byref(ok), NULL) == DEVICE


def test_binding_refuses_cpu_tensors():
    x = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(dfl.DFlashError):
        dfl.conv2tap(x, torch.zeros(1, 8, 128, dtype=torch.bfloat16))


@needs_lib
def test_verify_topkp_validation():
    f = dfl.lib().dflash_verify_sample_topkp
    n = ctypes.c_size_t(0)
    q = lambda B, T, V, tau, k, p: f(A[0], A[1], B, T, V, tau, k, p, 0, A[4], A[5], A[2], A[3], NULL,
                                     ctypes.byref(n), NULL)
    assert q(8, 8, 151936, 1.0, 20, 0.95) == OK and n.value == 8 * 8 * 38 * 20 * 8 + 8 * 8 * 784
    for bad in [(8, 8, 100, 1.0, 0, 0.95), (8, 8, 100, 1.0, 65, 0.95), (8, 8, 100, 1.0, 20, 0.0),
                (8, 8, 100, 1.0, 20, 1.5), (8, 8, 100, 1.0, 20, float("nan")), (8, 8, 100, 0.0, 20, 0.9),
                (8, 17, 100, 1.0, 20, 0.9), (8, 1, 100, 1.0, 20, 0.9), (0, 8, 100, 1.0, 20, 0.9)]:
        assert q(*bad) == INVALID, bad
    small = ctypes.c_size_t(n.value - 1)
    assert f(A[0], A[1], 8, 8, 151936, 1.0, 20, 0.95, 0, A[4], A[5], A[2], A[3], A[6], ctypes.byref(small),
             NULL) == WORKSPACE
    if not torch.cuda.is_available():
        ok = ctypes.c_size_t(n.value)
        assert f(A[0], A[1], 8, 8, 151936, 1.0, 20, 0.95, 0, A[4], A[5], A[2], A[3], A[6], ctypes.byref(ok),
                 NULL) == DEVICE


@needs_lib
def test_select_anchored_validation():
    f = dfl.lib().dflash_select_path_anchored
    n = ctypes.c_size_t(0)
    args = lambda B, P, K, V, r, anchor=A[8], out0=A[4], ws=NULL: (A[0], A[1], anchor, A[2], A[3], B, P, K, V, r,
                                                                   out0, A[5], A[6], ws, ctypes.byref(n), NULL)
    assert f(*args(4, 7, 16, 4096, 32)) == OK and n.value == 4 * 7 * 16 * 16 * 8
    assert f(*args(4, 1, 16, 4096, 32)) == OK and n.value == 4 * 1 * 16 * 16 * 8
    assert f(*args(4, 7, 16, 4096, 32, anchor=NULL)) == INVALID
    assert f(*args(4, 7, 16, 4096, 32, anchor=ctypes.c_void_p((9 << 40) + 2))) == INVALID   # misaligned
    assert f(*args(4, 7, 8, 4096, 32)) == UNSUPPORTED
    assert f(*args(4, 7, 16, 4096, 32, out0=A[8])) == INVALID                             # output on the anchor
    if not torch.cuda.is_available():
        n.value = 1 << 20
        assert f(*args(2, 7, 16, 4096, 192, ws=A[7])) == DEVICE


@needs_lib
def test_sampled_selector_and_q_verify_validation():
    f = dfl.lib().dflash_select_path_sampled
    n = ctypes.c_size_t(0)
    P8 = [ctypes.c_void_p((i + 1) << 40) for i in range(12)]
    def sel(rid=P8[8], pos0=P8[9], q=P8[6], anchor=None, K=16):
        return f(P8[0], P8[1], anchor, P8[2], P8[3], 8, 7, K, 4096, 32, 0, rid, pos0, P8[4], P8[5], q, None,
                 ctypes.byref(n), None)
    assert sel() == OK and n.value == 8 * 6 * 256 * 8
    assert sel(anchor=P8[7]) == OK and n.value == 8 * 7 * 256 * 8
    assert sel(rid=None) == INVALID and sel(pos0=None) == INVALID and sel(q=None) == INVALID
    assert sel(q=ctypes.c_void_p(((7) << 40) + 4)) == INVALID           # f64 output not 8-byte aligned
    assert sel(rid=P8[4]) == INVALID                                      # request ids overlap path_rank
    assert sel(K=8) == UNSUPPORTED
    g = dfl.lib().dflash_verify_sample_q
    def ver(qi=P8[8], qp=P8[9], out=P8[2]):
        return g(P8[0], P8[1], qi, qp, 8, 8, 151936, 1.0, 0, P8[4], P8[5], out, P8[3], None, ctypes.byref(n), None)
    assert ver() == OK and n.value >= 8 * 8 * 38 * 16
    assert ver(qi=None) == INVALID and ver(qp=None) == INVALID
    assert ver(qp=ctypes.c_void_p(((10) << 40) + 4)) == INVALID
    assert ver(out=P8[8]) == INVALID                                      # out_tok overlaps q_idx


@needs_lib
def test_greedy_fused_validation():
    f = dfl.lib().dflash_verify_greedy_fused
    n = ctypes.c_size_t(0)
    P8 = [ctypes.c_void_p((i + 1) << 40) for i in range(8)]
    def call(B=1, T=8, D=5120, V=151936, h=P8[0], out=P8[3]):
        return f(h, P8[1], P8[2], B, T, D, V, out, P8[4], None, ctypes.byref(n), None)
    assert call() == OK and n.value >= 1 * 8 * 512 * 16 * 8 + 8 * 16 * 8
    assert call(T=1) == INVALID and call(T=17) == INVALID and call(D=5121) == INVALID and call(V=15) == INVALID
    assert call(h=None) == INVALID
    assert call(h=ctypes.c_void_p((1 << 40) + 8)) == INVALID         # h_t not 16-byte aligned
    assert call(out=P8[2]) == INVALID                                # out_tok overlaps the drafts


@needs_lib
def test_sample_fused_validation():
    f = dfl.lib().dflash_verify_sample_fused
    n = ctypes.c_size_t(0)
    P8 = [ctypes.c_void_p((i + 1) << 40) for i in range(8)]
    def call(B=8, T=8, D=5120, V=151936, tau=1.0, rid=P8[5], out=P8[3]):
        return f(P8[0], P8[1], P8[2], B, T, D, V, tau, 0, rid, P8[6], out, P8[4], None, ctypes.byref(n), None)
    assert call() == OK and n.value == 8 * 8 * 9496 * 8
    assert call(tau=0.0) == INVALID and call(tau=float("nan")) == INVALID and call(rid=None) == INVALID
    assert call(T=17) == INVALID and call(V=8) == INVALID and call(D=12) == INVALID
    assert call(out=P8[2]) == INVALID


@needs_lib
def test_certify_and_bound_validation():
    L = dfl.lib()
    S0 = ctypes.c_void_p(0)
    # weight bound: null pointers, bad D, GPU-less host
    assert L.dflash_head_weight_bound(NULL, 100, 64, A[1], NULL) == INVALID
    assert L.dflash_head_weight_bound(A[0], 100, 60, A[1], NULL) == INVALID
    assert L.dflash_head_weight_bound(A[0], 0, 64, A[1], NULL) == INVALID
    assert L.dflash_head_weight_bound(A[0], 100, 64, A[1], NULL) in (DEVICE, OK)
    # certify: K, sizes, a workspace smaller than the head's
    need = ctypes.c_size_t(0)
    assert L.dflash_head_topk(A[0], A[1], 224, 256, 8192, 16, A[2], A[3], NULL, ctypes.byref(need), NULL) == OK
    args = lambda K=16, ws=need.value, M=224: (A[0], M, 256, 8192, K, A[4], A[2], A[5], ws, A[6], NULL)
    assert L.dflash_head_topk_certify(*args(K=8)) == UNSUPPORTED
    assert L.dflash_head_topk_certify(*args(M=0)) == INVALID
    assert L.dflash_head_topk_certify(*args(ws=need.value - 16)) == WORKSPACE
    assert L.dflash_head_topk_certify(A[0], 224, 256, 8192, 16, NULL, A[2], A[5], need.value, A[6], NULL) == INVALID
    assert L.dflash_head_topk_certify(*args()) in (DEVICE, OK)
