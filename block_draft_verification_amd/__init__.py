"""Python binding of libdflash.so: the DFlash 2 cycle tail on MI355X (gfx950).

Argument marshalling only.  Every step runs in the library's HIP kernels on the
caller's current torch stream; tensors provide device memory.  There is no
fallback: if the library is missing or a call fails, an exception is raised.

Entry points (same names and semantics as include/dflash.h):
    conv2tap(x, taps)                         -> y
    conv2tap_proj(x, w_tap)                   -> y   (taps projected in the call)
    head_topk(h, W, K=16)                     -> (top_val, top_idx)
    select_path(top_val, top_idx, F_l, F_r)   -> (path_rank, path_tok, path_score)
    verify_greedy(logits, draft)              -> (out_tok, n_emit)
    verify_sample(logits, draft, temperature, seed, request_id, pos0)
                                              -> (out_tok, n_emit)
and the variants select_path(..., anchor=...), select_path_sampled(...) ->
(path_rank, path_tok, path_q), verify_sample_q(...), verify_sample_topkp(...).
"""

import ctypes
import os

import torch  # loads the HIP runtime the library binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
# DFLASH_LIB names another build of the same library (the host-sanitized one
# for the C-ABI checks); by default the one next to this file.
LIB_PATH = os.environ.get("DFLASH_LIB") or os.path.join(_HERE, "libdflash.so")

_c_i32, _c_i64, _c_u64, _c_f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
_p, _psz = ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)

_SIGNATURES = {
    "dflash_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dflash_version": (ctypes.c_int, []),
    "dflash_conv2tap": (ctypes.c_int, [_p, _p, _p, _c_i64, _c_i32, _c_i32, _p]),
    "dflash_conv2tap_proj": (ctypes.c_int, [_p, _p, _p, _c_i64, _c_i32, _c_i32, _p]),
    "dflash_head_topk": (ctypes.c_int, [_p, _p, _c_i64, _c_i32, _c_i64, _c_i32, _p, _p, _p, _psz, _p]),
    "dflash_head_topk_noalloc": (ctypes.c_int, [_p, _p, _c_i64, _c_i32, _c_i64, _c_i32, _p, _p, _p]),
    "dflash_head_weight_bound": (ctypes.c_int, [_p, _c_i64, _c_i32, _p, _p]),
    "dflash_head_topk_certify": (ctypes.c_int, [_p, _c_i64, _c_i32, _c_i64, _c_i32, _p, _p, _p, ctypes.c_size_t,
                                                _p, _p]),
    "dflash_select_path": (ctypes.c_int, [_p, _p, _p, _p, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32,
                                          _p, _p, _p, _p, _psz, _p]),
    "dflash_select_path_anchored": (ctypes.c_int, [_p, _p, _p, _p, _p, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32,
                                                   _p, _p, _p, _p, _psz, _p]),
    "dflash_verify_greedy": (ctypes.c_int, [_p, _p, _c_i32, _c_i32, _c_i64, _p, _p, _p, _psz, _p]),
    "dflash_verify_sample": (ctypes.c_int, [_p, _p, _c_i32, _c_i32, _c_i64, _c_f32, _c_u64, _p, _p,
                                            _p, _p, _p, _psz, _p]),
    "dflash_verify_sample_topkp": (ctypes.c_int, [_p, _p, _c_i32, _c_i32, _c_i64, _c_f32, _c_i32, _c_f32,
                                                  _c_u64, _p, _p, _p, _p, _p, _psz, _p]),
    "dflash_select_path_sampled": (ctypes.c_int, [_p, _p, _p, _p, _p, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32,
                                                  _c_u64, _p, _p, _p, _p, _p, _p, _psz, _p]),
    "dflash_verify_sample_q": (ctypes.c_int, [_p, _p, _p, _p, _c_i32, _c_i32, _c_i64, _c_f32, _c_u64, _p, _p,
                                              _p, _p, _p, _psz, _p]),
    "dflash_verify_greedy_fused": (ctypes.c_int, [_p, _p, _p, _c_i32, _c_i32, _c_i32, _c_i64, _p, _p, _p, _psz,
                                                  _p]),
    "dflash_verify_sample_fused": (ctypes.c_int, [_p, _p, _p, _c_i32, _c_i32, _c_i32, _c_i64, _c_f32, _c_u64, _p,
                                                  _p, _p, _p, _p, _psz, _p]),
}
EXPORTS = tuple(_SIGNATURES)

_lib = None


class DFlashError(RuntimeError):
    pass


def lib():
    """Load libdflash.so once (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DFlashError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(code):
    return lib().dflash_status_string(code).decode()


def _check(code, what):
    if code != 0:
        raise DFlashError(f"{what}: {status_string(code)} ({code})")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name, dims=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise DFlashError(f"{name} must be a CUDA/HIP tensor")
    if t.dtype != dtype:
        raise DFlashError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise DFlashError(f"{name} must be contiguous")
    if dims is not None and t.dim() != dims:
        raise DFlashError(f"{name} must have {dims} dims, got {tuple(t.shape)}")


def _same_device(what, *ts):
    """Every tensor argument of one call must live on the same GPU."""
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise DFlashError(f"{what}: tensors on several devices {sorted(map(str, devs))}")


def _out(t, dtype, shape, device, name):
    """A caller-supplied output: the C ABI cannot see tensor sizes, so its
    dtype, exact shape, device and contiguity are checked here, before any
    launch."""
    _need(t, dtype, name)
    if tuple(t.shape) != tuple(shape):
        raise DFlashError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise DFlashError(f"{name} must be on {device}, got {t.device}")
    return t


def _outs(out, specs, device):
    """out=None allocates every output; else out is a tuple checked against
    specs [(dtype, shape, name), ...]."""
    if out is None:
        return tuple(torch.empty(shape, dtype=dt, device=device) for dt, shape, _ in specs)
    if not isinstance(out, (tuple, list)) or len(out) != len(specs):
        raise DFlashError(f"out must be a tuple of {len(specs)} tensors")
    return tuple(_out(t, dt, shape, device, name) for t, (dt, shape, name) in zip(out, specs))


def _workspace(fn, args_before, args_after, device, workspace):
    """Query the workspace size with a NULL workspace, then allocate if needed
    (a caller's workspace must be a contiguous uint8 tensor on the device)."""
    need = ctypes.c_size_t(0)
    _check(fn(*args_before, None, ctypes.byref(need), *args_after), fn.__name__ + " (workspace query)")
    n = max(int(need.value), 16)
    if workspace is not None:
        _need(workspace, torch.uint8, "workspace")
        if workspace.device != device:
            raise DFlashError(f"workspace must be on {device}, got {workspace.device}")
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(n, dtype=torch.uint8, device=device)
    return workspace, ctypes.c_size_t(workspace.numel())


def conv2tap(x, taps, out=None):
    """x bf16 [S][T][D], taps bf16 [S][T][2D] -> y bf16 [S][T][D]."""
    _need(x, torch.bfloat16, "x")
    _need(taps, torch.bfloat16, "taps")
    _same_device("conv2tap", x, taps)
    D = x.shape[-1]
    T = x.shape[-2]
    S = x.numel() // (T * D)
    if taps.shape[-1] != 2 * D or taps.numel() != 2 * x.numel():
        raise DFlashError("taps must be [..., T, 2*D] matching x")
    y = torch.empty_like(x) if out is None else _out(out, torch.bfloat16, x.shape, x.device, "out")
    _check(lib().dflash_conv2tap(_ptr(x), _ptr(taps), _ptr(y), S, T, D, _stream(x.device)),
           "dflash_conv2tap")
    return y


def conv2tap_proj(x, w_tap, out=None):
    """x bf16 [S][T][D], w_tap bf16 [2D][D] -> y bf16 [S][T][D]."""
    _need(x, torch.bfloat16, "x")
    _need(w_tap, torch.bfloat16, "w_tap")
    _same_device("conv2tap_proj", x, w_tap)
    D = x.shape[-1]
    T = x.shape[-2]
    S = x.numel() // (T * D)
    if tuple(w_tap.shape) != (2 * D, D):
        raise DFlashError("w_tap must be [2*D][D]")
    y = torch.empty_like(x) if out is None else _out(out, torch.bfloat16, x.shape, x.device, "out")
    _check(lib().dflash_conv2tap_proj(_ptr(x), _ptr(w_tap), _ptr(y), S, T, D, _stream(x.device)),
           "dflash_conv2tap_proj")
    return y


def head_topk(h, W, K=16, workspace=None, out=None):
    """h bf16 [M][D], W bf16 [V][D] -> (top_val f32 [M][K], top_idx i32 [M][K])."""
    _need(h, torch.bfloat16, "h", 2)
    _need(W, torch.bfloat16, "W", 2)
    M, D = h.shape
    V = W.shape[0]
    if W.shape[1] != D:
        raise DFlashError("W must be [V][D] with the same D as h")
    _same_device("head_topk", h, W)
    tv, ti = _outs(out, [(torch.float32, (M, K), "top_val"), (torch.int32, (M, K), "top_idx")], h.device)
    L = lib()
    before = (_ptr(h), _ptr(W), M, D, V, K, _ptr(tv), _ptr(ti))
    ws, nbytes = _workspace(L.dflash_head_topk, before, (_stream(h.device),), h.device, workspace)
    _check(L.dflash_head_topk(*before, _ptr(ws), ctypes.byref(nbytes), _stream(h.device)),
           "dflash_head_topk")
    return tv, ti


def head_weight_bound(W):
    """Bounds on W's rows for head_topk_certify: f32 [2] = (max row 2-norm,
    max row 1-norm), rounded up."""
    _need(W, torch.bfloat16, "W", 2)
    V, D = W.shape
    b = torch.empty(2, dtype=torch.float32, device=W.device)
    _check(lib().dflash_head_weight_bound(_ptr(W), V, D, _ptr(b), _stream(W.device)), "dflash_head_weight_bound")
    return b


def head_topk_certified(h, W, bound, K=16):
    """head_topk and its exactness certificate: (top_val, top_idx, certified
    i32 [M]: 1 where the 16 are shown to be the exact top-16).  bound from
    head_weight_bound(W)."""
    _need(h, torch.bfloat16, "h", 2)
    _need(W, torch.bfloat16, "W", 2)
    _need(bound, torch.float32, "bound", 1)
    if bound.numel() != 2:
        raise DFlashError("bound must hold 2 floats (head_weight_bound)")
    M, D = h.shape
    V = W.shape[0]
    if W.shape[1] != D:
        raise DFlashError("W must be [V][D] with the same D as h")
    _same_device("head_topk_certified", h, W, bound)
    L = lib()
    tv = torch.empty((M, K), dtype=torch.float32, device=h.device)
    ti = torch.empty((M, K), dtype=torch.int32, device=h.device)
    before = (_ptr(h), _ptr(W), M, D, V, K, _ptr(tv), _ptr(ti))
    ws, nbytes = _workspace(L.dflash_head_topk, before, (_stream(h.device),), h.device, None)
    _check(L.dflash_head_topk(*before, _ptr(ws), ctypes.byref(nbytes), _stream(h.device)), "dflash_head_topk")
    cert = torch.empty(M, dtype=torch.int32, device=h.device)
    _check(L.dflash_head_topk_certify(_ptr(h), M, D, V, K, _ptr(bound), _ptr(tv), _ptr(ws), nbytes.value,
                                      _ptr(cert), _stream(h.device)), "dflash_head_topk_certify")
    return tv, ti, cert


def head_topk_noalloc(h, W, K=16, out=None):
    """head_topk through the entry point that allocates nothing (the library's
    static per-GPU scratch array); out=(top_val, top_idx) may be preallocated."""
    _need(h, torch.bfloat16, "h", 2)
    _need(W, torch.bfloat16, "W", 2)
    M, D = h.shape
    V = W.shape[0]
    if W.shape[1] != D:
        raise DFlashError("W must be [V][D] with the same D as h")
    _same_device("head_topk_noalloc", h, W)
    tv, ti = _outs(out, [(torch.float32, (M, K), "top_val"), (torch.int32, (M, K), "top_idx")], h.device)
    _check(lib().dflash_head_topk_noalloc(_ptr(h), _ptr(W), M, D, V, K, _ptr(tv), _ptr(ti), _stream(h.device)),
           "dflash_head_topk_noalloc")
    return tv, ti


def select_path(top_val, top_idx, F_l, F_r, workspace=None, out=None, anchor=None):
    """top_val f32 [B][P][16], top_idx i32 [B][P][16], F_l/F_r f32 [V][r]
    -> (path_rank i32 [B][P], path_tok i32 [B][P], path_score f32 [B]).
    With anchor (i32 [B], the blocks' slot-0 tokens) the anchored selector runs."""
    _need(top_val, torch.float32, "top_val", 3)
    _need(top_idx, torch.int32, "top_idx", 3)
    _need(F_l, torch.float32, "F_l", 2)
    _need(F_r, torch.float32, "F_r", 2)
    B, P, K = top_val.shape
    V, r = F_l.shape
    if tuple(F_r.shape) != (V, r) or tuple(top_idx.shape) != (B, P, K):
        raise DFlashError("shape mismatch in select_path")
    if anchor is not None:
        _need(anchor, torch.int32, "anchor", 1)
        if anchor.numel() != B:
            raise DFlashError("anchor must hold one id per request")
    _same_device("select_path", top_val, top_idx, F_l, F_r, anchor)
    rank, tok, score = _outs(out, [(torch.int32, (B, P), "path_rank"), (torch.int32, (B, P), "path_tok"),
                                   (torch.float32, (B,), "path_score")], top_val.device)
    L = lib()
    if anchor is None:
        fn, name = L.dflash_select_path, "dflash_select_path"
        before = (_ptr(top_val), _ptr(top_idx), _ptr(F_l), _ptr(F_r), B, P, K, V, r, _ptr(rank), _ptr(tok),
                  _ptr(score))
    else:
        fn, name = L.dflash_select_path_anchored, "dflash_select_path_anchored"
        before = (_ptr(top_val), _ptr(top_idx), _ptr(anchor), _ptr(F_l), _ptr(F_r), B, P, K, V, r, _ptr(rank),
                  _ptr(tok), _ptr(score))
    ws, nbytes = _workspace(fn, before, (_stream(top_val.device),), top_val.device, workspace)
    _check(fn(*before, _ptr(ws), ctypes.byref(nbytes), _stream(top_val.device)), name)
    return rank, tok, score


def verify_greedy(logits, draft, workspace=None, out=None):
    """logits f32 [B][T][V], draft i32 [B][T-1] -> (out_tok i32 [B][T], n_emit i32 [B])."""
    _need(logits, torch.float32, "logits", 3)
    _need(draft, torch.int32, "draft", 2)
    B, T, V = logits.shape
    if tuple(draft.shape) != (B, T - 1):
        raise DFlashError("draft must be [B][T-1]")
    _same_device("verify_greedy", logits, draft)
    o, n = _outs(out, [(torch.int32, (B, T), "out_tok"), (torch.int32, (B,), "n_emit")], logits.device)
    L = lib()
    before = (_ptr(logits), _ptr(draft), B, T, V, _ptr(o), _ptr(n))
    ws, nbytes = _workspace(L.dflash_verify_greedy, before, (_stream(logits.device),), logits.device,
                            workspace)
    _check(L.dflash_verify_greedy(*before, _ptr(ws), ctypes.byref(nbytes), _stream(logits.device)),
           "dflash_verify_greedy")
    return o, n


def verify_sample(logits, draft, temperature, seed, request_id, pos0, workspace=None, out=None):
    """Rejection-sampling verification; request_id/pos0 int64 [B] (request ids
    are taken as their uint64 bit pattern)."""
    _need(logits, torch.float32, "logits", 3)
    _need(draft, torch.int32, "draft", 2)
    _need(request_id, torch.int64, "request_id", 1)
    _need(pos0, torch.int64, "pos0", 1)
    B, T, V = logits.shape
    if tuple(draft.shape) != (B, T - 1) or request_id.numel() != B or pos0.numel() != B:
        raise DFlashError("shape mismatch in verify_sample")
    _same_device("verify_sample", logits, draft, request_id, pos0)
    o, n = _outs(out, [(torch.int32, (B, T), "out_tok"), (torch.int32, (B,), "n_emit")], logits.device)
    L = lib()
    before = (_ptr(logits), _ptr(draft), B, T, V, float(temperature), int(seed) & (2**64 - 1),
              _ptr(request_id), _ptr(pos0), _ptr(o), _ptr(n))
    ws, nbytes = _workspace(L.dflash_verify_sample, before, (_stream(logits.device),), logits.device,
                            workspace)
    _check(L.dflash_verify_sample(*before, _ptr(ws), ctypes.byref(nbytes), _stream(logits.device)),
           "dflash_verify_sample")
    return o, n


def select_path_sampled(top_val, top_idx, F_l, F_r, seed, request_id, pos0, anchor=None, workspace=None, out=None):
    """Sampled-path selector: top_val/top_idx/F_l/F_r as for select_path,
    request_id/pos0 int64 [B], optional anchor int32 [B]
    -> (path_rank i32 [B][P], path_tok i32 [B][P], path_q f64 [B][P][16])."""
    _need(top_val, torch.float32, "top_val", 3)
    _need(top_idx, torch.int32, "top_idx", 3)
    _need(F_l, torch.float32, "F_l", 2)
    _need(F_r, torch.float32, "F_r", 2)
    _need(request_id, torch.int64, "request_id", 1)
    _need(pos0, torch.int64, "pos0", 1)
    B, P, K = top_val.shape
    V, r = F_l.shape
    if (tuple(F_r.shape) != (V, r) or tuple(top_idx.shape) != (B, P, K) or request_id.numel() != B
            or pos0.numel() != B):
        raise DFlashError("shape mismatch in select_path_sampled")
    if anchor is not None:
        _need(anchor, torch.int32, "anchor", 1)
        if anchor.numel() != B:
            raise DFlashError("anchor must hold one id per request")
    _same_device("select_path_sampled", top_val, top_idx, F_l, F_r, anchor, request_id, pos0)
    rank, tok, q = _outs(out, [(torch.int32, (B, P), "path_rank"), (torch.int32, (B, P), "path_tok"),
                               (torch.float64, (B, P, K), "path_q")], top_val.device)
    L = lib()
    before = (_ptr(top_val), _ptr(top_idx), None if anchor is None else _ptr(anchor), _ptr(F_l), _ptr(F_r), B, P,
              K, V, r, int(seed) & (2**64 - 1), _ptr(request_id), _ptr(pos0), _ptr(rank), _ptr(tok), _ptr(q))
    ws, nbytes = _workspace(L.dflash_select_path_sampled, before, (_stream(top_val.device),), top_val.device,
                            workspace)
    _check(L.dflash_select_path_sampled(*before, _ptr(ws), ctypes.byref(nbytes), _stream(top_val.device)),
           "dflash_select_path_sampled")
    return rank, tok, q


def verify_sample_q(logits, draft, q_idx, q_prob, temperature, seed, request_id, pos0, workspace=None, out=None):
    """Rejection-sampling verification of drafts drawn from proposals q:
    q_idx int32 [B][T-1][16], q_prob float64 [B][T-1][16]; the other
    arguments as for verify_sample."""
    _need(logits, torch.float32, "logits", 3)
    _need(draft, torch.int32, "draft", 2)
    _need(q_idx, torch.int32, "q_idx", 3)
    _need(q_prob, torch.float64, "q_prob", 3)
    _need(request_id, torch.int64, "request_id", 1)
    _need(pos0, torch.int64, "pos0", 1)
    B, T, V = logits.shape
    if (tuple(draft.shape) != (B, T - 1) or tuple(q_idx.shape) != (B, T - 1, 16)
            or tuple(q_prob.shape) != (B, T - 1, 16) or request_id.numel() != B or pos0.numel() != B):
        raise DFlashError("shape mismatch in verify_sample_q")
    _same_device("verify_sample_q", logits, draft, q_idx, q_prob, request_id, pos0)
    o, n = _outs(out, [(torch.int32, (B, T), "out_tok"), (torch.int32, (B,), "n_emit")], logits.device)
    L = lib()
    before = (_ptr(logits), _ptr(draft), _ptr(q_idx), _ptr(q_prob), B, T, V, float(temperature),
              int(seed) & (2**64 - 1), _ptr(request_id), _ptr(pos0), _ptr(o), _ptr(n))
    ws, nbytes = _workspace(L.dflash_verify_sample_q, before, (_stream(logits.device),), logits.device, workspace)
    _check(L.dflash_verify_sample_q(*before, _ptr(ws), ctypes.byref(nbytes), _stream(logits.device)),
           "dflash_verify_sample_q")
    return o, n


def verify_greedy_fused(h_t, W, draft, workspace=None, out=None):
    """Greedy verification from target hidden states h_t bf16 [B*T][D] and
    the LM head W bf16 [V][D] (argmax in the head GEMM's epilogue; logits are
    never written); draft int32 [B][T-1] -> (out_tok, n_emit)."""
    _need(h_t, torch.bfloat16, "h_t", 2)
    _need(W, torch.bfloat16, "W", 2)
    _need(draft, torch.int32, "draft", 2)
    B, P = draft.shape
    T = P + 1
    M, D = h_t.shape
    V = W.shape[0]
    if M != B * T or W.shape[1] != D:
        raise DFlashError("shape mismatch in verify_greedy_fused")
    _same_device("verify_greedy_fused", h_t, W, draft)
    o, n = _outs(out, [(torch.int32, (B, T), "out_tok"), (torch.int32, (B,), "n_emit")], h_t.device)
    L = lib()
    before = (_ptr(h_t), _ptr(W), _ptr(draft), B, T, D, V, _ptr(o), _ptr(n))
    ws, nbytes = _workspace(L.dflash_verify_greedy_fused, before, (_stream(h_t.device),), h_t.device, workspace)
    _check(L.dflash_verify_greedy_fused(*before, _ptr(ws), ctypes.byref(nbytes), _stream(h_t.device)),
           "dflash_verify_greedy_fused")
    return o, n


def verify_sample_fused(h_t, W, draft, temperature, seed, request_id, pos0, workspace=None, out=None):
    """Rejection-sampling verification from target hidden states h_t bf16
    [B*T][D] through the LM head W bf16 [V][D] (softmax statistics in the head
    GEMM's epilogue; logits are never written); the other arguments as for
    verify_sample."""
    _need(h_t, torch.bfloat16, "h_t", 2)
    _need(W, torch.bfloat16, "W", 2)
    _need(draft, torch.int32, "draft", 2)
    _need(request_id, torch.int64, "request_id", 1)
    _need(pos0, torch.int64, "pos0", 1)
    B, P = draft.shape
    T = P + 1
    M, D = h_t.shape
    V = W.shape[0]
    if M != B * T or W.shape[1] != D or request_id.numel() != B or pos0.numel() != B:
        raise DFlashError("shape mismatch in verify_sample_fused")
    _same_device("verify_sample_fused", h_t, W, draft, request_id, pos0)
    o, n = _outs(out, [(torch.int32, (B, T), "out_tok"), (torch.int32, (B,), "n_emit")], h_t.device)
    L = lib()
    before = (_ptr(h_t), _ptr(W), _ptr(draft), B, T, D, V, float(temperature), int(seed) & (2**64 - 1),
              _ptr(request_id), _ptr(pos0), _ptr(o), _ptr(n))
    ws, nbytes = _workspace(L.dflash_verify_sample_fused, before, (_stream(h_t.device),), h_t.device, workspace)
    _check(L.dflash_verify_sample_fused(*before, _ptr(ws), ctypes.byref(nbytes), _stream(h_t.device)),
           "dflash_verify_sample_fused")
    return o, n


def verify_sample_topkp(logits, draft, temperature, top_k, top_p, seed, request_id, pos0, workspace=None,
                        out=None):
    """Rejection-sampling verification against the top-k, then top-p
    filtered target; arguments as for verify_sample plus top_k (1..64) and
    top_p (0, 1]."""
    _need(logits, torch.float32, "logits", 3)
    _need(draft, torch.int32, "draft", 2)
    _need(request_id, torch.int64, "request_id", 1)
    _need(pos0, torch.int64, "pos0", 1)
    B, T, V = logits.shape
    if tuple(draft.shape) != (B, T - 1) or request_id.numel() != B or pos0.numel() != B:
        raise DFlashError("shape mismatch in verify_sample_topkp")
    _same_device("verify_sample_topkp", logits, draft, request_id, pos0)
    o, n = _outs(out, [(torch.int32, (B, T), "out_tok"), (torch.int32, (B,), "n_emit")], logits.device)
    L = lib()
    before = (_ptr(logits), _ptr(draft), B, T, V, float(temperature), int(top_k), float(top_p),
              int(seed) & (2**64 - 1), _ptr(request_id), _ptr(pos0), _ptr(o), _ptr(n))
    ws, nbytes = _workspace(L.dflash_verify_sample_topkp, before, (_stream(logits.device),), logits.device,
                            workspace)
    _check(L.dflash_verify_sample_topkp(*before, _ptr(ws), ctypes.byref(nbytes), _stream(logits.device)),
           "dflash_verify_sample_topkp")
    return o, n


# --------------------------------------------------------------------------
# Pre-marshalled calls for tight loops: each bind_* checks its tensors once and
# returns a zero-argument callable that makes exactly one C-ABI call on the
# stream that was current when it was bound (bind inside a graph-capture
# context to record into the graph).

def _bound(fn, args, what):
    def call():
        code = fn(*args)
        if code != 0:
            raise DFlashError(f"{what}: {status_string(code)} ({code})")
    return call


def _bind_ws(workspace, device):
    _need(workspace, torch.uint8, "workspace")
    if workspace.device != device:
        raise DFlashError(f"workspace must be on {device}, got {workspace.device}")


def _bind_sample_checks(logits, draft, request_id, pos0, out_tok, n_emit, workspace):
    _need(logits, torch.float32, "logits", 3)
    B, T, V = logits.shape
    _outs((draft, request_id, pos0), [(torch.int32, (B, T - 1), "draft"), (torch.int64, (B,), "request_id"),
                                      (torch.int64, (B,), "pos0")], logits.device)
    _outs((out_tok, n_emit), [(torch.int32, (B, T), "out_tok"), (torch.int32, (B,), "n_emit")], logits.device)
    _bind_ws(workspace, logits.device)


def _bind_fused_checks(h_t, W, draft, out_tok, n_emit, workspace):
    _need(h_t, torch.bfloat16, "h_t", 2)
    _need(W, torch.bfloat16, "W", 2)
    _need(draft, torch.int32, "draft", 2)
    B, P = draft.shape
    if h_t.shape[0] != B * (P + 1) or W.shape[1] != h_t.shape[1]:
        raise DFlashError("shape mismatch in fused verification")
    _same_device("fused verification", h_t, W, draft)
    _outs((out_tok, n_emit), [(torch.int32, (B, P + 1), "out_tok"), (torch.int32, (B,), "n_emit")], h_t.device)
    _bind_ws(workspace, h_t.device)


def bind_conv2tap_proj(x, w_tap, y):
    _need(x, torch.bfloat16, "x")
    _need(w_tap, torch.bfloat16, "w_tap")
    _out(y, torch.bfloat16, x.shape, x.device, "y")
    D, T = x.shape[-1], x.shape[-2]
    if tuple(w_tap.shape) != (2 * D, D):
        raise DFlashError("w_tap must be [2*D][D]")
    _same_device("conv2tap_proj", x, w_tap)
    S = x.numel() // (T * D)
    return _bound(lib().dflash_conv2tap_proj, (_ptr(x), _ptr(w_tap), _ptr(y), S, T, D, _stream(x.device)),
                  "dflash_conv2tap_proj")


def bind_conv2tap(x, taps, y):
    _need(x, torch.bfloat16, "x")
    _need(taps, torch.bfloat16, "taps")
    _out(y, torch.bfloat16, x.shape, x.device, "y")
    D, T = x.shape[-1], x.shape[-2]
    if taps.shape[-1] != 2 * D or taps.numel() != 2 * x.numel():
        raise DFlashError("taps must be [..., T, 2*D] matching x")
    _same_device("conv2tap", x, taps)
    S = x.numel() // (T * D)
    return _bound(lib().dflash_conv2tap, (_ptr(x), _ptr(taps), _ptr(y), S, T, D, _stream(x.device)),
                  "dflash_conv2tap")


def bind_head_topk(h, W, top_val, top_idx, workspace):
    _need(h, torch.bfloat16, "h", 2)
    _need(W, torch.bfloat16, "W", 2)
    M, D = h.shape
    if W.shape[1] != D:
        raise DFlashError("W must be [V][D] with the same D as h")
    _same_device("head_topk", h, W)
    _outs((top_val, top_idx), [(torch.float32, (M, 16), "top_val"), (torch.int32, (M, 16), "top_idx")], h.device)
    _bind_ws(workspace, h.device)
    nbytes = ctypes.c_size_t(workspace.numel())
    return _bound(lib().dflash_head_topk,
                  (_ptr(h), _ptr(W), M, D, W.shape[0], top_val.shape[-1], _ptr(top_val), _ptr(top_idx),
                   _ptr(workspace), ctypes.byref(nbytes), _stream(h.device)), "dflash_head_topk")


def bind_select_path(top_val, top_idx, F_l, F_r, rank, tok, score, workspace, anchor=None):
    _need(top_val, torch.float32, "top_val", 3)
    _need(top_idx, torch.int32, "top_idx", 3)
    _need(F_l, torch.float32, "F_l", 2)
    _need(F_r, torch.float32, "F_r", 2)
    B, P, K = top_val.shape
    V, r = F_l.shape
    if tuple(F_r.shape) != (V, r) or tuple(top_idx.shape) != (B, P, K):
        raise DFlashError("shape mismatch in select_path")
    _same_device("select_path", top_val, top_idx, F_l, F_r, anchor)
    _outs((rank, tok, score), [(torch.int32, (B, P), "path_rank"), (torch.int32, (B, P), "path_tok"),
                               (torch.float32, (B,), "path_score")], top_val.device)
    _bind_ws(workspace, top_val.device)
    nbytes = ctypes.c_size_t(workspace.numel())
    if anchor is None:
        return _bound(lib().dflash_select_path,
                      (_ptr(top_val), _ptr(top_idx), _ptr(F_l), _ptr(F_r), B, P, K, V, r, _ptr(rank), _ptr(tok),
                       _ptr(score), _ptr(workspace), ctypes.byref(nbytes), _stream(top_val.device)),
                      "dflash_select_path")
    _need(anchor, torch.int32, "anchor", 1)
    return _bound(lib().dflash_select_path_anchored,
                  (_ptr(top_val), _ptr(top_idx), _ptr(anchor), _ptr(F_l), _ptr(F_r), B, P, K, V, r, _ptr(rank),
                   _ptr(tok), _ptr(score), _ptr(workspace), ctypes.byref(nbytes), _stream(top_val.device)),
                  "dflash_select_path_anchored")


def bind_verify_greedy(logits, draft, out_tok, n_emit, workspace):
    _need(logits, torch.float32, "logits", 3)
    B, T, V = logits.shape
    _out(draft, torch.int32, (B, T - 1), logits.device, "draft")
    _outs((out_tok, n_emit), [(torch.int32, (B, T), "out_tok"), (torch.int32, (B,), "n_emit")], logits.device)
    _bind_ws(workspace, logits.device)
    nbytes = ctypes.c_size_t(workspace.numel())
    return _bound(lib().dflash_verify_greedy,
                  (_ptr(logits), _ptr(draft), B, T, V, _ptr(out_tok), _ptr(n_emit), _ptr(workspace),
                   ctypes.byref(nbytes), _stream(logits.device)), "dflash_verify_greedy")


def bind_verify_sample(logits, draft, temperature, seed, request_id, pos0, out_tok, n_emit, workspace):
    _bind_sample_checks(logits, draft, request_id, pos0, out_tok, n_emit, workspace)
    B, T, V = logits.shape
    nbytes = ctypes.c_size_t(workspace.numel())
    return _bound(lib().dflash_verify_sample,
                  (_ptr(logits), _ptr(draft), B, T, V, float(temperature), int(seed) & (2**64 - 1),
                   _ptr(request_id), _ptr(pos0), _ptr(out_tok), _ptr(n_emit), _ptr(workspace),
                   ctypes.byref(nbytes), _stream(logits.device)), "dflash_verify_sample")


def bind_verify_sample_topkp(logits, draft, temperature, top_k, top_p, seed, request_id, pos0, out_tok, n_emit,
                             workspace):
    _bind_sample_checks(logits, draft, request_id, pos0, out_tok, n_emit, workspace)
    B, T, V = logits.shape
    nbytes = ctypes.c_size_t(workspace.numel())
    return _bound(lib().dflash_verify_sample_topkp,
                  (_ptr(logits), _ptr(draft), B, T, V, float(temperature), int(top_k), float(top_p),
                   int(seed) & (2**64 - 1), _ptr(request_id), _ptr(pos0), _ptr(out_tok), _ptr(n_emit),
                   _ptr(workspace), ctypes.byref(nbytes), _stream(logits.device)), "dflash_verify_sample_topkp")


def bind_select_path_sampled(top_val, top_idx, F_l, F_r, seed, request_id, pos0, rank, tok, q, workspace,
                             anchor=None):
    _need(top_val, torch.float32, "top_val", 3)
    _need(top_idx, torch.int32, "top_idx", 3)
    _need(F_l, torch.float32, "F_l", 2)
    _need(F_r, torch.float32, "F_r", 2)
    B, P, K = top_val.shape
    V, r = F_l.shape
    if tuple(F_r.shape) != (V, r) or tuple(top_idx.shape) != (B, P, K):
        raise DFlashError("shape mismatch in select_path_sampled")
    _outs((request_id, pos0), [(torch.int64, (B,), "request_id"), (torch.int64, (B,), "pos0")], top_val.device)
    _same_device("select_path_sampled", top_val, top_idx, F_l, F_r, anchor)
    _outs((rank, tok, q), [(torch.int32, (B, P), "path_rank"), (torch.int32, (B, P), "path_tok"),
                           (torch.float64, (B, P, K), "path_q")], top_val.device)
    _bind_ws(workspace, top_val.device)
    nbytes = ctypes.c_size_t(workspace.numel())
    return _bound(lib().dflash_select_path_sampled,
                  (_ptr(top_val), _ptr(top_idx), None if anchor is None else _ptr(anchor), _ptr(F_l), _ptr(F_r), B,
                   P, K, V, r, int(seed) & (2**64 - 1), _ptr(request_id), _ptr(pos0), _ptr(rank), _ptr(tok), _ptr(q),
                   _ptr(workspace), ctypes.byref(nbytes), _stream(top_val.device)), "dflash_select_path_sampled")


def bind_verify_sample_q(logits, draft, q_idx, q_prob, temperature, seed, request_id, pos0, out_tok, n_emit,
                         workspace):
    _bind_sample_checks(logits, draft, request_id, pos0, out_tok, n_emit, workspace)
    B, T, V = logits.shape
    _outs((q_idx, q_prob), [(torch.int32, (B, T - 1, 16), "q_idx"), (torch.float64, (B, T - 1, 16), "q_prob")],
          logits.device)
    nbytes = ctypes.c_size_t(workspace.numel())
    return _bound(lib().dflash_verify_sample_q,
                  (_ptr(logits), _ptr(draft), _ptr(q_idx), _ptr(q_prob), B, T, V, float(temperature),
                   int(seed) & (2**64 - 1), _ptr(request_id), _ptr(pos0), _ptr(out_tok), _ptr(n_emit),
                   _ptr(workspace), ctypes.byref(nbytes), _stream(logits.device)), "dflash_verify_sample_q")


def bind_verify_greedy_fused(h_t, W, draft, out_tok, n_emit, workspace):
    _bind_fused_checks(h_t, W, draft, out_tok, n_emit, workspace)
    B, P = draft.shape
    nbytes = ctypes.c_size_t(workspace.numel())
    return _bound(lib().dflash_verify_greedy_fused,
                  (_ptr(h_t), _ptr(W), _ptr(draft), B, P + 1, h_t.shape[1], W.shape[0], _ptr(out_tok), _ptr(n_emit),
                   _ptr(workspace), ctypes.byref(nbytes), _stream(h_t.device)), "dflash_verify_greedy_fused")


def bind_verify_sample_fused(h_t, W, draft, temperature, seed, request_id, pos0, out_tok, n_emit, workspace):
    _bind_fused_checks(h_t, W, draft, out_tok, n_emit, workspace)
    B, P = draft.shape
    _outs((request_id, pos0), [(torch.int64, (B,), "request_id"), (torch.int64, (B,), "pos0")], h_t.device)
    nbytes = ctypes.c_size_t(workspace.numel())
    return _bound(lib().dflash_verify_sample_fused,
                  (_ptr(h_t), _ptr(W), _ptr(draft), B, P + 1, h_t.shape[1], W.shape[0], float(temperature),
                   int(seed) & (2**64 - 1), _ptr(request_id), _ptr(pos0), _ptr(out_tok), _ptr(n_emit),
                   _ptr(workspace), ctypes.byref(nbytes), _stream(h_t.device)), "dflash_verify_sample_fused")


def workspace_bytes(op, *shape_args):
    """Workspace size of an entry point for the given sizes, without a GPU call:
    op in {"head_topk": (M, D, V), "select_path": (B, P), "select_path_anchored": (B, P),
    "select_path_sampled": (B, P, anchored), "verify_greedy": (B, T, V), "verify_greedy_fused": (B, T, D, V),
    "verify_sample_fused": (B, T, D, V),
    "verify_sample": (B, T, V), "verify_sample_q": (B, T, V), "verify_sample_topkp": (B, T, V, top_k)}."""
    L = lib()
    n = ctypes.c_size_t(0)
    fake = [ctypes.c_void_p((i + 1) << 40) for i in range(12)]
    if op == "head_topk":
        M, D, V = shape_args
        code = L.dflash_head_topk(fake[0], fake[1], M, D, V, 16, fake[2], fake[3], None, ctypes.byref(n), None)
    elif op == "select_path":
        B, P = shape_args
        code = L.dflash_select_path(fake[0], fake[1], fake[2], fake[3], B, P, 16, 1024, 16, fake[4], fake[5],
                                    fake[6], None, ctypes.byref(n), None)
    elif op == "select_path_anchored":
        B, P = shape_args
        code = L.dflash_select_path_anchored(fake[0], fake[1], fake[7], fake[2], fake[3], B, P, 16, 1024, 16,
                                             fake[4], fake[5], fake[6], None, ctypes.byref(n), None)
    elif op == "select_path_sampled":
        B, P, anchored = shape_args
        code = L.dflash_select_path_sampled(fake[0], fake[1], fake[7] if anchored else None, fake[2], fake[3], B,
                                            P, 16, 1024, 16, 0, fake[8], fake[9], fake[4], fake[5], fake[6], None,
                                            ctypes.byref(n), None)
    elif op == "verify_greedy_fused":
        B, T, D, V = shape_args
        code = L.dflash_verify_greedy_fused(fake[0], fake[1], fake[2], B, T, D, V, fake[3], fake[4], None,
                                            ctypes.byref(n), None)
    elif op == "verify_sample_fused":
        B, T, D, V = shape_args
        code = L.dflash_verify_sample_fused(fake[0], fake[1], fake[2], B, T, D, V, 1.0, 0, fake[5], fake[6],
                                            fake[3], fake[4], None, ctypes.byref(n), None)
    elif op == "verify_greedy":
        B, T, V = shape_args
        code = L.dflash_verify_greedy(fake[0], fake[1], B, T, V, fake[2], fake[3], None, ctypes.byref(n), None)
    elif op == "verify_sample":
        B, T, V = shape_args
        code = L.dflash_verify_sample(fake[0], fake[1], B, T, V, 1.0, 0, fake[4], fake[5], fake[2], fake[3],
                                      None, ctypes.byref(n), None)
    elif op == "verify_sample_q":
        B, T, V = shape_args
        code = L.dflash_verify_sample_q(fake[0], fake[1], fake[8], fake[9], B, T, V, 1.0, 0, fake[4], fake[5],
                                        fake[2], fake[3], None, ctypes.byref(n), None)
    elif op == "verify_sample_topkp":
        B, T, V, k = shape_args
        code = L.dflash_verify_sample_topkp(fake[0], fake[1], B, T, V, 1.0, k, 1.0, 0, fake[4], fake[5], fake[2],
                                            fake[3], None, ctypes.byref(n), None)
    else:
        raise ValueError(op)
    _check(code, f"workspace query {op}")
    return max(int(n.value), 16)
