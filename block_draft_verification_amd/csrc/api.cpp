// C ABI of the cycle-tail library: host-side validation, workspace sizing and
// dispatch to the gfx950 kernels.  No HIP call happens before an argument check
// has passed, so every error path can be exercised without a GPU.

#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/dflash.h"

namespace dflash {
int launch_conv2tap(const uint16_t*, const uint16_t*, uint16_t*, int64_t, int, int, hipStream_t);
int launch_conv2tap_proj(const uint16_t*, const uint16_t*, uint16_t*, int64_t, int, int, hipStream_t);
int launch_head_topk(const uint16_t*, const uint16_t*, int64_t, int, int64_t, float*, int32_t*, void*,
                     hipStream_t);
size_t head_workspace_bytes(int64_t M, int64_t V);
size_t head_static_scratch_bytes();
int launch_head_topk_static(const uint16_t*, const uint16_t*, int64_t, int, int64_t, float*, int32_t*,
                            hipStream_t);
int launch_head_weight_bound(const uint16_t*, int64_t, int, float*, hipStream_t);
int launch_head_certify(const uint16_t*, int64_t, int, int64_t, const float*, const float*, const void*, int32_t*,
                        hipStream_t);
int launch_select_path(const float*, const int32_t*, const int32_t*, const float*, const float*, int, int, int64_t,
                       int, int32_t*, int32_t*, float*, void*, hipStream_t);
size_t select_workspace_bytes(int B, int P, bool anchored);
int launch_select_path_sampled(const float*, const int32_t*, const int32_t*, const float*, const float*, int, int,
                               int64_t, int, uint64_t, const uint64_t*, const int64_t*, int32_t*, int32_t*, double*,
                               void*, hipStream_t);
size_t greedy_workspace_bytes(int B, int T, int64_t V);
size_t sample_workspace_bytes(int B, int T, int64_t V);
size_t sample_topkp_workspace_bytes(int B, int T, int64_t V, int top_k);
int launch_verify_greedy(const float*, const int32_t*, int, int, int64_t, int32_t*, int32_t*, void*,
                         hipStream_t);
int launch_greedy_prefix(const int32_t*, const int32_t*, int, int, int32_t*, int32_t*, hipStream_t);
size_t sample_hidden_workspace_bytes(int B, int T, int64_t V);
int launch_verify_sample_hidden(const uint16_t*, const uint16_t*, const int32_t*, int, int, int, int64_t, float,
                                uint64_t, const uint64_t*, const int64_t*, int32_t*, int32_t*, void*, hipStream_t);
int launch_verify_sample(const float*, const int32_t*, const int32_t*, const double*, int, int, int64_t, float,
                         uint64_t, const uint64_t*, const int64_t*, int32_t*, int32_t*, void*, hipStream_t);
int launch_verify_sample_topkp(const float*, const int32_t*, int, int, int64_t, float, int, float, uint64_t,
                               const uint64_t*, const int64_t*, int32_t*, int32_t*, void*, hipStream_t);
}  // namespace dflash

using namespace dflash;

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];

// Current device must be a gfx950 (MI355X / MI350X).  Cached per device.
int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DFLASH_ERR_DEVICE;
    std::call_once(g_dev_once[dev], [dev]() {
        hipDeviceProp_t prop;
        g_dev_ok[dev] = (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                         strncmp(prop.gcnArchName, "gfx950", 6) == 0)
                            ? 1
                            : 0;
    });
    return g_dev_ok[dev] ? DFLASH_OK : DFLASH_ERR_DEVICE;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// [a, a+na) and [b, b+nb) overlap (byte ranges)
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

int workspace_check(void* ws, size_t* ws_bytes, size_t need, bool* query) {
    if (!ws_bytes) return DFLASH_ERR_INVALID;
    if (!ws) {
        *ws_bytes = need;
        *query = true;
        return DFLASH_OK;
    }
    *query = false;
    if (*ws_bytes < need) return DFLASH_ERR_WORKSPACE;
    if (!aligned16(ws)) return DFLASH_ERR_INVALID;
    return DFLASH_OK;
}

}  // namespace

extern "C" {

const char* dflash_status_string(int status) {
    switch (status) {
        case DFLASH_OK: return "ok";
        case DFLASH_ERR_INVALID: return "invalid argument";
        case DFLASH_ERR_UNSUPPORTED: return "unsupported size";
        case DFLASH_ERR_WORKSPACE: return "workspace too small";
        case DFLASH_ERR_LAUNCH: return "kernel launch failed";
        case DFLASH_ERR_DEVICE: return "current device is not gfx950";
        default: return "unknown status";
    }
}

int dflash_version(void) { return (1 << 16) | 0; }

int dflash_conv2tap(const uint16_t* x, const uint16_t* taps, uint16_t* y, int64_t n_seq, int32_t T,
                    int32_t D, void* stream) {
    if (!x || !taps || !y) return DFLASH_ERR_INVALID;
    if (n_seq < 1 || T < 1 || T > 16 || D < 8 || D % 8 != 0) return DFLASH_ERR_INVALID;
    if (n_seq > ((int64_t)1 << 40) / ((int64_t)T * D)) return DFLASH_ERR_INVALID;
    if (!aligned16(x) || !aligned16(taps) || !aligned16(y)) return DFLASH_ERR_INVALID;
    const size_t nx = (size_t)n_seq * T * D * 2;
    if (overlap(y, nx, x, nx) || overlap(y, nx, taps, 2 * nx)) return DFLASH_ERR_INVALID;
    int st = check_device();
    if (st != DFLASH_OK) return st;
    return launch_conv2tap(x, taps, y, n_seq, T, D, (hipStream_t)stream);
}

int dflash_conv2tap_proj(const uint16_t* x, const uint16_t* w_tap, uint16_t* y, int64_t n_seq, int32_t T,
                         int32_t D, void* stream) {
    if (!x || !w_tap || !y) return DFLASH_ERR_INVALID;
    if (n_seq < 1 || T < 1 || T > 16 || D < 64 || D > 65536 || D % 64 != 0) return DFLASH_ERR_INVALID;
    if (n_seq > ((int64_t)1 << 40) / ((int64_t)T * D)) return DFLASH_ERR_INVALID;
    if (!aligned16(x) || !aligned16(w_tap) || !aligned16(y)) return DFLASH_ERR_INVALID;
    const size_t nx = (size_t)n_seq * T * D * 2, nw = (size_t)2 * D * D * 2;
    if (overlap(y, nx, x, nx) || overlap(y, nx, w_tap, nw)) return DFLASH_ERR_INVALID;
    int st = check_device();
    if (st != DFLASH_OK) return st;
    return launch_conv2tap_proj(x, w_tap, y, n_seq, T, D, (hipStream_t)stream);
}

// Argument checks shared by the head entry points (no HIP call).
static int head_checks(const uint16_t* h, const uint16_t* W, int64_t M, int32_t D, int64_t V, int32_t K,
                       float* top_val, int32_t* top_idx) {
    if (!h || !W || !top_val || !top_idx) return DFLASH_ERR_INVALID;
    if (M < 1 || D < 8 || D % 8 != 0 || D > 65536 || V < 1) return DFLASH_ERR_INVALID;
    if (K != 16) return DFLASH_ERR_UNSUPPORTED;
    if (V < K || V >= ((int64_t)1 << 31) || M > ((int64_t)1 << 24)) return DFLASH_ERR_INVALID;
    if (!aligned16(h) || !aligned16(W) || !aligned4(top_val) || !aligned4(top_idx)) return DFLASH_ERR_INVALID;
    const size_t nout = (size_t)M * K * 4;
    if (overlap(top_val, nout, top_idx, nout) || overlap(top_val, nout, h, (size_t)M * D * 2) ||
        overlap(top_idx, nout, h, (size_t)M * D * 2) || overlap(top_val, nout, W, (size_t)V * D * 2) ||
        overlap(top_idx, nout, W, (size_t)V * D * 2))
        return DFLASH_ERR_INVALID;
    return DFLASH_OK;
}

int dflash_head_topk(const uint16_t* h, const uint16_t* W, int64_t M, int32_t D, int64_t V, int32_t K,
                     float* top_val, int32_t* top_idx, void* workspace, size_t* workspace_bytes,
                     void* stream) {
    int st = head_checks(h, W, M, D, V, K, top_val, top_idx);
    if (st != DFLASH_OK) return st;
    bool query = false;
    st = workspace_check(workspace, workspace_bytes, head_workspace_bytes(M, V), &query);
    if (st != DFLASH_OK || query) return st;
    const size_t nws = *workspace_bytes, nout = (size_t)M * K * 4;
    if (overlap(workspace, nws, h, (size_t)M * D * 2) || overlap(workspace, nws, W, (size_t)V * D * 2) ||
        overlap(workspace, nws, top_val, nout) || overlap(workspace, nws, top_idx, nout))
        return DFLASH_ERR_INVALID;
    st = check_device();
    if (st != DFLASH_OK) return st;
    return launch_head_topk(h, W, M, D, V, top_val, top_idx, workspace, (hipStream_t)stream);
}

int dflash_head_topk_noalloc(const uint16_t* h, const uint16_t* W, int64_t M, int32_t D, int64_t V, int32_t K,
                             float* top_val, int32_t* top_idx, void* stream) {
    int st = head_checks(h, W, M, D, V, K, top_val, top_idx);
    if (st != DFLASH_OK) return st;
    if (head_workspace_bytes(M, V) > head_static_scratch_bytes()) return DFLASH_ERR_WORKSPACE;
    st = check_device();
    if (st != DFLASH_OK) return st;
    return launch_head_topk_static(h, W, M, D, V, top_val, top_idx, (hipStream_t)stream);
}

int dflash_head_weight_bound(const uint16_t* W, int64_t V, int32_t D, float* bound, void* stream) {
    if (!W || !bound) return DFLASH_ERR_INVALID;
    if (D < 8 || D % 8 != 0 || D > 65536 || V < 1 || V >= ((int64_t)1 << 31)) return DFLASH_ERR_INVALID;
    if (!aligned16(W) || !aligned4(bound) || overlap(bound, 8, W, (size_t)V * D * 2)) return DFLASH_ERR_INVALID;
    const int st = check_device();
    if (st != DFLASH_OK) return st;
    return launch_head_weight_bound(W, V, D, bound, (hipStream_t)stream);
}

int dflash_head_topk_certify(const uint16_t* h, int64_t M, int32_t D, int64_t V, int32_t K, const float* bound,
                             const float* top_val, const void* workspace, size_t workspace_bytes,
                             int32_t* certified, void* stream) {
    if (!h || !bound || !top_val || !workspace || !certified) return DFLASH_ERR_INVALID;
    if (M < 1 || D < 8 || D % 8 != 0 || D > 65536 || V < 1) return DFLASH_ERR_INVALID;
    if (K != 16) return DFLASH_ERR_UNSUPPORTED;
    if (V < K || V >= ((int64_t)1 << 31) || M > ((int64_t)1 << 24)) return DFLASH_ERR_INVALID;
    if (!aligned16(h) || !aligned4(bound) || !aligned4(top_val) || !aligned16(workspace) || !aligned4(certified))
        return DFLASH_ERR_INVALID;
    if (workspace_bytes < head_workspace_bytes(M, V)) return DFLASH_ERR_WORKSPACE;
    const size_t nc = (size_t)M * 4;
    if (overlap(certified, nc, h, (size_t)M * D * 2) || overlap(certified, nc, top_val, (size_t)M * K * 4) ||
        overlap(certified, nc, workspace, workspace_bytes) || overlap(certified, nc, bound, 8))
        return DFLASH_ERR_INVALID;
    const int st = check_device();
    if (st != DFLASH_OK) return st;
    return launch_head_certify(h, M, D, V, bound, top_val, workspace, certified, (hipStream_t)stream);
}

// Draws of the sampled-path selector (on = false: the max-sum selector).
struct PathDraws {
    bool on;
    uint64_t seed;
    const uint64_t* request_id;
    const int64_t* pos0;
    double* path_q;
};

static int select_common(const float* top_val, const int32_t* top_idx, const int32_t* anchor, bool anchored,
                         const float* feat_l, const float* feat_r, int32_t B, int32_t P, int32_t K, int64_t V,
                         int32_t r, int32_t* path_rank, int32_t* path_tok, float* path_score, const PathDraws& dr,
                         void* workspace, size_t* workspace_bytes, void* stream) {
    if (!top_val || !top_idx || !feat_l || !feat_r || !path_rank || !path_tok) return DFLASH_ERR_INVALID;
    if (dr.on ? (!dr.request_id || !dr.pos0 || !dr.path_q) : !path_score) return DFLASH_ERR_INVALID;
    if (anchored && (!anchor || !aligned4(anchor))) return DFLASH_ERR_INVALID;
    if (B < 1 || P < 1 || P > 15 || V < 1 || r < 4 || r > 256 || r % 4 != 0) return DFLASH_ERR_INVALID;
    if (K != 16) return DFLASH_ERR_UNSUPPORTED;
    if (!aligned4(top_val) || !aligned4(top_idx) || !aligned16(feat_l) || !aligned16(feat_r) ||
        !aligned4(path_rank) || !aligned4(path_tok))
        return DFLASH_ERR_INVALID;
    if (dr.on ? (((uintptr_t)dr.request_id & 7u) || ((uintptr_t)dr.pos0 & 7u) || ((uintptr_t)dr.path_q & 7u))
              : !aligned4(path_score))
        return DFLASH_ERR_INVALID;
    const size_t nbp = (size_t)B * P * 4, nin = (size_t)B * P * K * 4, n8 = (size_t)B * 8;
    const void* outs[3] = {path_rank, path_tok, dr.on ? (const void*)dr.path_q : (const void*)path_score};
    const size_t outn[3] = {nbp, nbp, dr.on ? (size_t)B * P * K * 8 : (size_t)B * 4};
    const void* ins[7] = {top_val, top_idx, feat_l, feat_r, anchor, dr.request_id, dr.pos0};
    const size_t inn[7] = {nin, nin, (size_t)V * r * 4, (size_t)V * r * 4, anchored ? (size_t)B * 4 : 0,
                           dr.on ? n8 : 0, dr.on ? n8 : 0};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 7; ++j)
            if (overlap(outs[i], outn[i], ins[j], inn[j])) return DFLASH_ERR_INVALID;
        for (int j = i + 1; j < 3; ++j)
            if (overlap(outs[i], outn[i], outs[j], outn[j])) return DFLASH_ERR_INVALID;
    }
    bool query = false;
    int st = workspace_check(workspace, workspace_bytes, select_workspace_bytes(B, P, anchored), &query);
    if (st != DFLASH_OK || query) return st;
    const size_t nws = *workspace_bytes;
    for (int j = 0; j < 7; ++j)
        if (overlap(workspace, nws, ins[j], inn[j])) return DFLASH_ERR_INVALID;
    for (int i = 0; i < 3; ++i)
        if (overlap(workspace, nws, outs[i], outn[i])) return DFLASH_ERR_INVALID;
    st = check_device();
    if (st != DFLASH_OK) return st;
    if (dr.on)
        return launch_select_path_sampled(top_val, top_idx, anchored ? anchor : nullptr, feat_l, feat_r, B, P, V, r,
                                          dr.seed, dr.request_id, dr.pos0, path_rank, path_tok, dr.path_q, workspace,
                                          (hipStream_t)stream);
    return launch_select_path(top_val, top_idx, anchored ? anchor : nullptr, feat_l, feat_r, B, P, V, r, path_rank,
                              path_tok, path_score, workspace, (hipStream_t)stream);
}

int dflash_select_path(const float* top_val, const int32_t* top_idx, const float* feat_l,
                       const float* feat_r, int32_t B, int32_t P, int32_t K, int64_t V, int32_t r,
                       int32_t* path_rank, int32_t* path_tok, float* path_score, void* workspace,
                       size_t* workspace_bytes, void* stream) {
    return select_common(top_val, top_idx, nullptr, false, feat_l, feat_r, B, P, K, V, r, path_rank, path_tok,
                         path_score, PathDraws{false, 0, nullptr, nullptr, nullptr}, workspace, workspace_bytes,
                         stream);
}

int dflash_select_path_anchored(const float* top_val, const int32_t* top_idx, const int32_t* anchor,
                                const float* feat_l, const float* feat_r, int32_t B, int32_t P, int32_t K,
                                int64_t V, int32_t r, int32_t* path_rank, int32_t* path_tok, float* path_score,
                                void* workspace, size_t* workspace_bytes, void* stream) {
    return select_common(top_val, top_idx, anchor, true, feat_l, feat_r, B, P, K, V, r, path_rank, path_tok,
                         path_score, PathDraws{false, 0, nullptr, nullptr, nullptr}, workspace, workspace_bytes,
                         stream);
}

int dflash_select_path_sampled(const float* top_val, const int32_t* top_idx, const int32_t* anchor,
                               const float* feat_l, const float* feat_r, int32_t B, int32_t P, int32_t K, int64_t V,
                               int32_t r, uint64_t seed, const uint64_t* request_id, const int64_t* pos0,
                               int32_t* path_rank, int32_t* path_tok, double* path_q, void* workspace,
                               size_t* workspace_bytes, void* stream) {
    return select_common(top_val, top_idx, anchor, anchor != nullptr, feat_l, feat_r, B, P, K, V, r, path_rank,
                         path_tok, nullptr, PathDraws{true, seed, request_id, pos0, path_q}, workspace,
                         workspace_bytes, stream);
}

static int verify_common_checks(const float* logits, const int32_t* draft, int32_t B, int32_t T, int64_t V,
                                int32_t* out_tok, int32_t* n_emit) {
    if (!logits || !draft || !out_tok || !n_emit) return DFLASH_ERR_INVALID;
    if (B < 1 || T < 2 || T > 16 || V < 1 || V >= ((int64_t)1 << 31)) return DFLASH_ERR_INVALID;
    if (!aligned4(logits) || !aligned4(draft) || !aligned4(out_tok) || !aligned4(n_emit))
        return DFLASH_ERR_INVALID;
    const size_t nl = (size_t)B * T * V * 4, nd = (size_t)B * (T - 1) * 4, no = (size_t)B * T * 4,
                 nn = (size_t)B * 4;
    if (overlap(out_tok, no, logits, nl) || overlap(out_tok, no, draft, nd) || overlap(n_emit, nn, logits, nl) ||
        overlap(n_emit, nn, draft, nd) || overlap(out_tok, no, n_emit, nn))
        return DFLASH_ERR_INVALID;
    return DFLASH_OK;
}

int dflash_verify_greedy(const float* logits, const int32_t* draft, int32_t B, int32_t T, int64_t V,
                         int32_t* out_tok, int32_t* n_emit, void* workspace, size_t* workspace_bytes,
                         void* stream) {
    int st = verify_common_checks(logits, draft, B, T, V, out_tok, n_emit);
    if (st != DFLASH_OK) return st;
    bool query = false;
    st = workspace_check(workspace, workspace_bytes, greedy_workspace_bytes(B, T, V), &query);
    if (st != DFLASH_OK || query) return st;
    const size_t nws = *workspace_bytes;
    if (overlap(workspace, nws, logits, (size_t)B * T * V * 4) ||
        overlap(workspace, nws, draft, (size_t)B * (T - 1) * 4) ||
        overlap(workspace, nws, out_tok, (size_t)B * T * 4) || overlap(workspace, nws, n_emit, (size_t)B * 4))
        return DFLASH_ERR_INVALID;
    st = check_device();
    if (st != DFLASH_OK) return st;
    return launch_verify_greedy(logits, draft, B, T, V, out_tok, n_emit, workspace, (hipStream_t)stream);
}

// Workspace of the fused greedy verifier: the head's, then the target's
// top-16 values and ids [B*T][16] (256-byte aligned offsets).
static size_t fused_head_bytes(int64_t M, int64_t V) { return (head_workspace_bytes(M, V) + 255) / 256 * 256; }
static size_t fused_greedy_workspace_bytes(int64_t M, int64_t V) {
    return fused_head_bytes(M, V) + (size_t)M * 16 * 8;
}

int dflash_verify_greedy_fused(const uint16_t* h_t, const uint16_t* W, const int32_t* draft, int32_t B, int32_t T,
                               int32_t D, int64_t V, int32_t* out_tok, int32_t* n_emit, void* workspace,
                               size_t* workspace_bytes, void* stream) {
    if (!h_t || !W || !draft || !out_tok || !n_emit) return DFLASH_ERR_INVALID;
    if (B < 1 || T < 2 || T > 16 || D < 8 || D > 65536 || D % 8 != 0 || V < 16 || V >= ((int64_t)1 << 31))
        return DFLASH_ERR_INVALID;
    if (!aligned16(h_t) || !aligned16(W) || !aligned4(draft) || !aligned4(out_tok) || !aligned4(n_emit))
        return DFLASH_ERR_INVALID;
    const int64_t M = (int64_t)B * T;
    const size_t nh = (size_t)M * D * 2, nw = (size_t)V * D * 2, nd = (size_t)B * (T - 1) * 4,
                 no = (size_t)B * T * 4, nn = (size_t)B * 4;
    const void* ins[3] = {h_t, W, draft};
    const size_t inn[3] = {nh, nw, nd};
    for (int j = 0; j < 3; ++j)
        if (overlap(out_tok, no, ins[j], inn[j]) || overlap(n_emit, nn, ins[j], inn[j])) return DFLASH_ERR_INVALID;
    if (overlap(out_tok, no, n_emit, nn)) return DFLASH_ERR_INVALID;
    bool query = false;
    int st = workspace_check(workspace, workspace_bytes, fused_greedy_workspace_bytes(M, V), &query);
    if (st != DFLASH_OK || query) return st;
    const size_t nws = *workspace_bytes;
    for (int j = 0; j < 3; ++j)
        if (overlap(workspace, nws, ins[j], inn[j])) return DFLASH_ERR_INVALID;
    if (overlap(workspace, nws, out_tok, no) || overlap(workspace, nws, n_emit, nn)) return DFLASH_ERR_INVALID;
    st = check_device();
    if (st != DFLASH_OK) return st;
    unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
    float* tv = reinterpret_cast<float*>(ws + fused_head_bytes(M, V));
    int32_t* ti = reinterpret_cast<int32_t*>(tv + (size_t)M * 16);
    st = launch_head_topk(h_t, W, M, D, V, tv, ti, ws, (hipStream_t)stream);
    if (st != DFLASH_OK) return st;
    return launch_greedy_prefix(ti, draft, B, T, out_tok, n_emit, (hipStream_t)stream);
}

int dflash_verify_sample_fused(const uint16_t* h_t, const uint16_t* W, const int32_t* draft, int32_t B, int32_t T,
                               int32_t D, int64_t V, float temperature, uint64_t seed, const uint64_t* request_id,
                               const int64_t* pos0, int32_t* out_tok, int32_t* n_emit, void* workspace,
                               size_t* workspace_bytes, void* stream) {
    if (!h_t || !W || !draft || !out_tok || !n_emit || !request_id || !pos0) return DFLASH_ERR_INVALID;
    if (B < 1 || T < 2 || T > 16 || D < 8 || D > 65536 || D % 8 != 0 || V < 16 || V >= ((int64_t)1 << 31))
        return DFLASH_ERR_INVALID;
    if (!(temperature > 0.0f) || !isfinite(temperature)) return DFLASH_ERR_INVALID;
    if (!aligned16(h_t) || !aligned16(W) || !aligned4(draft) || !aligned4(out_tok) || !aligned4(n_emit) ||
        ((uintptr_t)request_id & 7u) || ((uintptr_t)pos0 & 7u))
        return DFLASH_ERR_INVALID;
    const int64_t M = (int64_t)B * T;
    const size_t no = (size_t)B * T * 4, nn = (size_t)B * 4, n8 = (size_t)B * 8;
    const void* ins[5] = {h_t, W, draft, request_id, pos0};
    const size_t inn[5] = {(size_t)M * D * 2, (size_t)V * D * 2, (size_t)B * (T - 1) * 4, n8, n8};
    for (int j = 0; j < 5; ++j)
        if (overlap(out_tok, no, ins[j], inn[j]) || overlap(n_emit, nn, ins[j], inn[j])) return DFLASH_ERR_INVALID;
    if (overlap(out_tok, no, n_emit, nn)) return DFLASH_ERR_INVALID;
    bool query = false;
    int st = workspace_check(workspace, workspace_bytes, sample_hidden_workspace_bytes(B, T, V), &query);
    if (st != DFLASH_OK || query) return st;
    const size_t nws = *workspace_bytes;
    for (int j = 0; j < 5; ++j)
        if (overlap(workspace, nws, ins[j], inn[j])) return DFLASH_ERR_INVALID;
    if (overlap(workspace, nws, out_tok, no) || overlap(workspace, nws, n_emit, nn)) return DFLASH_ERR_INVALID;
    st = check_device();
    if (st != DFLASH_OK) return st;
    return launch_verify_sample_hidden(h_t, W, draft, B, T, D, V, temperature, seed, request_id, pos0, out_tok,
                                       n_emit, workspace, (hipStream_t)stream);
}

static int sample_common(const float* logits, const int32_t* draft, const int32_t* q_idx, const double* q_prob,
                         bool with_q, int32_t B, int32_t T, int64_t V, float temperature, uint64_t seed,
                         const uint64_t* request_id, const int64_t* pos0, int32_t* out_tok, int32_t* n_emit,
                         void* workspace, size_t* workspace_bytes, void* stream) {
    int st = verify_common_checks(logits, draft, B, T, V, out_tok, n_emit);
    if (st != DFLASH_OK) return st;
    if (!request_id || !pos0 || !(temperature > 0.0f) || !isfinite(temperature)) return DFLASH_ERR_INVALID;
    if (((uintptr_t)request_id & 7u) || ((uintptr_t)pos0 & 7u)) return DFLASH_ERR_INVALID;
    if (with_q && (!q_idx || !q_prob || !aligned4(q_idx) || ((uintptr_t)q_prob & 7u))) return DFLASH_ERR_INVALID;
    const size_t no = (size_t)B * T * 4, nn = (size_t)B * 4, n8 = (size_t)B * 8;
    const size_t nqi = with_q ? (size_t)B * (T - 1) * 16 * 4 : 0, nqp = with_q ? (size_t)B * (T - 1) * 16 * 8 : 0;
    if (overlap(out_tok, no, request_id, n8) || overlap(out_tok, no, pos0, n8) ||
        overlap(n_emit, nn, request_id, n8) || overlap(n_emit, nn, pos0, n8) || overlap(out_tok, no, q_idx, nqi) ||
        overlap(out_tok, no, q_prob, nqp) || overlap(n_emit, nn, q_idx, nqi) || overlap(n_emit, nn, q_prob, nqp))
        return DFLASH_ERR_INVALID;
    bool query = false;
    st = workspace_check(workspace, workspace_bytes, sample_workspace_bytes(B, T, V), &query);
    if (st != DFLASH_OK || query) return st;
    const size_t nws = *workspace_bytes;
    if (overlap(workspace, nws, logits, (size_t)B * T * V * 4) ||
        overlap(workspace, nws, draft, (size_t)B * (T - 1) * 4) || overlap(workspace, nws, out_tok, no) ||
        overlap(workspace, nws, n_emit, nn) || overlap(workspace, nws, request_id, n8) ||
        overlap(workspace, nws, pos0, n8) || overlap(workspace, nws, q_idx, nqi) ||
        overlap(workspace, nws, q_prob, nqp))
        return DFLASH_ERR_INVALID;
    st = check_device();
    if (st != DFLASH_OK) return st;
    return launch_verify_sample(logits, draft, with_q ? q_idx : nullptr, with_q ? q_prob : nullptr, B, T, V,
                                temperature, seed, request_id, pos0, out_tok, n_emit, workspace, (hipStream_t)stream);
}

int dflash_verify_sample(const float* logits, const int32_t* draft, int32_t B, int32_t T, int64_t V,
                         float temperature, uint64_t seed, const uint64_t* request_id, const int64_t* pos0,
                         int32_t* out_tok, int32_t* n_emit, void* workspace, size_t* workspace_bytes,
                         void* stream) {
    return sample_common(logits, draft, nullptr, nullptr, false, B, T, V, temperature, seed, request_id, pos0,
                         out_tok, n_emit, workspace, workspace_bytes, stream);
}

int dflash_verify_sample_q(const float* logits, const int32_t* draft, const int32_t* q_idx, const double* q_prob,
                           int32_t B, int32_t T, int64_t V, float temperature, uint64_t seed,
                           const uint64_t* request_id, const int64_t* pos0, int32_t* out_tok, int32_t* n_emit,
                           void* workspace, size_t* workspace_bytes, void* stream) {
    return sample_common(logits, draft, q_idx, q_prob, true, B, T, V, temperature, seed, request_id, pos0, out_tok,
                         n_emit, workspace, workspace_bytes, stream);
}

int dflash_verify_sample_topkp(const float* logits, const int32_t* draft, int32_t B, int32_t T, int64_t V,
                               float temperature, int32_t top_k, float top_p, uint64_t seed,
                               const uint64_t* request_id, const int64_t* pos0, int32_t* out_tok,
                               int32_t* n_emit, void* workspace, size_t* workspace_bytes, void* stream) {
    int st = verify_common_checks(logits, draft, B, T, V, out_tok, n_emit);
    if (st != DFLASH_OK) return st;
    if (!request_id || !pos0 || !(temperature > 0.0f) || !isfinite(temperature)) return DFLASH_ERR_INVALID;
    if (top_k < 1 || top_k > 64 || !(top_p > 0.0f) || !(top_p <= 1.0f)) return DFLASH_ERR_INVALID;
    if (((uintptr_t)request_id & 7u) || ((uintptr_t)pos0 & 7u)) return DFLASH_ERR_INVALID;
    const size_t no = (size_t)B * T * 4, nn = (size_t)B * 4, n8 = (size_t)B * 8;
    if (overlap(out_tok, no, request_id, n8) || overlap(out_tok, no, pos0, n8) ||
        overlap(n_emit, nn, request_id, n8) || overlap(n_emit, nn, pos0, n8))
        return DFLASH_ERR_INVALID;
    bool query = false;
    st = workspace_check(workspace, workspace_bytes, sample_topkp_workspace_bytes(B, T, V, top_k), &query);
    if (st != DFLASH_OK || query) return st;
    const size_t nws = *workspace_bytes;
    if (overlap(workspace, nws, logits, (size_t)B * T * V * 4) ||
        overlap(workspace, nws, draft, (size_t)B * (T - 1) * 4) || overlap(workspace, nws, out_tok, no) ||
        overlap(workspace, nws, n_emit, nn) || overlap(workspace, nws, request_id, n8) ||
        overlap(workspace, nws, pos0, n8))
        return DFLASH_ERR_INVALID;
    st = check_device();
    if (st != DFLASH_OK) return st;
    return launch_verify_sample_topkp(logits, draft, B, T, V, temperature, top_k, top_p, seed, request_id, pos0,
                                      out_tok, n_emit, workspace, (hipStream_t)stream);
}

}  // extern "C"
