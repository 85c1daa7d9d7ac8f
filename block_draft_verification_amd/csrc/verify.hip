// Greedy and rejection-sampling verification of a drafted block (gfx950).
//
// Source: tamsi.dev "DFlash 2 - 3x plus de tokens...", section "Les chiffres
// qui comptent..." (greedy output equals the target's; rejection sampling
// keeps the target distribution); latenode.com "DFlash 2: un drafter de
// 3.43x...", FAQ (same guarantee) and section "El desacuerdo empieza..."
// (acceptance length = tokens completed per verify step).
//
// Both verifiers stream the B*T target rows once, split along the vocabulary
// into 4096-float chunks (one 256-thread workgroup each, 16 floats per thread,
// 16-byte loads when rows are 16-byte aligned), and write one small record per
// (row, chunk).  A second kernel, one workgroup per request, takes the
// per-slot decisions from those records; the sampler re-reads at most the
// logits of the chunks it inverts the CDF in, plus one logit per slot.
//
// Sampling arithmetic is float64 throughout (weights, sums, decisions) so the
// decisions agree with an exact evaluation except within ~1e-15 of a boundary.

#include "common.hpp"
#include "exp64.hpp"
#include "keysort.hpp"
#include "philox.hpp"

namespace dflash {


constexpr int kChunk = 4096;
constexpr int kVerifyThreads = 256;
constexpr int kPerThread = kChunk / kVerifyThreads;  // 16

struct ChunkStat {  // one per (row, chunk) for the sampler
    double mass;    // sum over the chunk of exp((l - m_chunk) * inv_tau)
    float m;        // chunk maximum
    int pad;
};

// ----------------------------------------------------------------- reductions
__device__ __forceinline__ void argmax_combine(float& v, int& i, float v2, int i2) {
    if (ranks_before(v2, i2, v, i)) {
        v = v2;
        i = i2;
    }
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float v2 = __shfl_xor(v, off);
        const int i2 = __shfl_xor(i, off);
        argmax_combine(v, i, v2, i2);
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = min(v, __shfl_xor(v, off));
    return v;
}

// Block (256 threads) reductions; `scratch` must hold 4 entries; every thread
// gets the result.
__device__ float block_max(float v, float* scratch) {
    v = wave_max(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) scratch[w] = v;
    __syncthreads();
    return fmaxf(fmaxf(scratch[0], scratch[1]), fmaxf(scratch[2], scratch[3]));
}

__device__ double block_sum(double v, double* scratch) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) scratch[w] = v;
    __syncthreads();
    return (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
}

__device__ int block_min_int(int v, int* scratch) {
    v = wave_min_int(v);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    __syncthreads();
    if (l == 0) scratch[w] = v;
    __syncthreads();
    return min(min(scratch[0], scratch[1]), min(scratch[2], scratch[3]));
}

// Exclusive prefix sum over the block in thread order; returns the prefix and
// writes the block total.
__device__ double block_exclusive_scan(double v, double* scratch, double& total) {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    double incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double up = __shfl_up(incl, off);
        if (l >= off) incl += up;
    }
    __syncthreads();
    if (l == 63) scratch[w] = incl;
    __syncthreads();
    double before = 0.0;
    for (int k = 0; k < w; ++k) before += scratch[k];
    total = ((scratch[0] + scratch[1]) + scratch[2]) + scratch[3];
    return before + incl - v;
}

// ------------------------------------------------------- streaming loaders
// Loads this thread's (up to) 16 logits of chunk `chunk` of a row.  With VEC
// the row start is 16-byte aligned and V % 4 == 0: thread t reads float4s at
// element offsets 4*(t + 256*i), i = 0..3 (coalesced).  Missing elements get
// -inf and index INT_MAX.
template <bool VEC>
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int64_t V, int chunk,
                                           float (&v)[kPerThread], int (&idx)[kPerThread]) {
    const int64_t c0 = (int64_t)chunk * kChunk;
    if (VEC) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t e = c0 + 4 * ((int64_t)threadIdx.x + kVerifyThreads * i);
            if (e < V) {
                const floatx4 q = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(row + e));
                v[4 * i + 0] = q.x;
                v[4 * i + 1] = q.y;
                v[4 * i + 2] = q.z;
                v[4 * i + 3] = q.w;
#pragma unroll
                for (int j = 0; j < 4; ++j) idx[4 * i + j] = (int)(e + j);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[4 * i + j] = -INFINITY;
                    idx[4 * i + j] = 0x7FFFFFFF;
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
            const int64_t e = c0 + threadIdx.x + (int64_t)kVerifyThreads * i;
            if (e < V) {
                v[i] = __builtin_nontemporal_load(row + e);
                idx[i] = (int)e;
            } else {
                v[i] = -INFINITY;
                idx[i] = 0x7FFFFFFF;
            }
        }
    }
}

// ================================================================== greedy
template <bool VEC>
__global__ __launch_bounds__(kVerifyThreads) void greedy_partial_kernel(
    const float* __restrict__ logits, int64_t V, int n_chunks, float2* __restrict__ part) {
    __shared__ float sv[4];
    __shared__ int si[4];
    const int64_t row = blockIdx.y;
    const int chunk = blockIdx.x;
    float v[kPerThread];
    int idx[kPerThread];
    load_chunk<VEC>(logits + row * V, V, chunk, v, idx);
    float bv = v[0];
    int bi = idx[0];
#pragma unroll
    for (int i = 1; i < kPerThread; ++i) argmax_combine(bv, bi, v[i], idx[i]);
    wave_argmax(bv, bi);
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    if (l == 0) {
        sv[w] = bv;
        si[w] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int k = 1; k < 4; ++k) argmax_combine(bv, bi, sv[k], si[k]);
        part[row * n_chunks + chunk] = make_float2(bv, __int_as_float(bi));
    }
}

// One workgroup per request, one wavefront per row (T wavefronts): reduce the
// row's chunk records to g[t]; then one lane applies the longest-prefix rule.
__global__ __launch_bounds__(1024) void greedy_decide_kernel(const float2* __restrict__ part,
                                                             const int32_t* __restrict__ draft,
                                                             int T, int n_chunks,
                                                             int32_t* __restrict__ out_tok,
                                                             int32_t* __restrict__ n_emit) {
    __shared__ int g[16];
    __shared__ int d[16];
    const int b = blockIdx.x;
    const int t = threadIdx.x >> 6;
    const int l = threadIdx.x & 63;
    const int P = T - 1;
    // the drafts are read once, with the chunk records (one round trip)
    if (threadIdx.x < P) d[threadIdx.x] = draft[(int64_t)b * P + threadIdx.x];
    const float2* rp = part + ((int64_t)b * T + t) * n_chunks;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int c = l; c < n_chunks; c += 64) {
        const float2 e = rp[c];
        argmax_combine(bv, bi, e.x, __float_as_int(e.y));
    }
    wave_argmax(bv, bi);
    if (l == 0) g[t] = bi;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t* o = out_tok + (int64_t)b * T;
        int n = 0;
        while (n < P && d[n] == g[n]) {
            o[n] = d[n];
            ++n;
        }
        o[n] = g[n];
        for (int k = n + 1; k < T; ++k) o[k] = -1;
        n_emit[b] = n + 1;
    }
}

// Greedy verification from the target's top-16 lists (the LM head's argmax
// fused into its GEMM epilogue: the lists come from the head kernels, whose
// exact re-scoring makes entry 0 the exact argmax, lowest id on ties).  One
// wavefront per request: g[t] = top_idx[b*T + t][0], then the prefix rule.
__global__ __launch_bounds__(64) void greedy_prefix_kernel(const int32_t* __restrict__ top_idx,
                                                           const int32_t* __restrict__ draft, int T,
                                                           int32_t* __restrict__ out_tok,
                                                           int32_t* __restrict__ n_emit) {
    __shared__ int g[16];
    __shared__ int d[16];
    const int b = blockIdx.x, l = threadIdx.x;
    const int P = T - 1;
    if (l < T) g[l] = top_idx[((int64_t)b * T + l) * kTopK];
    if (l < P) d[l] = draft[(int64_t)b * P + l];
    __syncthreads();
    if (l == 0) {
        int32_t* o = out_tok + (int64_t)b * T;
        int n = 0;
        while (n < P && d[n] == g[n]) {
            o[n] = d[n];
            ++n;
        }
        o[n] = g[n];
        for (int k = n + 1; k < T; ++k) o[k] = -1;
        n_emit[b] = n + 1;
    }
}

int launch_greedy_prefix(const int32_t* top_idx, const int32_t* draft, int B, int T, int32_t* out_tok,
                         int32_t* n_emit, hipStream_t stream) {
    hipLaunchKernelGGL(greedy_prefix_kernel, dim3(B), dim3(64), 0, stream, top_idx, draft, T, out_tok, n_emit);
    return launch_status();
}

// ================================================================ sampling
template <bool VEC>
__global__ __launch_bounds__(kVerifyThreads) void sample_stats_kernel(
    const float* __restrict__ logits, int64_t V, int n_chunks, double inv_tau,
    ChunkStat* __restrict__ stats) {
    __shared__ float smax[4];
    __shared__ double ssum[4];
    const int64_t row = blockIdx.y;
    const int chunk = blockIdx.x;
    float v[kPerThread];
    int idx[kPerThread];
    load_chunk<VEC>(logits + row * V, V, chunk, v, idx);
    float m = v[0];
#pragma unroll
    for (int i = 1; i < kPerThread; ++i) m = fmaxf(m, v[i]);
    m = block_max(m, smax);
    const double md = (double)m;
    // branch-free: an entry past the row end holds -inf and weighs exp64(-inf)
    // = 0 (so does -inf - -inf, NaN, in a chunk of -inf logits), so all 16
    // exponentials are scheduled together and share their constants
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) s += exp64(((double)v[i] - md) * inv_tau);
    s = block_sum(s, ssum);
    if (threadIdx.x == 0) {
        ChunkStat cs;
        cs.mass = s;
        cs.m = m;
        cs.pad = 0;
        stats[row * n_chunks + chunk] = cs;
    }
}

// Residual weights of the draft's proposal support: token id[k] weighs w[k]
// instead of exp((l - m) * inv_tau) (ids outside the row never match).  A
// one-hot proposal at d is the single entry (d, 0).
struct Residual {
    int n;
    const int* id;     // LDS
    const double* w;   // LDS
    __device__ __forceinline__ double weight(int64_t v, double x) const {
        for (int k = 0; k < n; ++k)
            if ((int64_t)id[k] == v) x = w[k];
        return x;
    }
    // bit j set: token e0 + j has an entry (j < 16)
    __device__ __forceinline__ uint32_t mask16(int64_t e0) const {
        uint32_t m = 0;
        for (int k = 0; k < n; ++k) {
            const int64_t d = (int64_t)id[k] - e0;
            if (id[k] >= 0 && d >= 0 && d < 16) m |= 1u << d;
        }
        return m;
    }
};

// Inverse CDF over a row, starting at chunk `c_start` whose preceding mass is
// `before`: returns the smallest v >= c_start*kChunk with before + sum of
// weights up to v > target, or -1 if the row ends first.  Weights are
// exp((l - m) * inv_tau), replaced by the residual weights of the support.
__device__ int inverse_cdf_from(const float* __restrict__ row, int64_t V, int n_chunks,
                                int c_start, double before, double target, double m,
                                double inv_tau, const Residual& res, double* dscr, int* iscr) {
    for (int c = c_start; c < n_chunks; ++c) {
        const int64_t e0 = (int64_t)c * kChunk + (int64_t)threadIdx.x * kPerThread;
        const uint32_t mask = res.mask16(e0);
        double w[kPerThread];
        double own = 0.0;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int64_t e = e0 + j;
            double x = 0.0;
            if (e < V) {
                x = exp64(((double)row[e] - m) * inv_tau);
                if ((mask >> j) & 1u) x = res.weight(e, x);
            }
            w[j] = x;
            own += x;
        }
        double total;
        const double excl = block_exclusive_scan(own, dscr, total);
        int found = 0x7FFFFFFF;
        double run = before + excl;
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            run += w[j];
            if (found == 0x7FFFFFFF && w[j] > 0.0 && run > target) found = (int)(e0 + j);
        }
        found = block_min_int(found, iscr);
        if (found != 0x7FFFFFFF) return found;
        before += total;
    }
    return -1;
}

// Largest v with non-zero weight: the inverse-CDF fallback when rounding
// leaves the target beyond the accumulated mass.
__device__ int last_positive(const float* __restrict__ row, int64_t V, double m, double inv_tau,
                             const Residual& res, int* iscr) {
    for (int64_t c0 = ((V - 1) / kChunk) * kChunk; c0 >= 0; c0 -= kChunk) {
        int best = -1;
        for (int j = 0; j < kPerThread; ++j) {
            const int64_t e = c0 + (int64_t)threadIdx.x * kPerThread + j;
            if (e < V && res.weight(e, exp64(((double)row[e] - m) * inv_tau)) > 0.0) best = (int)e;
        }
        best = -block_min_int(-best, iscr);
        if (best >= 0) return best;
    }
    return 0;
}

// One workgroup per request decides the slots in order.  QGEN = false: the
// draft is deterministic (q = one-hot(d)): accept iff u_acc * Z < e(d), the
// residual is p without d.  QGEN = true: the draft of slot s was drawn from
// the proposal q given by q_idx / q_prob [B][P][16] (ids, probabilities;
// repeated ids add up, ids outside the vocabulary weigh nothing): accept iff
// u_acc * q(d) * Z < e(d), the residual weight of a support token v is
// max(0, e(v) - q(v) * Z).  With q one-hot at d both give the same numbers.
template <bool QGEN>
__global__ __launch_bounds__(kVerifyThreads) void sample_decide_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ draft, const int32_t* __restrict__ q_idx,
    const double* __restrict__ q_prob, const ChunkStat* __restrict__ stats, int T, int64_t V, int n_chunks,
    double inv_tau, uint64_t seed, const uint64_t* __restrict__ request_id, const int64_t* __restrict__ pos0,
    int32_t* __restrict__ out_tok, int32_t* __restrict__ n_emit) {
    __shared__ double dscr[4];
    __shared__ float fscr[4];
    __shared__ int iscr[4];
    __shared__ double cum[kVerifyThreads];
    __shared__ double u_sh[2];
    __shared__ int res_id[kTopK];      // the support's tokens (-1: no entry)
    __shared__ double res_e[kTopK];    // their weights e(v)
    __shared__ double res_w[kTopK];    // their residual weights
    __shared__ int raw_id[kTopK];
    __shared__ double raw_q[kTopK];
    __shared__ double s_qd;
    const int b = blockIdx.x;
    const int P = T - 1;
    const uint64_t rid = request_id[b];
    const int64_t p0 = pos0[b];
    int32_t* o = out_tok + (int64_t)b * T;
    int n = 0;
    int emitted = -1;
    for (int s = 1; s <= T && emitted < 0; ++s) {
        const int t = (s <= P) ? s - 1 : T - 1;
        const int64_t rowid = (int64_t)b * T + t;
        const float* row = logits + rowid * V;
        const ChunkStat* st = stats + rowid * n_chunks;
        // row maximum and normaliser from the chunk records
        float mf = -INFINITY;
        for (int c = threadIdx.x; c < n_chunks; c += kVerifyThreads) mf = fmaxf(mf, st[c].m);
        mf = block_max(mf, fscr);
        const double m = (double)mf;
        double zpart = 0.0;
        for (int c = threadIdx.x; c < n_chunks; c += kVerifyThreads)
            zpart += st[c].mass * exp64(((double)st[c].m - m) * inv_tau);
        const double Z = block_sum(zpart, dscr);
        if (threadIdx.x == 0) {
            const Philox4 r = philox4x64_10(1ull, rid, (uint64_t)(p0 + s), 0ull, seed, 0ull);
            u_sh[0] = (double)(r.w[0] >> 11) * 0x1p-53;
            u_sh[1] = (double)(r.w[1] >> 11) * 0x1p-53;
        }
        int n_res = 0;  // entries of the residual table
        double target;
        if (s <= P) {
            const int d = draft[(int64_t)b * P + (s - 1)];
            const bool d_ok = d >= 0 && (int64_t)d < V;  // an id outside the vocabulary has p = 0
            const double ed = d_ok ? exp64(((double)row[d] - m) * inv_tau) : 0.0;
            if (!QGEN) {
                if (threadIdx.x == 0) {
                    res_id[0] = d_ok ? d : -1;
                    res_e[0] = ed;
                    res_w[0] = 0.0;
                    s_qd = 1.0;
                }
                n_res = 1;
            } else {
                const int64_t qo = ((int64_t)b * P + (s - 1)) * kTopK;
                if (threadIdx.x < kTopK) {
                    raw_id[threadIdx.x] = q_idx[qo + threadIdx.x];
                    raw_q[threadIdx.x] = q_prob[qo + threadIdx.x];
                }
                if (threadIdx.x == 0) s_qd = 0.0;
                __syncthreads();
                if (threadIdx.x < kTopK) {
                    const int k = threadIdx.x, v = raw_id[k];
                    const bool ok = v >= 0 && (int64_t)v < V;
                    bool first = ok;
                    double qsum = 0.0;
                    for (int k2 = 0; k2 < kTopK; ++k2) {
                        if (raw_id[k2] == v) {
                            qsum += raw_q[k2];
                            if (k2 < k) first = false;
                        }
                    }
                    const double ev = first ? exp64(((double)row[v] - m) * inv_tau) : 0.0;
                    res_id[k] = first ? v : -1;
                    res_e[k] = ev;
                    res_w[k] = first ? fmax(0.0, ev - qsum * Z) : 0.0;
                    if (first && v == d) s_qd = qsum;
                }
                n_res = kTopK;
            }
            __syncthreads();
            const double u_acc = u_sh[0];
            if (u_acc * s_qd * Z < ed) {
                if (threadIdx.x == 0) o[n] = d;
                ++n;
                __syncthreads();
                continue;
            }
            double adj = 0.0;
            for (int k = 0; k < n_res; ++k) adj += res_e[k] - res_w[k];
            target = u_sh[1] * (Z - adj);
        } else {
            __syncthreads();
            target = u_sh[1] * Z;
        }
        const Residual res{n_res, res_id, res_w};
        // locate the chunk holding the target from the chunk masses
        double before = 0.0;
        int c_hit = -1;
        for (int c0 = 0; c0 < n_chunks && c_hit < 0; c0 += kVerifyThreads) {
            const int c = c0 + threadIdx.x;
            double mass = 0.0;
            if (c < n_chunks) {
                mass = st[c].mass * exp64(((double)st[c].m - m) * inv_tau);
                for (int k = 0; k < n_res; ++k)
                    if (res_id[k] >= 0 && res_id[k] / kChunk == c) mass -= res_e[k] - res_w[k];
            }
            double total;
            const double excl = block_exclusive_scan(mass, dscr, total);
            const int hit = (c < n_chunks && before + excl + mass > target) ? c : 0x7FFFFFFF;
            const int first = block_min_int(hit, iscr);
            if (first != 0x7FFFFFFF) {
                if (c == first) cum[0] = before + excl;
                __syncthreads();
                before = cum[0];
                c_hit = first;
                __syncthreads();
            } else {
                before += total;
            }
        }
        int tok = -1;
        if (c_hit >= 0) tok = inverse_cdf_from(row, V, n_chunks, c_hit, before, target, m, inv_tau, res, dscr, iscr);
        if (tok < 0) tok = last_positive(row, V, m, inv_tau, res, iscr);
        emitted = tok;
    }
    if (threadIdx.x == 0) {
        o[n] = emitted;
        for (int k = n + 1; k < T; ++k) o[k] = -1;
        n_emit[b] = n + 1;
    }
}

// ============================== sampling fused into the target's LM head
// The target head GEMM (launch_head_stats) leaves, per (row, 16-token tile),
// the tile maximum m_i and s_i = sum of exp((z - m_i) / tau) over the tile,
// from float32 logits.  One workgroup per request then decides the slots in
// order as sample_decide_kernel does, with
//   m = max_i m_i, Z = sum_i s_i exp((m_i - m) / tau)            (float64),
//   e(d) from the draft's logit re-scored exactly (float64 dot product),
// and on a rejection (or for the bonus) locates the tile holding the target
// by a scan over the tile masses, re-scores that tile's 16 logits exactly and
// inverts the CDF inside it (ascending ids, the draft weighted 0).  If
// rounding leaves the target past the tile's exact mass, the tile's last
// token of non-zero weight is taken.
__device__ double exact_logit(const uint16_t* __restrict__ hr, const uint16_t* __restrict__ wr, int D, double* dscr) {
    double acc = 0.0;
    for (int k = threadIdx.x * 8; k < D; k += kVerifyThreads * 8) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(hr + k);
        const u32x4 w = *reinterpret_cast<const u32x4*>(wr + k);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc = fma((double)bf16_to_f32(a[q] & 0xFFFFu), (double)bf16_to_f32(w[q] & 0xFFFFu), acc);
            acc = fma((double)bf16_to_f32(a[q] >> 16), (double)bf16_to_f32(w[q] >> 16), acc);
        }
    }
    return block_sum(acc, dscr);
}

__global__ __launch_bounds__(kVerifyThreads) void sample_hidden_decide_kernel(
    const float2* __restrict__ rec, int64_t n16, const uint16_t* __restrict__ h_t, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ draft, int T, int D, int64_t V, double inv_tau, uint64_t seed,
    const uint64_t* __restrict__ request_id, const int64_t* __restrict__ pos0, int32_t* __restrict__ out_tok,
    int32_t* __restrict__ n_emit) {
    __shared__ double dscr[4];
    __shared__ float fscr[4];
    __shared__ int iscr[4];
    __shared__ double s_before;
    __shared__ double s_u[2];
    __shared__ double s_z[16];
    __shared__ int s_tok;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int P = T - 1;
    const uint64_t rid = request_id[b];
    const int64_t p0 = pos0[b];
    int32_t* o = out_tok + (int64_t)b * T;
    int n = 0;
    int emitted = -1;
    for (int s = 1; s <= T && emitted < 0; ++s) {
        const int t = (s <= P) ? s - 1 : T - 1;
        const int64_t row = (int64_t)b * T + t;
        const float2* rr = rec + row * n16;
        const uint16_t* hr = h_t + row * D;
        // each thread owns a contiguous run of tiles; loads unrolled so that
        // several are in flight
        const int64_t per = (n16 + kVerifyThreads - 1) / kVerifyThreads;
        const int64_t i0 = min<int64_t>((int64_t)tid * per, n16), i1 = min<int64_t>(i0 + per, n16);
        float mf = -INFINITY;
#pragma unroll 8
        for (int64_t i = i0; i < i1; ++i) mf = fmaxf(mf, rr[i].x);
        mf = block_max(mf, fscr);
        const double m = (double)mf;
        double zp = 0.0;  // this run's mass
#pragma unroll 8
        for (int64_t i = i0; i < i1; ++i) zp += (double)rr[i].y * exp64(((double)rr[i].x - m) * inv_tau);
        const double Z = block_sum(zp, dscr);
        if (tid == 0) {
            const Philox4 r = philox4x64_10(1ull, rid, (uint64_t)(p0 + s), 0ull, seed, 0ull);
            s_u[0] = (double)(r.w[0] >> 11) * 0x1p-53;
            s_u[1] = (double)(r.w[1] >> 11) * 0x1p-53;
        }
        __syncthreads();
        int skip = -1;
        double ed = 0.0, target;
        if (s <= P) {
            const int d = draft[(int64_t)b * P + (s - 1)];
            const bool d_ok = d >= 0 && (int64_t)d < V;
            if (d_ok) ed = exp64((exact_logit(hr, W + (int64_t)d * D, D, dscr) - m) * inv_tau);
            if (s_u[0] * Z < ed) {
                if (tid == 0) o[n] = d;
                ++n;
                __syncthreads();
                continue;
            }
            skip = d_ok ? d : -1;
            target = s_u[1] * (Z - ed);
        } else {
            target = s_u[1] * Z;
        }
        // the tile holding the target, from the tile masses (the draft's tile
        // without the draft): each thread sums a contiguous run of tiles, one
        // block scan finds the run holding the target, its thread walks it
        auto tile_mass = [&](int64_t i) -> double {
            double mass = (double)rr[i].y * exp64(((double)rr[i].x - m) * inv_tau);
            if (skip >= 0 && skip / 16 == i) mass = fmax(0.0, mass - ed);
            return mass;
        };
        // the run's mass without the draft: its tile loses min(mass, e(d))
        double run = zp;
        if (skip >= 0 && skip / 16 >= i0 && skip / 16 < i1) {
            const int64_t i = skip / 16;
            const double mass = (double)rr[i].y * exp64(((double)rr[i].x - m) * inv_tau);
            run -= mass - fmax(0.0, mass - ed);
        }
        double total;
        const double excl = block_exclusive_scan(run, dscr, total);
        const int owner = block_min_int(i0 < i1 && excl + run > target ? tid : 0x7FFFFFFF, iscr);
        if (tid == (owner == 0x7FFFFFFF ? kVerifyThreads - 1 : owner)) {
            // rounding can leave the target past the total: the last run then
            int64_t hit_i = i1 > i0 ? i1 - 1 : n16 - 1;
            double c = excl, before_i = excl;
            for (int64_t i = i0; i < i1; ++i) {
                const double w = tile_mass(i);
                if (c + w > target) {
                    hit_i = i;
                    before_i = c;
                    break;
                }
                c += w;
                before_i = c - w;
            }
            s_before = before_i;
            s_tok = (int)hit_i;
        }
        __syncthreads();
        const double before = s_before;
        const int64_t hit = s_tok;
        __syncthreads();
        // the hit tile's 16 logits, exactly: a group of 16 lanes per token
        // (loads unrolled), summed across the group in a fixed order
        {
            const int k = tid >> 4, l = tid & 15;
            const int64_t v = hit * 16 + k;
            double acc = 0.0;
            if (v < V) {
                const uint16_t* wr = W + v * D;
#pragma unroll 8
                for (int kk = l * 8; kk < D; kk += 16 * 8) {
                    const u32x4 a = *reinterpret_cast<const u32x4*>(hr + kk);
                    const u32x4 x = *reinterpret_cast<const u32x4*>(wr + kk);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        acc = fma((double)bf16_to_f32(a[q] & 0xFFFFu), (double)bf16_to_f32(x[q] & 0xFFFFu), acc);
                        acc = fma((double)bf16_to_f32(a[q] >> 16), (double)bf16_to_f32(x[q] >> 16), acc);
                    }
                }
            }
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) acc += __shfl_xor(acc, off, 16);
            if (l == 0) s_z[k] = acc;
        }
        __syncthreads();
        if (tid == 0) {
            int tok = -1, last = -1;
            double c = before;
            for (int k = 0; k < 16; ++k) {
                const int64_t v = hit * 16 + k;
                if (v >= V || (int)v == skip) continue;
                const double wv = exp64((s_z[k] - m) * inv_tau);
                if (wv > 0.0) last = (int)v;
                c += wv;
                if (tok < 0 && wv > 0.0 && c > target) tok = (int)v;
            }
            s_tok = tok >= 0 ? tok : (last >= 0 ? last : (int)(hit * 16));
        }
        __syncthreads();
        emitted = s_tok;
    }
    if (tid == 0) {
        o[n] = emitted;
        for (int k = n + 1; k < T; ++k) o[k] = -1;
        n_emit[b] = n + 1;
    }
}

size_t head_stats_bytes(int64_t M, int64_t V);
int launch_head_stats(const uint16_t*, const uint16_t*, int64_t, int, int64_t, double, float2*, hipStream_t);

size_t sample_hidden_workspace_bytes(int B, int T, int64_t V) { return head_stats_bytes((int64_t)B * T, V); }

int launch_verify_sample_hidden(const uint16_t* h_t, const uint16_t* W, const int32_t* draft, int B, int T, int D,
                                int64_t V, float temperature, uint64_t seed, const uint64_t* request_id,
                                const int64_t* pos0, int32_t* out_tok, int32_t* n_emit, void* ws,
                                hipStream_t stream) {
    const double inv_tau = 1.0 / (double)temperature;
    float2* rec = reinterpret_cast<float2*>(ws);
    int st = launch_head_stats(h_t, W, (int64_t)B * T, D, V, inv_tau, rec, stream);
    if (st != DFLASH_OK) return st;
    hipLaunchKernelGGL(sample_hidden_decide_kernel, dim3(B), dim3(kVerifyThreads), 0, stream, rec, (V + 15) / 16,
                       h_t, W, draft, T, D, V, inv_tau, seed, request_id, pos0, out_tok, n_emit);
    return launch_status();
}

// ================================================ top-k / top-p sampling
// Source: latenode.com "DFlash 2: un drafter de 3.43x...", FAQ (the published
// figures sample at temperature 1.0, top-p 0.95, top-k 20).  The target row is
// filtered before the rejection test: its top_k logits (ties to the lower id),
// weights exp((l - l_max) / tau), then the shortest rank prefix whose mass
// reaches top_p of theirs; the decisions are those of the unfiltered sampler
// on the filtered distribution.
//
// topk_chunk_kernel streams the logits once (the same 4096-entry chunks) and
// writes each chunk's top_k keys (rank_key, descending).  Threshold first:
// each wavefront sorts its 64 lanes' best keys, the top_k-th of them is
// reached by top_k distinct entries, and the largest such bound over the
// wavefronts leaves only a few dozen candidates, which one wavefront sorts.
// topkp_set_kernel (one workgroup per row) merges the row's chunk lists the
// same way, evaluates the nucleus in float64 in rank order and writes the
// kept tokens by ascending id; topkp_decide_kernel (one per request) takes the
// slot decisions from those records.
constexpr int kMaxTopK = 64;
constexpr int kCandCap = kVerifyThreads;  // candidates sorted per chunk or row

// Top 64 of two descending 64-key sequences a (this lane: a[lane]) and b:
// the lane-wise maximum with b reversed is bitonic; half-cleaners sort it.
__device__ __forceinline__ uint64_t merge64_desc(uint64_t a, uint64_t b_rev, int lane) {
    uint64_t k = a > b_rev ? a : b_rev;
    k = cx(k, xor_lane_u64<32>(k, lane), (lane & 32) == 0);
    k = cx(k, xor_lane_u64<16>(k, lane), (lane & 16) == 0);
    k = cx(k, xor_lane_u64<8>(k, lane), (lane & 8) == 0);
    k = cx(k, xor_lane_u64<4>(k, lane), (lane & 4) == 0);
    k = cx(k, xor_lane_u64<2>(k, lane), (lane & 2) == 0);
    k = cx(k, xor_lane_u64<1>(k, lane), (lane & 1) == 0);
    return k;
}


// Appends this lane's keys >= thr (and non-zero) to cand[] at a workgroup
// counter; returns nothing, the count is *count (may exceed kCandCap: then
// only the first kCandCap are stored).
template <int N>
__device__ __forceinline__ void gather_candidates(const uint64_t (&k)[N], uint64_t thr, uint64_t* cand,
                                                  int* count) {
    int mine = 0;
#pragma unroll
    for (int i = 0; i < N; ++i) mine += (k[i] != 0 && k[i] >= thr) ? 1 : 0;
    // wavefront exclusive prefix of the counts, then one reservation per wavefront
    const int lane = threadIdx.x & 63;
    int incl = mine;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    const int total = __shfl(incl, 63);
    int base = 0;
    if (lane == 63 && total > 0) base = atomicAdd(count, total);
    base = __shfl(base, 63) + incl - mine;
#pragma unroll
    for (int i = 0; i < N; ++i)
        if (k[i] != 0 && k[i] >= thr) {
            if (base < kCandCap) cand[base] = k[i];
            ++base;
        }
}

// The best `keep` (<= 64) of n <= kCandCap candidate keys in cand[], sorted
// descending, in lanes 0..keep-1 of wavefront 0 (other lanes: 0).  All
// threads of the workgroup call it; grp[] is LDS scratch of kCandCap keys.
__device__ __forceinline__ uint64_t best_of_candidates(const uint64_t* cand, int n, uint64_t* grp) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t k = (threadIdx.x < n) ? cand[threadIdx.x] : 0ull;
    if (n > 64) {
        k = sort64_desc(k, lane);
        grp[threadIdx.x] = k;
        __syncthreads();
        if (wave == 0) {
            const uint64_t a = merge64_desc(grp[lane], grp[64 + 63 - lane], lane);
            const uint64_t b = merge64_desc(grp[128 + lane], grp[192 + 63 - lane], lane);
            k = merge64_desc(a, __shfl(b, 63 - lane), lane);
        }
        __syncthreads();
    } else if (wave == 0) {
        k = sort64_desc(k, lane);
    }
    return k;
}

template <bool VEC>
__global__ __launch_bounds__(kVerifyThreads) void topk_chunk_kernel(const float* __restrict__ logits, int64_t V,
                                                                    int n_chunks, int top_k,
                                                                    uint64_t* __restrict__ part) {
    __shared__ uint64_t s_thr[4];
    __shared__ uint64_t cand[kCandCap];
    __shared__ uint64_t grp[kCandCap];
    __shared__ int s_count;
    const int64_t row = blockIdx.y;
    const int chunk = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float v[kPerThread];
    int idx[kPerThread];
    load_chunk<VEC>(logits + row * V, V, chunk, v, idx);
    uint64_t k[kPerThread];
    uint64_t mk = 0;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
        k[i] = idx[i] != 0x7FFFFFFF ? rank_key(v[i], idx[i]) : 0ull;
        mk = k[i] > mk ? k[i] : mk;
    }
    if (threadIdx.x == 0) s_count = 0;
    // the wavefront's top_k-th best lane maximum: top_k distinct entries reach it
    const uint64_t sorted = sort64_desc(mk, lane);
    if (lane == 0) s_thr[wave] = readlane_u64(sorted, top_k - 1);
    __syncthreads();
    uint64_t thr = s_thr[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) thr = s_thr[w] > thr ? s_thr[w] : thr;
    gather_candidates(k, thr, cand, &s_count);
    __syncthreads();
    const int n = s_count;
    uint64_t* out = part + ((int64_t)row * n_chunks + chunk) * top_k;
    if (n <= kCandCap) {
        const uint64_t best = best_of_candidates(cand, n, grp);
        if (wave == 0 && lane < top_k) out[lane] = best;
        return;
    }
    // more than kCandCap entries tie at the bound (e.g. constant rows): take
    // the best top_k one at a time
    __shared__ uint64_t s_best[4];
    for (int r = 0; r < top_k; ++r) {
        uint64_t m = 0;
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) m = k[i] > m ? k[i] : m;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint64_t o = shfl_xor_u64(m, off);
            m = o > m ? o : m;
        }
        if (lane == 0) s_best[wave] = m;
        __syncthreads();
        uint64_t b = s_best[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) b = s_best[w] > b ? s_best[w] : b;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPerThread; ++i)
            if (k[i] == b) k[i] = 0;  // keys are unique (distinct ids)
        if (threadIdx.x == 0) out[r] = b;
    }
}

// One target row's filtered set, written as a KeptSet record.
struct KeptSet {
    double z;                // Z': mass of the kept tokens
    int n;                   // kept tokens (1..64)
    int pad;
    int id[kMaxTopK];        // ascending ids
    double w[kMaxTopK];      // their weights exp((l - l_max) / tau)
};

__global__ __launch_bounds__(kVerifyThreads) void topkp_set_kernel(const uint64_t* __restrict__ part, int n_chunks,
                                                                   int top_k, double inv_tau, double top_p,
                                                                   KeptSet* __restrict__ sets) {
    __shared__ uint64_t cand[kCandCap];
    __shared__ uint64_t grp[kCandCap];
    __shared__ int s_count;
    __shared__ uint64_t s_thr;
    __shared__ double s_e[kMaxTopK];
    __shared__ int s_id[kMaxTopK];
    __shared__ int s_kept;
    const int64_t row = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    KeptSet* rec = sets + row;
    {
        const uint64_t* lists = part + row * n_chunks * top_k;
        // bound: the top_k-th best list head (a running top 64 over groups of heads)
        if (wave == 0) {
            uint64_t run = 0;
            for (int g = 0; g < n_chunks; g += 64) {
                uint64_t h = (g + lane < n_chunks) ? lists[(int64_t)(g + lane) * top_k] : 0ull;
                h = sort64_desc(h, lane);
                run = g == 0 ? h : merge64_desc(run, __shfl(h, 63 - lane), lane);
            }
            const uint64_t thr = readlane_u64(run, top_k - 1);
            if (lane == 0) {
                s_thr = thr;
                s_count = 0;
            }
        }
        __syncthreads();
        const uint64_t thr = s_thr;
        // candidates: the entries at or above the bound (a prefix of each list)
        for (int c = threadIdx.x; c < n_chunks; c += kVerifyThreads) {
            for (int j = 0; j < top_k; ++j) {
                const uint64_t key = lists[(int64_t)c * top_k + j];
                if (key == 0 || key < thr) break;
                const int pos = atomicAdd(&s_count, 1);
                if (pos < kCandCap) cand[pos] = key;
            }
        }
        __syncthreads();
        const int n = s_count;
        uint64_t best;
        if (n <= kCandCap) {
            best = best_of_candidates(cand, n, grp);
        } else {
            // ties beyond the buffer: k-way selection of the best top_k heads
            best = 0;
            if (wave == 0) {
                for (int r = 0; r < top_k; ++r) {
                    uint64_t m = 0;
                    for (int c = lane; c < n_chunks; c += 64)
                        for (int j = 0; j < top_k; ++j) {
                            const uint64_t key = lists[(int64_t)c * top_k + j];
                            const bool taken = r > 0 && key >= readlane_u64(best, r - 1);
                            if (!taken && key > m) m = key;
                            if (!taken) break;
                        }
#pragma unroll
                    for (int off = 32; off >= 1; off >>= 1) {
                        const uint64_t o = shfl_xor_u64(m, off);
                        m = o > m ? o : m;
                    }
                    if (lane == r) best = m;
                }
            }
        }
        // weights in rank order, then the nucleus in float64, sequentially
        if (wave == 0) {
            const bool real = lane < top_k && best != 0;
            const double lv = real ? (double)key_value(best) : 0.0;
            const double l0 = (double)key_value(readlane_u64(best, 0));
            s_e[lane] = real ? exp64((lv - l0) * inv_tau) : 0.0;
            s_id[lane] = real ? key_id(best) : 0x7FFFFFFF;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            double zk = 0.0;
            int nk = 0;
            for (int j = 0; j < top_k && s_id[j] != 0x7FFFFFFF; ++j) {
                zk += s_e[j];
                ++nk;
            }
            const double bound = top_p * zk;
            double c = 0.0;
            int kept = 0;
            for (int j = 0; j < nk; ++j) {
                if (kept > 0 && c >= bound) break;
                c += s_e[j];
                ++kept;
            }
            rec->n = kept;
            rec->z = c;
            s_kept = kept;
        }
        __syncthreads();
        // kept tokens by ascending id
        if (wave == 0) {
            const int kept = s_kept;
            uint64_t ik = lane < kept ? (((uint64_t)(0x7FFFFFFF - s_id[lane]) << 32) | (uint32_t)lane) : 0ull;
            ik = sort64_desc(ik, lane);
            if (lane < kept) {
                const int j = (int)(uint32_t)ik;
                rec->id[lane] = s_id[j];
                rec->w[lane] = s_e[j];
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(64) void topkp_decide_kernel(const int32_t* __restrict__ draft,
                                                         const KeptSet* __restrict__ sets, int T, uint64_t seed,
                                                         const uint64_t* __restrict__ request_id,
                                                         const int64_t* __restrict__ pos0,
                                                         int32_t* __restrict__ out_tok, int32_t* __restrict__ n_emit) {
    __shared__ KeptSet s_sets[16];
    __shared__ double s_u[16][2];
    const int b = blockIdx.x;
    // the request's records and every slot's uniforms, fetched and drawn in parallel
    {
        // lane l fetches entry l of every row: all loads in flight together
        const KeptSet* src = sets + (int64_t)b * T;
        const int l = threadIdx.x;
        int id[16];
        double w[16], z[16];
        int n[16];
#pragma unroll
        for (int t = 0; t < 16; ++t)
            if (t < T) {
                id[t] = src[t].id[l];
                w[t] = src[t].w[l];
                z[t] = src[t].z;
                n[t] = src[t].n;
            }
#pragma unroll
        for (int t = 0; t < 16; ++t)
            if (t < T) {
                s_sets[t].id[l] = id[t];
                s_sets[t].w[l] = w[t];
                if (l == 0) {
                    s_sets[t].z = z[t];
                    s_sets[t].n = n[t];
                }
            }
        if (threadIdx.x < T) {
            const int s = threadIdx.x + 1;
            const Philox4 r = philox4x64_10(1ull, request_id[b], (uint64_t)(pos0[b] + s), 0ull, seed, 0ull);
            s_u[threadIdx.x][0] = (double)(r.w[0] >> 11) * 0x1p-53;
            s_u[threadIdx.x][1] = (double)(r.w[1] >> 11) * 0x1p-53;
        }
    }
    __syncthreads();
    // ---- decisions, in slot order (one thread; at most 64 kept tokens a row)
    if (threadIdx.x == 0) {
        const int P = T - 1;
        int32_t* o = out_tok + (int64_t)b * T;
        int n = 0, emitted = -1;
        for (int s = 1; s <= T && emitted < 0; ++s) {
            const int t = (s <= P) ? s - 1 : T - 1;
            const double u_acc = s_u[s - 1][0], u_res = s_u[s - 1][1];
            const KeptSet& ks = s_sets[t];
            const int kept = ks.n;
            const double Z = ks.z;
            int skip = -1;
            double ed = 0.0;
            if (s <= P) {
                const int d = draft[(int64_t)b * P + (s - 1)];
                for (int i = 0; i < kept; ++i)
                    if (ks.id[i] == d) {
                        skip = i;
                        ed = ks.w[i];
                    }
                if (u_acc * Z < ed) {
                    o[n++] = d;
                    continue;
                }
            }
            const double target = u_res * (Z - ed);
            double run = 0.0;
            int last = -1;
            for (int i = 0; i < kept; ++i) {
                const double w = i == skip ? 0.0 : ks.w[i];
                run += w;
                if (w > 0.0) {
                    last = i;
                    if (run > target) {
                        emitted = ks.id[i];
                        break;
                    }
                }
            }
            if (emitted < 0) emitted = last >= 0 ? ks.id[last] : ks.id[0];
        }
        o[n] = emitted;
        for (int k = n + 1; k < T; ++k) o[k] = -1;
        n_emit[b] = n + 1;
    }
}

// ------------------------------------------------------------------- hosts
size_t greedy_workspace_bytes(int B, int T, int64_t V) {
    const int64_t n_chunks = (V + kChunk - 1) / kChunk;
    return (size_t)B * T * n_chunks * sizeof(float2);
}

size_t sample_workspace_bytes(int B, int T, int64_t V) {
    const int64_t n_chunks = (V + kChunk - 1) / kChunk;
    return (size_t)B * T * n_chunks * sizeof(ChunkStat);
}

int launch_verify_greedy(const float* logits, const int32_t* draft, int B, int T, int64_t V,
                         int32_t* out_tok, int32_t* n_emit, void* ws, hipStream_t stream) {
    const int n_chunks = (int)((V + kChunk - 1) / kChunk);
    float2* part = reinterpret_cast<float2*>(ws);
    const dim3 grid(n_chunks, B * T);
    const bool vec = (V % 4 == 0) && ((uintptr_t)logits % 16 == 0);
    if (vec)
        hipLaunchKernelGGL(greedy_partial_kernel<true>, grid, dim3(kVerifyThreads), 0, stream, logits, V, n_chunks, part);
    else
        hipLaunchKernelGGL(greedy_partial_kernel<false>, grid, dim3(kVerifyThreads), 0, stream, logits, V, n_chunks, part);
    int st = launch_status();
    if (st != DFLASH_OK) return st;
    hipLaunchKernelGGL(greedy_decide_kernel, dim3(B), dim3(64 * T), 0, stream, part, draft, T, n_chunks, out_tok,
                       n_emit);
    return launch_status();
}

int launch_verify_sample(const float* logits, const int32_t* draft, const int32_t* q_idx, const double* q_prob,
                         int B, int T, int64_t V, float temperature, uint64_t seed, const uint64_t* request_id,
                         const int64_t* pos0, int32_t* out_tok, int32_t* n_emit, void* ws, hipStream_t stream) {
    const int n_chunks = (int)((V + kChunk - 1) / kChunk);
    ChunkStat* stats = reinterpret_cast<ChunkStat*>(ws);
    const double inv_tau = 1.0 / (double)temperature;
    const dim3 grid(n_chunks, B * T);
    const bool vec = (V % 4 == 0) && ((uintptr_t)logits % 16 == 0);
    if (vec)
        hipLaunchKernelGGL(sample_stats_kernel<true>, grid, dim3(kVerifyThreads), 0, stream, logits, V, n_chunks, inv_tau, stats);
    else
        hipLaunchKernelGGL(sample_stats_kernel<false>, grid, dim3(kVerifyThreads), 0, stream, logits, V, n_chunks, inv_tau, stats);
    int st = launch_status();
    if (st != DFLASH_OK) return st;
    if (q_idx)
        hipLaunchKernelGGL(sample_decide_kernel<true>, dim3(B), dim3(kVerifyThreads), 0, stream, logits, draft, q_idx,
                           q_prob, stats, T, V, n_chunks, inv_tau, seed, request_id, pos0, out_tok, n_emit);
    else
        hipLaunchKernelGGL(sample_decide_kernel<false>, dim3(B), dim3(kVerifyThreads), 0, stream, logits, draft,
                           nullptr, nullptr, stats, T, V, n_chunks, inv_tau, seed, request_id, pos0, out_tok, n_emit);
    return launch_status();
}

size_t sample_topkp_workspace_bytes(int B, int T, int64_t V, int top_k) {
    const int64_t n_chunks = (V + kChunk - 1) / kChunk;
    return (size_t)B * T * n_chunks * top_k * sizeof(uint64_t) + (size_t)B * T * sizeof(KeptSet);
}

int launch_verify_sample_topkp(const float* logits, const int32_t* draft, int B, int T, int64_t V,
                               float temperature, int top_k, float top_p, uint64_t seed,
                               const uint64_t* request_id, const int64_t* pos0, int32_t* out_tok,
                               int32_t* n_emit, void* ws, hipStream_t stream) {
    if (top_k < 1 || top_k > kMaxTopK || T > 16) return DFLASH_ERR_INVALID;  // the ABI bounds, again
    const int n_chunks = (int)((V + kChunk - 1) / kChunk);
    uint64_t* part = reinterpret_cast<uint64_t*>(ws);
    KeptSet* sets = reinterpret_cast<KeptSet*>(part + (size_t)B * T * n_chunks * top_k);
    const double inv_tau = 1.0 / (double)temperature;
    const dim3 grid(n_chunks, B * T);
    const bool vec = (V % 4 == 0) && ((uintptr_t)logits % 16 == 0);
    if (vec)
        hipLaunchKernelGGL(topk_chunk_kernel<true>, grid, dim3(kVerifyThreads), 0, stream, logits, V, n_chunks,
                           top_k, part);
    else
        hipLaunchKernelGGL(topk_chunk_kernel<false>, grid, dim3(kVerifyThreads), 0, stream, logits, V, n_chunks,
                           top_k, part);
    int st = launch_status();
    if (st != DFLASH_OK) return st;
    hipLaunchKernelGGL(topkp_set_kernel, dim3(B * T), dim3(kVerifyThreads), 0, stream, part, n_chunks, top_k,
                       inv_tau, (double)top_p, sets);
    st = launch_status();
    if (st != DFLASH_OK) return st;
    hipLaunchKernelGGL(topkp_decide_kernel, dim3(B), dim3(64), 0, stream, draft, sets, T, seed, request_id, pos0,
                       out_tok, n_emit);
    return launch_status();
}

}  // namespace dflash
