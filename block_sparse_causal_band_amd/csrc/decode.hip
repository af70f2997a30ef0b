// decode.hip -- one query per (batch, head) against a rolling-buffer KV cache
// with resident sink rows, for gfx950.
//
// Cache rows per (batch, head): rows 0..g-1 hold the sink positions 0..g-1;
// rows g..g+w-1 are the rolling buffer where position t lives in slot t mod w
// ("Sliding Window and Sparse Attention, from Longformer to CSA2", s2:
// rolling buffer and attention sinks; "Local and Sparse Attention: Reading
// Fewer Token Positions", Figure 4: circular overwrite, always-read positions
// stay stored).  For the query at position p (its own K/V already appended):
//   * ring slot s holds the latest position t <= p with t = s mod w; it is
//     read when t >= 0 exists, i.e. always once p >= w-1, else iff s <= p;
//   * sink row t is read only when t has left the window (t < p-w+1);
//     otherwise the ring holds the same position and that copy is read, so
//     every position is read once (Figure 2 text of the second page);
//   * keys at a position < g get the sink bias.
//
// Decode is bound by HBM bandwidth (first page, s1: the decode step streams
// the cache): every cache row is read once, with 16-byte loads where 16 (d=128
// bf16) consecutive lanes cover one row, so one wave-wide load instruction
// reads 4 whole consecutive rows.  The q.k dot is an fp32 FMA chain plus a
// butterfly over the lanes of a row; the online softmax keeps one (m, l) per
// row group and each lane accumulates its own 8 output columns.  Groups are
// merged through LDS at the end; when one (batch, head) is split over several
// workgroups, partial (m, l, o) go to the workspace and a second kernel merges
// them by log-sum-exp (s10 glossary, LSE).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.h"

namespace swa {

constexpr int kDecThreads = 256;
constexpr int kDecUnroll = 4;  // row loads in flight per lane per step, for K and for V each

template <bool BF16, int D>
struct DecodeCfg {
    using T = typename std::conditional<BF16, uint16_t, float>::type;
    static constexpr int kEPC = BF16 ? 8 : 4;     // elements per 16-byte chunk
    static constexpr int kLPR = D / kEPC;         // lanes per cache row
    static constexpr int kRPI = 64 / kLPR;        // rows per wave-wide load
    static constexpr int kGroups = (kDecThreads / 64) * kRPI;  // row groups per workgroup
    static constexpr int kRowsPerStep = (kDecThreads / 64) * kDecUnroll * kRPI;
};

template <bool BF16>
__device__ __forceinline__ void unpack(const uint4 &x, float *f) {
    if constexpr (BF16) {
        const uint32_t *u = reinterpret_cast<const uint32_t *>(&x);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16lo(u[i]);
            f[2 * i + 1] = bf16hi(u[i]);
        }
    } else {
        f[0] = __uint_as_float(x.x);
        f[1] = __uint_as_float(x.y);
        f[2] = __uint_as_float(x.z);
        f[3] = __uint_as_float(x.w);
    }
}

// x of another lane through a DPP move (ctrl: quad_perm 0x00-0xff, row
// mirror 0x140, half-row mirror 0x141); every lane is active where it is used.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the LPR lanes that share one cache row (aligned groups of 8, 16 or
// 32 lanes).  Within 16 lanes every step is a DPP move: swap neighbours, swap
// pairs, then the half-row mirror (lane i <- 7-i: quad 0 meets quad 1) and the
// row mirror (lane i <- 15-i: half 0 meets half 1), each pairing lanes that
// hold equal partial sums so far.  32 lanes add one cross-row shuffle.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(LPR == 8 || LPR == 16 || LPR == 32, "row group of 8, 16 or 32 lanes");
    x += dpp_mov<0xb1>(x);   // quad_perm [1,0,3,2]
    x += dpp_mov<0x4e>(x);   // quad_perm [2,3,0,1]
    x += dpp_mov<0x141>(x);
    if constexpr (LPR >= 16) x += dpp_mov<0x140>(x);
    if constexpr (LPR >= 32) x += __shfl_xor(x, 16, 64);
    return x;
}

// Partial state of one workgroup: m (raw q.k units incl. bias), l, o[D]
// (unnormalised), for each of its GQ query heads.  The GQ query heads share
// one key/value head (grouped-query attention), so each cache row is read
// once for all of them.
template <bool BF16, int D, int GQ>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const void *__restrict__ qp, const void *__restrict__ kcp, const void *__restrict__ vcp,
    const int64_t *__restrict__ pos, void *__restrict__ op, float *__restrict__ lsep, int heads, int kv_heads,
    int w, int g, float c2, float scale, float bias_raw, int splits, int rows_per_split, float *__restrict__ ws) {
    using C = DecodeCfg<BF16, D>;
    using T = typename C::T;
    constexpr int EPC = C::kEPC, LPR = C::kLPR, RPI = C::kRPI;
    __shared__ float sh_m[C::kGroups], sh_l[C::kGroups];
    __shared__ float sh_o[C::kGroups][D];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp_in_wave = lane / LPR, sub = lane % LPR;
    const int group = wave * RPI + grp_in_wave;
    const int split = blockIdx.x % splits;
    const int job = blockIdx.x / splits;       // (batch, kv head, chunk of GQ query heads)
    const int chunks = heads / kv_heads / GQ;  // query-head chunks per kv head
    const int chunk = job % chunks;
    const int kvu = job / chunks;              // batch * kv_heads + kv head
    const int b = kvu / kv_heads;
    const int h0 = (kvu % kv_heads) * (heads / kv_heads) + chunk * GQ;  // first query head
    const int unit0 = b * heads + h0;          // batch * heads + query head of head 0
    const int R = g + w;
    const int64_t p = pos[b];

    const T *kc = reinterpret_cast<const T *>(kcp) + (size_t)kvu * R * D;
    const T *vc = reinterpret_cast<const T *>(vcp) + (size_t)kvu * R * D;

    // the lane's chunk of each query: fp32 values, and for bf16 also the
    // packed pairs that the q.k dot2 instructions take as they are
    float qf[GQ][EPC];
    uint4 qx[GQ];
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
        const T *q = reinterpret_cast<const T *>(qp) + (size_t)(unit0 + j) * D;
        qx[j] = *reinterpret_cast<const uint4 *>(q + sub * EPC);
        if constexpr (!BF16) unpack<BF16>(qx[j], qf[j]);
    }

    // ring geometry for this query position
    const bool ring_full = (p >= (int64_t)w - 1);
    const int pm = (p >= 0) ? (int)(p % w) : 0;  // slot of the query itself
    const int64_t win_lo = p - w + 1;           // first window position

    float m[GQ], l[GQ], o[GQ][EPC];
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
        m[j] = kNegInf;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) o[j][e] = 0.f;
    }

    const int r_begin = split * rows_per_split;
    const int r_end = min(R, r_begin + rows_per_split);
    for (int r0 = r_begin; r0 < r_end; r0 += C::kRowsPerStep) {
        uint4 kx[kDecUnroll], vx[kDecUnroll];
        int rows[kDecUnroll];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            int r = r0 + (wave * kDecUnroll + u) * RPI + grp_in_wave;
            rows[u] = r;
            if (r < r_end) {
                kx[u] = load_stream16(kc + (size_t)r * D + sub * EPC);
                vx[u] = load_stream16(vc + (size_t)r * D + sub * EPC);
            } else {
                kx[u] = make_uint4(0, 0, 0, 0);
                vx[u] = make_uint4(0, 0, 0, 0);
            }
        }
        float s[GQ][kDecUnroll];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) {
            // which position does row r hold, and is it read?
            int r = rows[u];
            bool valid;
            int64_t t;
            if (r >= r_end || p < 0) {
                valid = false;
                t = 0;
            } else if (r < g) {
                t = r;
                valid = (t <= p) && (t < win_lo);
            } else {
                int sl = r - g;
                if (ring_full) {
                    int dd = pm - sl;
                    if (dd < 0) dd += w;
                    t = p - dd;
                    valid = true;
                } else {
                    t = sl;
                    valid = (sl <= p);
                }
            }
            const float bias = (t < g) ? bias_raw : 0.f;
#pragma unroll
            for (int j = 0; j < GQ; ++j) {
                float acc = 0.f;
                if constexpr (BF16) {
                    // bf16 pairs straight from the cache: products exact, fp32 sums
                    const bf16x2 *k2 = reinterpret_cast<const bf16x2 *>(&kx[u]);
                    const bf16x2 *q2 = reinterpret_cast<const bf16x2 *>(&qx[j]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_fdot2_f32_bf16(q2[e], k2[e], acc, false);
                } else {
                    float kf[EPC];
                    unpack<BF16>(kx[u], kf);
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc = fmaf(qf[j][e], kf[e], acc);
                }
                acc = group_sum<LPR>(acc) + bias;
                s[j][u] = valid ? acc : kNegInf;
            }
        }
        float vf[kDecUnroll][EPC];
#pragma unroll
        for (int u = 0; u < kDecUnroll; ++u) unpack<BF16>(vx[u], vf[u]);
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
            float mx = s[j][0];
#pragma unroll
            for (int u = 1; u < kDecUnroll; ++u) mx = fmaxf(mx, s[j][u]);
            const float m_new = fmaxf(m[j], mx);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = fast_exp2((m[j] - m_use) * c2);
            const float neg = -m_use * c2;
            l[j] *= alpha;
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[j][e] *= alpha;
#pragma unroll
            for (int u = 0; u < kDecUnroll; ++u) {
                const float pu = fast_exp2(fmaf(s[j][u], c2, neg));
                l[j] += pu;
#pragma unroll
                for (int e = 0; e < EPC; ++e) o[j][e] = fmaf(pu, vf[u][e], o[j][e]);
            }
            m[j] = m_new;
        }
    }

    // ---- merge the row groups of this workgroup, one query head at a time ----
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
        const int unit = unit0 + j;
        if (j > 0) __syncthreads();  // the previous head's merge has read the LDS
        if (sub == 0) {
            sh_m[group] = m[j];
            sh_l[group] = l[j];
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e) sh_o[group][sub * EPC + e] = o[j][e];
        __syncthreads();
        float M = kNegInf;
#pragma unroll
        for (int gi = 0; gi < C::kGroups; ++gi) M = fmaxf(M, sh_m[gi]);
        const float M_use = (M == kNegInf) ? 0.f : M;
        float L = 0.f;
#pragma unroll
        for (int gi = 0; gi < C::kGroups; ++gi) L += sh_l[gi] * fast_exp2((sh_m[gi] - M_use) * c2);

        if (splits == 1) {
            const float inv = (L > 0.f) ? 1.f / L : __builtin_nanf("");
            T *out = reinterpret_cast<T *>(op) + (size_t)unit * D;
            for (int c = tid; c < D; c += kDecThreads) {
                float acc = 0.f;
#pragma unroll
                for (int gi = 0; gi < C::kGroups; ++gi) acc += sh_o[gi][c] * fast_exp2((sh_m[gi] - M_use) * c2);
                float x = acc * inv;
                if constexpr (BF16)
                    out[c] = (uint16_t)f32_to_bf16_bits(x);
                else
                    out[c] = x;
            }
            if (lsep != nullptr && tid == 0) lsep[unit] = (L > 0.f) ? M * scale + logf(L) : __builtin_nanf("");
        } else {
            float *rec = ws + ((size_t)unit * splits + split) * (2 + D);
            for (int c = tid; c < D; c += kDecThreads) {
                float acc = 0.f;
#pragma unroll
                for (int gi = 0; gi < C::kGroups; ++gi) acc += sh_o[gi][c] * fast_exp2((sh_m[gi] - M_use) * c2);
                rec[2 + c] = acc;
            }
            if (tid == 0) {
                rec[0] = M;
                rec[1] = L;
            }
        }
    }
}

// Merge S partial states of one (batch, head) by log-sum-exp.
template <bool BF16, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float *__restrict__ ws, void *__restrict__ op,
                                                         float *__restrict__ lsep, int splits, float c2,
                                                         float scale) {
    using T = typename std::conditional<BF16, uint16_t, float>::type;
    const int unit = blockIdx.x, c = threadIdx.x;
    const float *rec = ws + (size_t)unit * splits * (2 + D);
    float M = kNegInf;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, rec[s * (2 + D)]);
    const float M_use = (M == kNegInf) ? 0.f : M;
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float *r = rec + s * (2 + D);
        float f = fast_exp2((r[0] - M_use) * c2);
        L += r[1] * f;
        acc += r[2 + c] * f;
    }
    float x = (L > 0.f) ? acc / L : __builtin_nanf("");
    T *out = reinterpret_cast<T *>(op) + (size_t)unit * D;
    if constexpr (BF16)
        out[c] = (uint16_t)f32_to_bf16_bits(x);
    else
        out[c] = x;
    if (lsep != nullptr && c == 0) lsep[unit] = (L > 0.f) ? M * scale + logf(L) : __builtin_nanf("");
}

// Query heads per decode workgroup: the largest power of two <= 8 that
// divides the group size (query heads per key/value head).
int decode_heads_per_wg(int group) {
    int gq = 1;
    while (gq < 8 && group % (2 * gq) == 0) gq *= 2;
    return gq;
}

// Split count: enough workgroups to cover the chip, at least 256 cache rows each.
int decode_splits(int jobs, int rows) {
    if (jobs >= 1024) return 1;
    int s = (2048 + jobs - 1) / jobs;
    int max_s = rows / 256;
    if (max_s < 1) max_s = 1;
    if (s > max_s) s = max_s;
    if (s > 64) s = 64;
    return s < 1 ? 1 : s;
}

// jobs = batch * heads / (query heads per workgroup): workgroups before splitting
static int decode_jobs(int batch, int heads, int kv_heads) {
    return batch * (heads / decode_heads_per_wg(heads / kv_heads));
}

size_t decode_workspace_bytes(int batch, int heads, int kv_heads, int d, int rows) {
    int s = decode_splits(decode_jobs(batch, heads, kv_heads), rows);
    if (s == 1) return 0;
    return (size_t)batch * heads * s * (2 + d) * sizeof(float);
}

template <bool BF16, int D, int GQ>
static hipError_t launch_decode_t(const void *q, const void *kc, const void *vc, const int64_t *pos, void *o,
                                  float *lse, int batch, int heads, int kv_heads, int w, int g, float scale,
                                  float sink_bias, void *ws, hipStream_t stream) {
    const int R = g + w;
    const int jobs = decode_jobs(batch, heads, kv_heads);
    const int splits = decode_splits(jobs, R);
    const int rps = (R + splits - 1) / splits;
    const float c2 = (float)((double)scale * kLog2e);
    const float bias_raw = (float)((double)sink_bias / (double)scale);
    hipLaunchKernelGGL((decode_kernel<BF16, D, GQ>), dim3(jobs * splits), dim3(kDecThreads), 0, stream, q, kc, vc,
                       pos, o, lse, heads, kv_heads, w, g, c2, scale, bias_raw, splits, rps, (float *)ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    hipLaunchKernelGGL((decode_merge_kernel<BF16, D>), dim3(batch * heads), dim3(D), 0, stream, (const float *)ws,
                       o, lse, splits, c2, scale);
    return hipGetLastError();
}

template <bool BF16, int D>
static hipError_t launch_decode_d(const void *q, const void *kc, const void *vc, const int64_t *pos, void *o,
                                  float *lse, int batch, int heads, int kv_heads, int w, int g, float scale,
                                  float sink_bias, void *ws, hipStream_t stream) {
    switch (decode_heads_per_wg(heads / kv_heads)) {
        case 8: return launch_decode_t<BF16, D, 8>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale, sink_bias, ws, stream);
        case 4: return launch_decode_t<BF16, D, 4>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale, sink_bias, ws, stream);
        case 2: return launch_decode_t<BF16, D, 2>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale, sink_bias, ws, stream);
        default: return launch_decode_t<BF16, D, 1>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale, sink_bias, ws, stream);
    }
}

hipError_t launch_decode(const void *q, const void *kc, const void *vc, const int64_t *pos, void *o, float *lse,
                         int batch, int heads, int kv_heads, int d, int w, int g, float scale, float sink_bias,
                         bool bf16, void *ws, hipStream_t stream) {
    if (bf16) {
        if (d == 128) return launch_decode_d<true, 128>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale, sink_bias, ws, stream);
        return launch_decode_d<true, 64>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale, sink_bias, ws, stream);
    }
    if (d == 128) return launch_decode_d<false, 128>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale, sink_bias, ws, stream);
    return launch_decode_d<false, 64>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale, sink_bias, ws, stream);
}

// ---------------------------------------------------------------------------
// kv_append: token j of batch entry b is at position P = pos[b] + j.  It goes
// to ring row g + P mod w when it is one of the last w new tokens (earlier
// ones would be overwritten by a later token of the same call), and to sink
// row P when P < g.  One thread copies 16 bytes of K and 16 bytes of V.
template <int ELEM>
__global__ __launch_bounds__(256) void kv_append_kernel(uint8_t *__restrict__ kc, uint8_t *__restrict__ vc,
                                                        const uint8_t *__restrict__ kn,
                                                        const uint8_t *__restrict__ vn,
                                                        const int64_t *__restrict__ pos, int heads, int tn,
                                                        int d, int w, int g, long long total) {
    const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
    if (id >= total) return;
    const int cpr = d * ELEM / 16;  // 16-byte chunks per row
    const int chunk = (int)(id % cpr);
    const long long rowid = id / cpr;
    const int j = (int)(rowid % tn);
    const long long unit = rowid / tn;
    const int b = (int)(unit / heads);
    const int64_t P0 = pos[b];
    if (P0 < 0) return;
    const int64_t P = P0 + j;
    const size_t row_bytes = (size_t)d * ELEM;
    const size_t src = ((size_t)unit * tn + j) * row_bytes + (size_t)chunk * 16;
    const uint4 kx = *reinterpret_cast<const uint4 *>(kn + src);
    const uint4 vx = *reinterpret_cast<const uint4 *>(vn + src);
    const size_t cache_base = (size_t)unit * (g + w) * row_bytes + (size_t)chunk * 16;
    if (j >= tn - w) {
        const size_t dst = cache_base + (size_t)(g + (int)(P % w)) * row_bytes;
        *reinterpret_cast<uint4 *>(kc + dst) = kx;
        *reinterpret_cast<uint4 *>(vc + dst) = vx;
    }
    if (P < g) {
        const size_t dst = cache_base + (size_t)P * row_bytes;
        *reinterpret_cast<uint4 *>(kc + dst) = kx;
        *reinterpret_cast<uint4 *>(vc + dst) = vx;
    }
}

hipError_t launch_kv_append(void *kc, void *vc, const void *kn, const void *vn, const int64_t *pos, int batch,
                            int heads, int tn, int d, int w, int g, bool bf16, hipStream_t stream) {
    const int elem = bf16 ? 2 : 4;
    const long long total = (long long)batch * heads * tn * (d * elem / 16);
    const long long blocks = (total + 255) / 256;
    if (bf16)
        hipLaunchKernelGGL(kv_append_kernel<2>, dim3((unsigned)blocks), dim3(256), 0, stream, (uint8_t *)kc,
                           (uint8_t *)vc, (const uint8_t *)kn, (const uint8_t *)vn, pos, heads, tn, d, w, g, total);
    else
        hipLaunchKernelGGL(kv_append_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream, (uint8_t *)kc,
                           (uint8_t *)vc, (const uint8_t *)kn, (const uint8_t *)vn, pos, heads, tn, d, w, g, total);
    return hipGetLastError();
}

}  // namespace swa
