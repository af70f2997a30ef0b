// prefill.hip -- block-sparse causal sliding-window attention (+ sinks),
// prefill phase, for gfx950.
//
// What is computed ("Sliding Window and Sparse Attention, from Longformer to
// CSA2", s1 and s2; "Local and Sparse Attention: Reading Fewer Token
// Positions", Figures 1-2): o_i = softmax over j in A_i of
// (scale q_i.k_j + sink_bias [j<g]) applied to v_j, where A_i is the window
// i-w+1..i united with the sink positions 0..g-1, causal, each key once; an
// excluded pair gets -inf, never 0.
//
// How (tiled exact attention, s1 last paragraph of the first page; the FA
// description there is prior art, the layout below is gfx950's own):
//  * one workgroup = 4 waves = 128 query rows of one (batch, head); each wave
//    owns 32 rows for the whole run, so its row statistics never leave it;
//  * the workgroup visits only the key tiles of its band and sink blocks
//    (schedule.h), 64 keys per tile, double-buffered in LDS;
//  * both products run on the matrix cores with the 32x32 MFMA shapes:
//      S^T = K Q^T   (A = K tile from LDS, B = the wave's Q held in VGPRs)
//      O^T += V^T P^T (A = V tile stored transposed in LDS, B = P in VGPRs)
//    Computing the transposes makes the MFMA result layout put one query row
//    per lane (lanes l and l+32 share a row), so the online-softmax row max
//    and row sum are in-register reductions plus one permlane32 swap, the
//    probabilities P feed the second MFMA straight from the first one's
//    accumulators, and the output rescale needs no cross-lane traffic;
//  * FULL tiles skip masking; EDGE tiles (band edges, sinks, the ragged tail)
//    evaluate the exact per-pair predicate and set excluded scores to -inf;
//  * scores stay in raw q.k units; exp2 with scale*log2(e) folded into one
//    FMA per score.  A row with no attended key yet keeps m = -inf and is
//    guarded so that no -inf - -inf is ever formed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.h"
#include "schedule.h"

namespace swa {

constexpr int kBQ = 128;      // query rows per workgroup (4 waves x 32)
constexpr int kBK = 64;       // keys per tile (2 MFMA sub-blocks of 32)
constexpr int kThreads = 256;

template <bool BF16, int D>
struct PrefillCfg {
    using T = typename std::conditional<BF16, uint16_t, float>::type;
    static constexpr int kElem = BF16 ? 2 : 4;
    static constexpr int kEPC = 16 / kElem;            // elements per 16-byte chunk
    static constexpr int kCPR = D / kEPC;               // chunks per K/V row
    static constexpr int kKPad = BF16 ? 8 : 4;          // K row pad (elements)
    static constexpr int kVPad = 4;                     // V^T row pad (elements)
    static constexpr int kKStride = D + kKPad;
    static constexpr int kVStride = kBK + kVPad;
    static constexpr int kKElems = kBK * kKStride;
    static constexpr int kVElems = D * kVStride;
    static constexpr int kStage = kKElems + kVElems;
    static constexpr int kKChunks = kBK * kCPR / kThreads;         // 16-B K loads per thread
    static constexpr int kVBlocksAll = (kBK / 4) * kCPR;           // 4-key x 16-B V blocks per tile
    static constexpr int kVBlocks = (kVBlocksAll + kThreads - 1) / kThreads;  // per thread
    static_assert(kBK * kCPR % kThreads == 0, "K tile split");
    static_assert(kVBlocksAll % kThreads == 0 || kVBlocksAll < kThreads, "V tile split");
};

// One K/V tile: HBM -> registers (buffer loads; rows >= n come back as 0
// from the hardware range check) -> LDS (K row-major [key][d], V transposed
// [d][key]).  Per-thread offsets are fixed for the whole run; only the row
// of the tile start changes, which moves the buffer base (scalar work).
// A thread moves 4 keys x one 16-byte column chunk of V; the key group is the
// fastest-varying index across lanes, so the 16 lanes that write one V^T row
// together cover 128 contiguous bytes: with 32 four-byte LDS banks those
// writes, the K writes and both MFMA operand reads are free of bank conflicts
// (with the chunk index fastest instead, the transposed writes hit rows eight
// apart and collide 8-way).
template <bool BF16, int D>
struct TileLoader {
    using C = PrefillCfg<BF16, D>;
    using T = typename C::T;
    static constexpr uint32_t kRowBytes = D * C::kElem;
    uint4 k[C::kKChunks];
    uint4 v[C::kVBlocks][4];

    __device__ __forceinline__ void load(const T *kb, const T *vb, int k0, int n, int tid) {
        const uint32_t bytes = (uint32_t)(n - k0) * kRowBytes;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb + (size_t)k0 * D, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb + (size_t)k0 * D, bytes);
#pragma unroll
        for (int i = 0; i < C::kKChunks; ++i) {
            const int id = tid + kThreads * i;
            const int row = id / C::kCPR, cc = id % C::kCPR;
            k[i] = buffer_load16(rk, row * kRowBytes + cc * 16);
        }
#pragma unroll
        for (int i = 0; i < C::kVBlocks; ++i) {
            const int id = tid + kThreads * i;
            const int kg = id % (kBK / 4), cg = id / (kBK / 4);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                // ids past the tile's V blocks read past the resource: zeros, unused
                const uint32_t off = (id < C::kVBlocksAll) ? (4 * kg + rr) * kRowBytes + cg * 16 : 0xfffffff0u;
                v[i][rr] = buffer_load16(rv, off);
            }
        }
    }

    __device__ __forceinline__ void store(T *ks, T *vts, int tid) const {
#pragma unroll
        for (int i = 0; i < C::kKChunks; ++i) {
            const int id = tid + kThreads * i;
            const int row = id / C::kCPR, cc = id % C::kCPR;
            *reinterpret_cast<uint4 *>(ks + row * C::kKStride + cc * C::kEPC) = k[i];
        }
#pragma unroll
        for (int i = 0; i < C::kVBlocks; ++i) {
            const int id = tid + kThreads * i;
            if constexpr (C::kVBlocksAll % kThreads != 0) {
                if (id >= C::kVBlocksAll) break;
            }
            const int kg = id % (kBK / 4), cg = id / (kBK / 4);
            const uint32_t *r0 = reinterpret_cast<const uint32_t *>(&v[i][0]);
            const uint32_t *r1 = reinterpret_cast<const uint32_t *>(&v[i][1]);
            const uint32_t *r2 = reinterpret_cast<const uint32_t *>(&v[i][2]);
            const uint32_t *r3 = reinterpret_cast<const uint32_t *>(&v[i][3]);
            if constexpr (BF16) {
                // 4 keys x 8 columns -> 8 columns of 4 keys (8 bytes each)
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
                    const uint32_t lo = __builtin_amdgcn_perm(r1[cc >> 1], r0[cc >> 1], sel);
                    const uint32_t hi = __builtin_amdgcn_perm(r3[cc >> 1], r2[cc >> 1], sel);
                    *reinterpret_cast<uint2 *>(vts + (cg * 8 + cc) * C::kVStride + 4 * kg) = make_uint2(lo, hi);
                }
            } else {
                // 4 keys x 4 columns -> 4 columns of 4 keys (16 bytes each)
#pragma unroll
                for (int cc = 0; cc < 4; ++cc)
                    *reinterpret_cast<uint4 *>(vts + (cg * 4 + cc) * C::kVStride + 4 * kg) =
                        make_uint4(r0[cc], r1[cc], r2[cc], r3[cc]);
            }
        }
    }
};

template <bool BF16, int D>
__global__ __launch_bounds__(kThreads, BF16 ? 2 : 1) void prefill_kernel(
    const void *__restrict__ qp, const void *__restrict__ kp, const void *__restrict__ vp,
    void *__restrict__ op, float *__restrict__ lsep, int n, int nqb, int w, int g,
    float c2, float scale, float bias_raw, int total_wg) {
    using C = PrefillCfg<BF16, D>;
    using T = typename C::T;
    __shared__ __attribute__((aligned(16))) T smem[2 * C::kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 31;  // query row of this lane within the wave
    const int lh = lane >> 5;  // which half of the wave

    int unit, qb;
    workgroup_order(blockIdx.x, total_wg, nqb, &unit, &qb);
    const size_t base = (size_t)unit * n * D;
    const T *Q = reinterpret_cast<const T *>(qp) + base;
    const T *K = reinterpret_cast<const T *>(kp) + base;
    const T *V = reinterpret_cast<const T *>(vp) + base;

    const int q0 = qb * kBQ;
    const int q1 = min(q0 + kBQ, n) - 1;
    const int qi = q0 + wave * 32 + lr;  // this lane's query position
    const BandRange band = band_range(q0, q1, w, g, kBK);
    const int ntiles = band.count();
    // A score more than tau above the running max forces a rescale; below
    // that the stale max is kept (probabilities stay <= 2^8, exact after the
    // final normalisation).
    const float tau = 8.f / c2;

    // ---- Q of this wave's 32 rows as the B operand (kept in VGPRs) ----
    constexpr int kQRegs = BF16 ? D / 16 : D / 2;
    using QReg = typename std::conditional<BF16, bf16x8, float>::type;
    QReg qf[kQRegs];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + (size_t)q0 * D, (uint32_t)(n - q0) * D * C::kElem);
        const uint32_t rowoff = (uint32_t)(wave * 32 + lr) * D * C::kElem;
        if constexpr (BF16) {
#pragma unroll
            for (int c = 0; c < kQRegs; ++c)
                qf[c] = __builtin_bit_cast(bf16x8, buffer_load16(rq, rowoff + (16 * c + 8 * lh) * 2));
        } else {
#pragma unroll
            for (int c4 = 0; c4 < kQRegs / 4; ++c4) {
                // lane half lh takes the odd/even d of each pair: d = 2c + lh
                const uint4 a = buffer_load16(rq, rowoff + (8 * c4) * 4);
                const uint4 b = buffer_load16(rq, rowoff + (8 * c4 + 4) * 4);
                const uint32_t e[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) qf[4 * c4 + j] = __uint_as_float(lh ? e[2 * j + 1] : e[2 * j]);
            }
        }
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
    float m_run = kNegInf;  // reference row max (raw q.k units, bias included)
    float negm = 0.f;       // -m_run * c2, or 0 while m_run = -inf
    float l_run = 0.f;      // row sum over this lane's half of the keys

    TileLoader<BF16, D> ld;
    ld.load(K, V, band.block(0) * kBK, n, tid);
    ld.store(smem, smem + C::kKElems, tid);
    __syncthreads();

    // One tile of keys: K/V of tile t are in LDS stage `stage`; the loads of
    // tile t+1 go out first and land in the other stage at the end.
    auto do_tile = [&](int t, int stage, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const T *Ks = smem + stage * C::kStage;
        const T *Vts = Ks + C::kKElems;
        const int k0 = band.block(t) * kBK;
        const bool has_next = (t + 1 < ntiles);
        if (has_next) ld.load(K, V, band.block(t + 1) * kBK, n, tid);

        // ---- S^T = K Q^T for the two 32-key sub-blocks ----
        f32x16 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
            if constexpr (BF16) {
                const T *krow = Ks + (32 * sb + lr) * C::kKStride + 8 * lh;
#pragma unroll
                for (int c = 0; c < D / 16; ++c) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(krow + 16 * c);
                    s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[sb], 0, 0, 0);
                }
            } else {
                const T *krow = Ks + (32 * sb + lr) * C::kKStride + lh;
#pragma unroll
                for (int c = 0; c < D / 2; ++c)
                    s[sb] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * c], qf[c], s[sb], 0, 0, 0);
            }
        }
        // s[sb][r] = q_qi . k_j with j = k0 + 32 sb + 8 (r/4) + 4 lh + r%4

        // ---- exact masking (and sink bias) on tiles the band or sinks cut ----
        if constexpr (MASKED) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = k0 + 32 * sb + 8 * (r >> 2) + 4 * lh + (r & 3);
                    const float x = s[sb][r] + (j < g ? bias_raw : 0.f);
                    s[sb][r] = pair_attended(qi, j, n, w, g) ? x : kNegInf;
                }
        }

        // ---- online softmax with a lazily moved reference max ----
        float mx = kNegInf;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
        mx = half_swap_max(mx);
        if (__any(mx > m_run + tau)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_run - m_new) * c2);
            m_run = m_new;
            negm = (m_new == kNegInf) ? 0.f : -m_new * c2;
            l_run *= alpha;
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
        }

        // ---- P = exp2(s c2 - m c2); O^T += V^T P^T ----
        if constexpr (BF16) {
            bf16x8 pb[4];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pb[kc][e] = static_cast<__bf16>(fast_exp2(fmaf(s[kc >> 1][8 * (kc & 1) + e], c2, negm)));
            // row sum of the bf16 probabilities the value product uses
            const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
            float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const bf16x2 p01 = {pb[kc][0], pb[kc][1]}, p23 = {pb[kc][2], pb[kc][3]};
                const bf16x2 p45 = {pb[kc][4], pb[kc][5]}, p67 = {pb[kc][6], pb[kc][7]};
                ls0 = __builtin_amdgcn_fdot2_f32_bf16(p01, ones, ls0, false);
                ls1 = __builtin_amdgcn_fdot2_f32_bf16(p23, ones, ls1, false);
                ls0 = __builtin_amdgcn_fdot2_f32_bf16(p45, ones, ls0, false);
                ls1 = __builtin_amdgcn_fdot2_f32_bf16(p67, ones, ls1, false);
            }
            l_run += ls0 + ls1;
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const T *vrow = Vts + (32 * cb + lr) * C::kVStride + 4 * lh;
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + 16 * kc);
                    const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 16 * kc + 8);
                    const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                    oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc], oacc[cb], 0, 0, 0);
                }
            }
        } else {
            float lsum = 0.f;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[sb][r] = fast_exp2(fmaf(s[sb][r], c2, negm));
                    lsum += s[sb][r];
                }
            l_run += lsum;
#pragma unroll
            for (int cb = 0; cb < D / 32; ++cb) {
                const T *vrow = Vts + (32 * cb + lr) * C::kVStride + 4 * lh;
#pragma unroll
                for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float a = vrow[32 * sb + 8 * (r >> 2) + (r & 3)];
                        oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[sb][r], oacc[cb], 0, 0, 0);
                    }
            }
        }

        if (has_next) {
            T *nxt = smem + (stage ^ 1) * C::kStage;
            ld.store(nxt, nxt + C::kKElems, tid);
        }
        __syncthreads();
    };

    // Visiting order: sink tiles and the band's lower-edge tiles (masked),
    // then the run of FULL tiles in a tight loop of its own, then the
    // diagonal tiles (masked).  The FULL run is contiguous in key-block order.
    int t_full_lo = ntiles, t_full_hi = ntiles;  // FULL tiles are [t_full_lo, t_full_hi)
    for (int t = 0; t < ntiles; ++t) {
        const int kb = band.block(t);
        if (tile_full(q0, q1, kb * kBK, kb * kBK + kBK - 1, n, w, g)) {
            if (t_full_lo == ntiles) t_full_lo = t;
            t_full_hi = t + 1;
        }
    }
    int t = 0, stage = 0;
    for (; t < t_full_lo; ++t, stage ^= 1) do_tile(t, stage, std::true_type{});
    for (; t < t_full_hi; ++t, stage ^= 1) do_tile(t, stage, std::false_type{});
    for (; t < ntiles; ++t, stage ^= 1) do_tile(t, stage, std::true_type{});

    // ---- epilogue: normalise, store O (and LSE) ----
    const float l_tot = half_swap_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qi < n) {
        T *O = reinterpret_cast<T *>(op) + base + (size_t)qi * D;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                const int c = 32 * cb + 8 * gq + 4 * lh;
                const float x0 = oacc[cb][4 * gq + 0] * inv, x1 = oacc[cb][4 * gq + 1] * inv;
                const float x2 = oacc[cb][4 * gq + 2] * inv, x3 = oacc[cb][4 * gq + 3] * inv;
                if constexpr (BF16) {
                    *reinterpret_cast<uint2 *>(O + c) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
                } else {
                    *reinterpret_cast<float4 *>(O + c) = make_float4(x0, x1, x2, x3);
                }
            }
        if (lsep != nullptr && lh == 0) lsep[(size_t)unit * n + qi] = m_run * scale + logf(l_tot);
    }
}

// Host launcher (validated arguments only).
template <bool BF16, int D>
static hipError_t launch_prefill_t(const void *q, const void *k, const void *v, void *o, float *lse,
                                   int units, int n, int w, int g, float scale, float sink_bias,
                                   hipStream_t stream) {
    const int nqb = (n + kBQ - 1) / kBQ;
    const int total = units * nqb;
    const float c2 = (float)((double)scale * kLog2e);
    const float bias_raw = (float)((double)sink_bias / (double)scale);
    hipLaunchKernelGGL((prefill_kernel<BF16, D>), dim3(total), dim3(kThreads), 0, stream, q, k, v, o, lse, n,
                       nqb, w, g, c2, scale, bias_raw, total);
    return hipGetLastError();
}

hipError_t launch_prefill(const void *q, const void *k, const void *v, void *o, float *lse, int units,
                          int n, int d, int w, int g, float scale, float sink_bias, bool bf16,
                          hipStream_t stream) {
    if (bf16) {
        if (d == 128) return launch_prefill_t<true, 128>(q, k, v, o, lse, units, n, w, g, scale, sink_bias, stream);
        return launch_prefill_t<true, 64>(q, k, v, o, lse, units, n, w, g, scale, sink_bias, stream);
    }
    if (d == 128) return launch_prefill_t<false, 128>(q, k, v, o, lse, units, n, w, g, scale, sink_bias, stream);
    return launch_prefill_t<false, 64>(q, k, v, o, lse, units, n, w, g, scale, sink_bias, stream);
}

}  // namespace swa
