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

#include <mutex>
#include <type_traits>

#include "common.h"

namespace swa {

constexpr int kDecThreads = 256;

// Cache element kinds: each lane reads one chunk of kEPC elements (kBytes)
// of a row per load; kUnroll rows per lane are in flight, for K and for V.
struct CacheBf16 {
    static constexpr int kEPC = 8, kBytes = 16, kUnroll = 4;
};
struct CacheF32 {
    static constexpr int kEPC = 4, kBytes = 16, kUnroll = 4;
};
struct CacheFp8 {  // OCP E4M3 bytes, 8 per lane: the same lane layout as bf16, twice the rows in flight
    static constexpr int kEPC = 8, kBytes = 8, kUnroll = 8;
};
struct CacheFp8W {  // OCP E4M3 bytes, 16 per lane (8 lanes per 128-byte row): one query head per workgroup
    static constexpr int kEPC = 16, kBytes = 16, kUnroll = 4;
};
template <typename CK>
constexpr bool is_fp8() { return std::is_same<CK, CacheFp8>::value || std::is_same<CK, CacheFp8W>::value; }

template <typename CK, int D>
struct DecodeCfg {
    using V = typename std::conditional<CK::kBytes == 16, uint4, uint2>::type;  // one lane's chunk
    static constexpr int kEPC = CK::kEPC;
    static constexpr int kLPR = D / kEPC;         // lanes per cache row
    static constexpr int kRPI = 64 / kLPR;        // rows per wave-wide load
    static constexpr int kUnroll = CK::kUnroll;
    static constexpr int kRowBytes = D * CK::kBytes / CK::kEPC;
    static constexpr int kGroups = (kDecThreads / 64) * kRPI;  // row groups per workgroup
    static constexpr int kRowsPerStep = (kDecThreads / 64) * kUnroll * kRPI;
};

__device__ __forceinline__ void load_chunk(const uint8_t *p, uint4 &x) { x = load_stream16(p); }
__device__ __forceinline__ void load_chunk(const uint8_t *p, uint2 &x) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
    x = make_uint2(v[0], v[1]);
}
__device__ __forceinline__ void zero_chunk(uint4 &x) { x = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void zero_chunk(uint2 &x) { x = make_uint2(0, 0); }

// chunk -> fp32 values (fp8: the hardware conversion of OCP E4M3, exact)
template <typename CK>
__device__ __forceinline__ void unpack(const typename DecodeCfg<CK, 64>::V &x, float *f) {
    if constexpr (std::is_same<CK, CacheBf16>::value) {
        const uint32_t *u = reinterpret_cast<const uint32_t *>(&x);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = bf16lo(u[i]);
            f[2 * i + 1] = bf16hi(u[i]);
        }
    } else if constexpr (std::is_same<CK, CacheF32>::value) {
        f[0] = __uint_as_float(x.x);
        f[1] = __uint_as_float(x.y);
        f[2] = __uint_as_float(x.z);
        f[3] = __uint_as_float(x.w);
    } else {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        constexpr int NW = sizeof(x) / 4;  // 32-bit words of 4 codes
        const uint32_t *u = reinterpret_cast<const uint32_t *>(&x);
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[i], false);
            const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[i], true);
            f[4 * i + 0] = a.x;
            f[4 * i + 1] = a.y;
            f[4 * i + 2] = b.x;
            f[4 * i + 3] = b.y;
        }
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
// once for all of them.  QT: type of q and o (bf16 bits or fp32); CK: cache
// element kind.  An fp8 cache carries one scale per (batch, key/value head)
// for K (ksc) and V (vsc): a row's value is scale x its E4M3 value.
template <typename QT, typename CK, int D, int GQ>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const void *__restrict__ qp, const void *__restrict__ kcp, const void *__restrict__ vcp,
    const int64_t *__restrict__ pos, void *__restrict__ op, float *__restrict__ lsep, int heads, int kv_heads,
    int w, int g, float c2, float scale, float bias_raw, int splits, int rows_per_split, float *__restrict__ ws,
    const float *__restrict__ ksc, const float *__restrict__ vsc) {
    using C = DecodeCfg<CK, D>;
    using CV = typename C::V;
    constexpr int EPC = C::kEPC, LPR = C::kLPR, RPI = C::kRPI, UN = C::kUnroll;
    constexpr bool kDot2 = std::is_same<QT, uint16_t>::value && std::is_same<CK, CacheBf16>::value;
    constexpr bool kFp8 = is_fp8<CK>();
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
    const float kscale = kFp8 ? ksc[kvu] : 1.f;
    const float vscale = kFp8 ? vsc[kvu] : 1.f;

    const uint8_t *kc = reinterpret_cast<const uint8_t *>(kcp) + (size_t)kvu * R * C::kRowBytes;
    const uint8_t *vc = reinterpret_cast<const uint8_t *>(vcp) + (size_t)kvu * R * C::kRowBytes;

    // the lane's EPC elements of each query: fp32 values, and for bf16 q over a
    // bf16 cache also the packed pairs that the q.k dot2 instructions take
    float qf[GQ][EPC];
    uint4 qx[GQ];
#pragma unroll
    for (int j = 0; j < GQ; ++j) {
        const QT *q = reinterpret_cast<const QT *>(qp) + (size_t)(unit0 + j) * D + sub * EPC;
        if constexpr (std::is_same<QT, uint16_t>::value) {
            qx[j] = *reinterpret_cast<const uint4 *>(q);
            if constexpr (!kDot2) {
#pragma unroll
                for (int e = 0; e < EPC; e += 8) unpack<CacheBf16>(*reinterpret_cast<const uint4 *>(q + e), &qf[j][e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < EPC; e += 4) {
                const float4 f = *reinterpret_cast<const float4 *>(q + e);
                qf[j][e] = f.x;
                qf[j][e + 1] = f.y;
                qf[j][e + 2] = f.z;
                qf[j][e + 3] = f.w;
            }
        }
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
        CV kx[UN], vx[UN];
        int rows[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
            int r = r0 + (wave * UN + u) * RPI + grp_in_wave;
            rows[u] = r;
            if (r < r_end) {
                load_chunk(kc + (size_t)r * C::kRowBytes + sub * CK::kBytes, kx[u]);
                load_chunk(vc + (size_t)r * C::kRowBytes + sub * CK::kBytes, vx[u]);
            } else {
                zero_chunk(kx[u]);
                zero_chunk(vx[u]);
            }
        }
        float s[GQ][UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
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
            // a row that is not read may hold anything (an unwritten slot):
            // its score is -inf and its value chunk is zeroed, so that 0 * NaN
            // cannot reach the output
            if (!valid) zero_chunk(vx[u]);
            float kf[EPC];
            if constexpr (!kDot2) unpack<CK>(kx[u], kf);
#pragma unroll
            for (int j = 0; j < GQ; ++j) {
                float acc = 0.f;
                if constexpr (kDot2) {
                    // bf16 pairs straight from the cache: products exact, fp32 sums
                    const bf16x2 *k2 = reinterpret_cast<const bf16x2 *>(&kx[u]);
                    const bf16x2 *q2 = reinterpret_cast<const bf16x2 *>(&qx[j]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_fdot2_f32_bf16(q2[e], k2[e], acc, false);
                } else {
#pragma unroll
                    for (int e = 0; e < EPC; ++e) acc = fmaf(qf[j][e], kf[e], acc);
                }
                acc = group_sum<LPR>(acc);
                if constexpr (kFp8) acc *= kscale;
                acc += bias;
                s[j][u] = valid ? acc : kNegInf;
            }
        }
        float vf[UN][EPC];
#pragma unroll
        for (int u = 0; u < UN; ++u) unpack<CK>(vx[u], vf[u]);
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
            float mx = s[j][0];
#pragma unroll
            for (int u = 1; u < UN; ++u) mx = fmaxf(mx, s[j][u]);
            const float m_new = fmaxf(m[j], mx);
            const float m_use = (m_new == kNegInf) ? 0.f : m_new;
            const float alpha = fast_exp2((m[j] - m_use) * c2);
            const float neg = -m_use * c2;
            l[j] *= alpha;
#pragma unroll
            for (int e = 0; e < EPC; ++e) o[j][e] *= alpha;
#pragma unroll
            for (int u = 0; u < UN; ++u) {
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
            const float inv = (L > 0.f) ? vscale / L : __builtin_nanf("");
            QT *out = reinterpret_cast<QT *>(op) + (size_t)unit * D;
            for (int c = tid; c < D; c += kDecThreads) {
                float acc = 0.f;
#pragma unroll
                for (int gi = 0; gi < C::kGroups; ++gi) acc += sh_o[gi][c] * fast_exp2((sh_m[gi] - M_use) * c2);
                float x = acc * inv;
                if constexpr (std::is_same<QT, uint16_t>::value)
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
                rec[2 + c] = acc * vscale;
            }
            if (tid == 0) {
                rec[0] = M;
                rec[1] = L;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped-query decode on the matrix cores (bf16 q and cache).  The query
// heads that share one key/value head are the 16-wide side of the MFMAs
// (heads past the group's are zero):
//   S^T[16 keys x 16 heads] = K[16 keys x 32 d] Q^T  (v_mfma_f32_16x16x32_bf16, D/32 of them)
//   O^T[16 d x 16 heads]   += V^T[16 d x 16 keys] P^T (v_mfma_f32_16x16x16_bf16, one per 16 columns)
// so each cache row is read once for the whole group and the dot products
// leave the VALU.  Lane l holds head l%16 in S^T, P^T and O^T alike (the
// score result is the probability operand as it stands), so a head's
// softmax state sits in the 4 lanes l%16 = h and the accumulators need no
// cross-lane traffic; the reference max moves lazily as in the prefill.
// K and V of a block of 16 cache rows go to LDS by non-temporal DMA, each
// load instruction moving 1 KB of whole rows, so the cache streams as a
// plain sequential read (a non-temporal stream of half cache lines, as an
// A-operand-shaped load from memory would be, reads every line twice); the
// 16-byte chunks of each row are XOR-swizzled so that both the 16-byte K
// operand reads (16 rows, one chunk) and the transposing V reads
// (ds_read_b64_tr_b16: 8 keys, two chunks) hit distinct banks.  Each wave
// takes every 4th block of the workgroup's share with the next block always
// in flight (two stages); waves merge through LDS at the end.
constexpr int kMfmaRows = 16;  // cache rows per block

// Query heads per MFMA-decode workgroup: the largest divisor of the group
// size that is at most 16.
int decode_mfma_heads_per_wg(int group) {
    for (int h = 16; h > 1; --h)
        if (group % h == 0) return h;
    return 1;
}

typedef float mf32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
constexpr int vmcnt_only(int n) { return (n & 0xf) | ((n >> 4) << 14) | (0x7 << 4) | (0xf << 8); }
typedef short ms16x4 __attribute__((ext_vector_type(4)));

// 16-byte non-temporal buffer load of every lane into LDS at lds + 16 * lane
// (one wave; aux 2 is the nt cache policy).
__device__ __forceinline__ void dma16_lds_nt(__amdgpu_buffer_rsrc_t r, uint8_t *lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, 0, 0, 2);
}

// XOR swizzle of the 16-byte chunks of cache row r (of a 16-row block) in
// LDS: chunk c sits at slot c ^ swz(r).  D = 128 (16 chunks of a 256-byte
// row): a bijection on r, so 16 rows at one chunk fill all 64 banks, and the
// 8 rows of a transposing read pass (r & 7) differ in the upper 3 bits of
// the slot, so 8 rows x 2 adjacent chunks are 16 distinct slots.  D = 64
// (8 chunks of a 128-byte row, two rows per 256 bytes): the same properties
// within each row parity.
template <int D>
__device__ __forceinline__ int mfma_swz(int r) {
    if constexpr (D == 128) return ((r & 7) << 1) | ((r >> 3) & 1);
    else return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
}

__device__ __forceinline__ ms16x4 lds_tr16(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) ms16x4 *)p);
}

// lane l <-> lane l^16 exchange combined by max / sum (v_permlane16_swap
// pairs 16-lane rows 0-1 and 2-3)
__device__ __forceinline__ float quarter_swap_max(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quarter_swap_sum(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_mfma_kernel(
    const uint16_t *__restrict__ qp, const uint16_t *__restrict__ kcp, const uint16_t *__restrict__ vcp,
    const int64_t *__restrict__ pos, uint16_t *__restrict__ op, float *__restrict__ lsep, int heads, int kv_heads,
    int gw, int w, int g, float c2, float scale, float bias_raw, int splits, int rows_per_split,
    float *__restrict__ ws) {
    constexpr int KS = D / 32;                          // 32-wide d steps of the score product
    constexpr int DB = D / 16;                          // 16-wide column blocks of the output
    constexpr int kRowBytes = D * 2;
    constexpr int kBlockBytes = kMfmaRows * kRowBytes;  // K (or V) of one block
    constexpr int kDma = kBlockBytes / 1024;            // 1 KB DMA loads per K (or V) block
    constexpr int kWaves = kDecThreads / 64;
    // LDS: stage 0 of every wave in sbuf0, stage 1 in sbuf1 (two arrays, so
    // that the compiler sees that the reads of one stage do not alias the DMA
    // into the other and does not wait for that DMA before them); a stage of
    // a wave is its block's K then V.  sbuf0 is reused for the merge.
    constexpr int kStageBytes = 2 * kBlockBytes;
    constexpr int kBufBytes = kWaves * kStageBytes;
    constexpr int kMergeBytes = kWaves * 16 * (D + 2) * 4;
    __shared__ __attribute__((aligned(1024))) uint8_t sbuf0[kBufBytes > kMergeBytes ? kBufBytes : kMergeBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t sbuf1[kBufBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hl = lane & 15, grp = lane >> 4;
    const int split = blockIdx.x % splits;
    const int job = blockIdx.x / splits;
    const int G = heads / kv_heads;
    const int chunks = G / gw;
    const int chunk = job % chunks;
    const int kvu = job / chunks;  // batch * kv_heads + kv head
    const int b = kvu / kv_heads;
    const int h0 = (kvu % kv_heads) * G + chunk * gw;
    const int unit0 = b * heads + h0;
    const int R = g + w;
    const int64_t p = pos[b];
    const uint16_t *kc = kcp + (size_t)kvu * R * D;
    const uint16_t *vc = vcp + (size_t)kvu * R * D;

    // Q^T as the B operand: head hl, d 32 ks + 8 grp .. +8 (zero past the group)
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        uint4 x = make_uint4(0, 0, 0, 0);
        if (hl < gw) x = *reinterpret_cast<const uint4 *>(qp + (size_t)(unit0 + hl) * D + 32 * ks + 8 * grp);
        qf[ks] = __builtin_bit_cast(bf16x8, x);
    }

    // ring geometry for this query position (as in decode_kernel)
    const bool ring_full = (p >= (int64_t)w - 1);
    const int pm = (p >= 0) ? (int)(p % w) : 0;
    const int64_t win_lo = p - w + 1;

    const int r_begin = split * rows_per_split;
    const int r_end = min(R, r_begin + rows_per_split);
    const int nblk = (r_end - r_begin + kMfmaRows - 1) / kMfmaRows;

    // DMA load i of a block fills LDS bytes [1 KB i, 1 KB (i+1)) of its K (or
    // V) area: row r = byte / kRowBytes, slot (byte % kRowBytes) / 16, which
    // holds chunk slot ^ swz(r) of the row.
    uint32_t doff[kDma];
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
        const int o = 1024 * i + 16 * lane;
        const int r = o / kRowBytes, slot = (o % kRowBytes) / 16;
        doff[i] = (uint32_t)(r * kRowBytes + 16 * (slot ^ mfma_swz<D>(r)));
    }
    // K operand read (16 bytes): key hl, chunk 4 ks + grp
    const int swz_k = mfma_swz<D>(hl);
    // transposed V read: lane j of group grp supplies key 4 grp + j/4 and the
    // 8-byte piece of columns 16 db + 4 (j%4) .. +3, which is half (j%4)&1 of
    // chunk 2 db + (j%4)/2; the instruction hands lane j of the group column
    // 16 db + j of the group's four keys
    const int vr = 4 * grp + (hl >> 2);
    const int swz_v = mfma_swz<D>(vr);
    const uint32_t vrow = (uint32_t)(vr * kRowBytes + 8 * (hl & 1));
    const int vchunk = (hl >> 1) & 1;

    mf32x4 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = mf32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, negm = 0.f, l_run = 0.f;
    const float tau = 8.f / c2;

    // First cache row of block blk of this wave's share; a block past the
    // share starts at row R, past the buffer range, so its loads read zeros
    // and move no memory (the prefetch below is issued unconditionally: no
    // branch around it, hence no point where the compiler must assume either
    // history and wait for every load in flight).
    auto block_row = [&](int blk) -> int { return (blk < nblk) ? r_begin + blk * kMfmaRows : R; };
    auto stage = [&](int st) -> uint8_t * { return (st ? sbuf1 : sbuf0) + wave * kStageBytes; };
    auto load = [&](int blk, int st) {
        const int row0 = block_row(blk);
        const uint32_t range = (uint32_t)(R - row0) * kRowBytes;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kc + (size_t)row0 * D, range);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vc + (size_t)row0 * D, range);
        uint8_t *dst = stage(st);
#pragma unroll
        for (int i = 0; i < kDma; ++i) dma16_lds_nt(rk, dst + 1024 * i, doff[i]);
#pragma unroll
        for (int i = 0; i < kDma; ++i) dma16_lds_nt(rv, dst + kBlockBytes + 1024 * i, doff[i]);
    };
    // one block: scores, mask, softmax, O^T += V^T P^T
    auto compute = [&](int blk, int st) {
        const int row0 = r_begin + blk * kMfmaRows;
        const uint8_t *kb = stage(st);
        const uint8_t *vb = kb + kBlockBytes;
        mf32x4 sc = mf32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kb + hl * kRowBytes + 16 * ((4 * ks + grp) ^ swz_k));
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], sc, 0, 0, 0);
        }
        // lane (hl, grp) holds keys 4 grp + i of the block: which position
        // each row holds and whether it is read (as in decode_kernel)
        float mx = kNegInf;
        uint32_t vkeep[2] = {0xffffffffu, 0xffffffffu};  // per 2 key slots
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = row0 + 4 * grp + i;
            const int sl = r - g;
            int dd = pm - sl;
            dd += (dd < 0) ? w : 0;
            const int64_t t = (r < g) ? (int64_t)r : (ring_full ? p - dd : (int64_t)sl);
            const bool v_sink = ((int64_t)r <= p) && ((int64_t)r < win_lo);
            const bool v_ring = ring_full || ((int64_t)sl <= p);
            const bool valid = (r < r_end) && (p >= 0) && ((r < g) ? v_sink : v_ring);
            const float x = sc[i] + ((t < g) ? bias_raw : 0.f);
            sc[i] = valid ? x : kNegInf;
            mx = fmaxf(mx, sc[i]);
            if (!valid) vkeep[i >> 1] &= (i & 1) ? 0x0000ffffu : 0xffff0000u;
        }
        // a row that is not read may hold anything (an unwritten slot): its
        // P is 0 and, where such rows occur, its V values are zeroed too, so
        // that 0 * NaN cannot reach the output
        const bool any_unread = __any((vkeep[0] & vkeep[1]) != 0xffffffffu);
        mx = half_swap_max(quarter_swap_max(mx));  // over the head's 4 lanes
        if (__any(mx > m_run + tau)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_run - m_new) * c2);
            m_run = m_new;
            negm = (m_new == kNegInf) ? 0.f : -m_new * c2;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        }
        // P^T as the B operand: keys 4 grp + i
        const bf16x2 p01 = {static_cast<__bf16>(fast_exp2(fmaf(sc[0], c2, negm))),
                            static_cast<__bf16>(fast_exp2(fmaf(sc[1], c2, negm)))};
        const bf16x2 p23 = {static_cast<__bf16>(fast_exp2(fmaf(sc[2], c2, negm))),
                            static_cast<__bf16>(fast_exp2(fmaf(sc[3], c2, negm)))};
        {
            const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
            const float ls = __builtin_amdgcn_fdot2_f32_bf16(p01, ones, 0.f, false);
            l_run += __builtin_amdgcn_fdot2_f32_bf16(p23, ones, ls, false);
        }
        const ms16x4 pk = __builtin_bit_cast(
            ms16x4, make_uint2(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)));
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            ms16x4 vf = lds_tr16(vb + vrow + 16 * ((2 * db + vchunk) ^ swz_v));
            if (any_unread) {
                uint2 u = __builtin_bit_cast(uint2, vf);
                u.x &= vkeep[0];
                u.y &= vkeep[1];
                vf = __builtin_bit_cast(ms16x4, u);
            }
            oacc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pk, oacc[db], 0, 0, 0);
        }
    };

    // this wave's blocks wave, wave + 4, ...: the next one always in flight
    // while one is computed, stages 0 and 1 alternating (the loop is
    // unrolled by two so that each stage is named statically)
    const int my_blocks = (nblk > wave) ? (nblk - wave + kWaves - 1) / kWaves : 0;
    if (my_blocks > 0) {
        load(wave, 0);
        // (sched_barrier: the next block's loads all issue before the wait)
        for (int it = 0;; it += 2) {
            const int blk = wave + it * kWaves;
            load(blk + kWaves, 1);  // an empty block past the share's end
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kDma));  // block it has landed
            compute(blk, 0);
            if (it + 1 >= my_blocks) break;
            load(blk + 2 * kWaves, 0);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_only(2 * kDma));  // block it + 1 has landed
            compute(blk + kWaves, 1);
            if (it + 2 >= my_blocks) break;
        }
    }
    // the last prefetch (an empty block) writes LDS: done before the merge reuses it
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));

    // ---- merge the waves: per head h, (m, l, o[D]) of each wave ----
    const float l_head = half_swap_sum(quarter_swap_sum(l_run));
    __syncthreads();  // every wave is done with its stages
    float *sm = reinterpret_cast<float *>(sbuf0);  // [wave][head][D + 2]: o[D], m, l
    {
        float *rec = sm + (wave * 16 + hl) * (D + 2);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) rec[16 * db + 4 * grp + i] = oacc[db][i];
        if (grp == 0) {
            rec[D] = m_run;
            rec[D + 1] = l_head;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < gw * D; idx += kDecThreads) {
        const int h = idx / D, c = idx - h * D;
        float M = kNegInf;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) M = fmaxf(M, sm[(wv * 16 + h) * (D + 2) + D]);
        const float M_use = (M == kNegInf) ? 0.f : M;
        float L = 0.f, acc = 0.f;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) {
            const float *rec = sm + (wv * 16 + h) * (D + 2);
            const float f = fast_exp2((rec[D] - M_use) * c2);
            L += rec[D + 1] * f;
            acc += rec[c] * f;
        }
        const int unit = unit0 + h;
        if (splits == 1) {
            const float x = (L > 0.f) ? acc / L : __builtin_nanf("");
            op[(size_t)unit * D + c] = (uint16_t)f32_to_bf16_bits(x);
            if (lsep != nullptr && c == 0) lsep[unit] = (L > 0.f) ? M * scale + logf(L) : __builtin_nanf("");
        } else {
            float *rec = ws + ((size_t)unit * splits + split) * (2 + D);
            rec[2 + c] = acc;
            if (c == 0) {
                rec[0] = M;
                rec[1] = L;
            }
        }
    }
}

// Merge S partial states of one (batch, head) by log-sum-exp.
template <typename QT, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float *__restrict__ ws, void *__restrict__ op,
                                                         float *__restrict__ lsep, int splits, float c2,
                                                         float scale) {
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
    QT *out = reinterpret_cast<QT *>(op) + (size_t)unit * D;
    if constexpr (std::is_same<QT, uint16_t>::value)
        out[c] = (uint16_t)f32_to_bf16_bits(x);
    else
        out[c] = x;
    if (lsep != nullptr && c == 0) lsep[unit] = (L > 0.f) ? M * scale + logf(L) : __builtin_nanf("");
}

// Query heads per decode workgroup: the largest power of two <= cap that
// divides the group size (query heads per key/value head).  fp8 caches cap
// it at 4 (twice the rows in flight per lane leave registers for 4 heads).
int decode_heads_per_wg(int group, int cap) {
    int gq = 1;
    while (gq < cap && group % (2 * gq) == 0) gq *= 2;
    return gq;
}

template <typename CK>
constexpr int heads_cap() { return std::is_same<CK, CacheFp8>::value ? 4 : 8; }

// Split count: enough workgroups to cover the chip, at least 256 cache rows
// each.  The VALU kernels aim at 2048 workgroups; the MFMA kernel (two
// workgroups per CU by LDS) at one round of 512, which measured 2 % faster on
// 64 x 8 key/value heads than two splits and 7 % faster than four.
int decode_splits(int jobs, int rows, int kind) {
    const int target = (kind == 2) ? 512 : 2048;
    if (jobs >= ((kind == 2) ? 512 : 1024)) return 1;
    int s = (target + jobs - 1) / jobs;
    int max_s = rows / 256;
    if (max_s < 1) max_s = 1;
    if (s > max_s) s = max_s;
    if (s > 64) s = 64;
    return s < 1 ? 1 : s;
}

// Workgroups before splitting: batch * heads / (query heads per
// workgroup).  kind: 0 the VALU kernel (up to 8 heads per workgroup), 1 the
// fp8 VALU kernel (up to 4), 2 the MFMA kernel (up to 16; bf16 groups of 2+).
static int decode_jobs(int batch, int heads, int kv_heads, int kind) {
    if (kind == 2) return batch * (heads / decode_mfma_heads_per_wg(heads / kv_heads));
    return batch * (heads / decode_heads_per_wg(heads / kv_heads, kind == 1 ? 4 : 8));
}

// Which kernel a launch uses.
int decode_kind(bool bf16, bool fp8, int heads, int kv_heads) {
    if (fp8) return 1;
    return (bf16 && heads / kv_heads >= 2) ? 2 : 0;
}

// Workspace of a launch of this kind (0 when it does not split); kind -1:
// the most any kind needs (fewest workgroups, most splits).
size_t decode_workspace_bytes(int batch, int heads, int kv_heads, int d, int rows, int kind) {
    if (kind < 0) {
        size_t m = 0;
        for (int k = 0; k < 3; ++k) {
            const size_t b = decode_workspace_bytes(batch, heads, kv_heads, d, rows, k);
            if (b > m) m = b;
        }
        return m;
    }
    int s = decode_splits(decode_jobs(batch, heads, kv_heads, kind), rows, kind);
    if (s == 1) return 0;
    return (size_t)batch * heads * s * (2 + d) * sizeof(float);
}

template <typename QT, typename CK, int D, int GQ>
static hipError_t launch_decode_t(const void *q, const void *kc, const void *vc, const int64_t *pos, void *o,
                                  float *lse, int batch, int heads, int kv_heads, int w, int g, float scale,
                                  float sink_bias, void *ws, const float *ksc, const float *vsc,
                                  hipStream_t stream) {
    const int R = g + w;
    const int kind = is_fp8<CK>() ? 1 : 0;
    const int jobs = decode_jobs(batch, heads, kv_heads, kind);
    const int splits = decode_splits(jobs, R, kind);
    const int rps = (R + splits - 1) / splits;
    const float c2 = (float)((double)scale * kLog2e);
    const float bias_raw = (float)((double)sink_bias / (double)scale);
    hipLaunchKernelGGL((decode_kernel<QT, CK, D, GQ>), dim3(jobs * splits), dim3(kDecThreads), 0, stream, q, kc,
                       vc, pos, o, lse, heads, kv_heads, w, g, c2, scale, bias_raw, splits, rps, (float *)ws, ksc,
                       vsc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    hipLaunchKernelGGL((decode_merge_kernel<QT, D>), dim3(batch * heads), dim3(D), 0, stream, (const float *)ws, o,
                       lse, splits, c2, scale);
    return hipGetLastError();
}

template <typename QT, typename CK, int D>
static hipError_t launch_decode_d(const void *q, const void *kc, const void *vc, const int64_t *pos, void *o,
                                  float *lse, int batch, int heads, int kv_heads, int w, int g, float scale,
                                  float sink_bias, void *ws, const float *ksc, const float *vsc,
                                  hipStream_t stream) {
#define SWA_DEC(GQ)                                                                                              \
    launch_decode_t<QT, CK, D, GQ>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale, sink_bias, ws, \
                                   ksc, vsc, stream)
    switch (decode_heads_per_wg(heads / kv_heads, heads_cap<CK>())) {
        case 8:
            if constexpr (heads_cap<CK>() >= 8) return SWA_DEC(8);
            return hipErrorInvalidValue;
        case 4: return SWA_DEC(4);
        case 2: return SWA_DEC(2);
        default:
            if constexpr (std::is_same<CK, CacheFp8>::value && D == 128)
                return launch_decode_t<QT, CacheFp8W, D, 1>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g,
                                                            scale, sink_bias, ws, ksc, vsc, stream);
            return SWA_DEC(1);
    }
#undef SWA_DEC
}

template <int D>
static hipError_t launch_decode_mfma(const void *q, const void *kc, const void *vc, const int64_t *pos, void *o,
                                    float *lse, int batch, int heads, int kv_heads, int w, int g, float scale,
                                    float sink_bias, void *ws, hipStream_t stream) {
    const int R = g + w;
    const int gw = decode_mfma_heads_per_wg(heads / kv_heads);
    const int jobs = decode_jobs(batch, heads, kv_heads, 2);
    const int splits = decode_splits(jobs, R, 2);
    const int rps = (R + splits - 1) / splits;
    const float c2 = (float)((double)scale * kLog2e);
    const float bias_raw = (float)((double)sink_bias / (double)scale);
    hipLaunchKernelGGL((decode_mfma_kernel<D>), dim3(jobs * splits), dim3(kDecThreads), 0, stream,
                       (const uint16_t *)q, (const uint16_t *)kc, (const uint16_t *)vc, pos, (uint16_t *)o, lse, heads,
                       kv_heads, gw, w, g, c2, scale, bias_raw, splits, rps, (float *)ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    hipLaunchKernelGGL((decode_merge_kernel<uint16_t, D>), dim3(batch * heads), dim3(D), 0, stream,
                       (const float *)ws, o, lse, splits, c2, scale);
    return hipGetLastError();
}

hipError_t launch_decode(const void *q, const void *kc, const void *vc, const int64_t *pos, void *o, float *lse,
                         int batch, int heads, int kv_heads, int d, int w, int g, float scale, float sink_bias,
                         bool bf16, void *ws, hipStream_t stream) {
    if (decode_kind(bf16, false, heads, kv_heads) == 2) {
        if (d == 128)
            return launch_decode_mfma<128>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale, sink_bias,
                                           ws, stream);
        return launch_decode_mfma<64>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale, sink_bias, ws,
                                      stream);
    }
    if (bf16) {
        if (d == 128)
            return launch_decode_d<uint16_t, CacheBf16, 128>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g,
                                                             scale, sink_bias, ws, nullptr, nullptr, stream);
        return launch_decode_d<uint16_t, CacheBf16, 64>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale,
                                                        sink_bias, ws, nullptr, nullptr, stream);
    }
    if (d == 128)
        return launch_decode_d<float, CacheF32, 128>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale,
                                                     sink_bias, ws, nullptr, nullptr, stream);
    return launch_decode_d<float, CacheF32, 64>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale,
                                                sink_bias, ws, nullptr, nullptr, stream);
}

// fp8 (E4M3) caches with per-(batch, key/value head) scales; q and o bf16 or fp32.
hipError_t launch_decode_fp8(const void *q, const void *kc, const void *vc, const float *ksc, const float *vsc,
                             const int64_t *pos, void *o, float *lse, int batch, int heads, int kv_heads, int d,
                             int w, int g, float scale, float sink_bias, bool bf16, void *ws, hipStream_t stream) {
    if (bf16) {
        if (d == 128)
            return launch_decode_d<uint16_t, CacheFp8, 128>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g,
                                                            scale, sink_bias, ws, ksc, vsc, stream);
        return launch_decode_d<uint16_t, CacheFp8, 64>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale,
                                                       sink_bias, ws, ksc, vsc, stream);
    }
    if (d == 128)
        return launch_decode_d<float, CacheFp8, 128>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale,
                                                     sink_bias, ws, ksc, vsc, stream);
    return launch_decode_d<float, CacheFp8, 64>(q, kc, vc, pos, o, lse, batch, heads, kv_heads, w, g, scale,
                                                sink_bias, ws, ksc, vsc, stream);
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
    // no valid position (a negative one, or one whose last token would pass
    // INT64_MAX and wrap to a negative ring row): the batch entry is a no-op
    if (P0 < 0 || P0 > INT64_MAX - tn) return;
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

// ---------------------------------------------------------------------------
// fp8 cache append.  E4M3 in its OCP form ("Sliding Window and Sparse
// Attention, from Longformer to CSA2", s10 glossary, E4M3: 1 sign, 4
// exponent, 3 mantissa bits; exponent bias 7, no infinities, S.1111.111 is
// NaN, largest finite 448).  A value x of key/value head (b, h) is stored as
// the code of y = x / scale[b][h] (fp32 division, correctly rounded), y
// rounded to the nearest code with ties to even mantissa and |y| >= 448
// saturated to 448; NaN stays NaN.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t bits = __float_as_uint(y);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const uint32_t a = bits & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;  // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;  // |y| >= 448 (and infinity): saturate
    if (a < 0x3c800000u) {                      // |y| < 2^-6: multiples of 2^-9
        const float m = __builtin_rintf(__uint_as_float(a) * 512.f);  // exact scaling, then ties to even
        return sign | (uint32_t)m;              // m = 8 is the smallest normal's code
    }
    // keep 3 mantissa bits, ties to even (a carry moves into the exponent),
    // then rebias the exponent from 127 to 7
    const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    return sign | ((r >> 20) - (120u << 3));
}

// One thread quantises 8 consecutive elements of one K row and one V row
// and writes them where kv_append_kernel would write the bf16/fp32 row.
template <bool BF16>
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(uint8_t *__restrict__ kc, uint8_t *__restrict__ vc,
                                                            const void *__restrict__ kn, const void *__restrict__ vn,
                                                            const int64_t *__restrict__ pos,
                                                            const float *__restrict__ ksc,
                                                            const float *__restrict__ vsc, int heads, int tn, int d,
                                                            int w, int g, long long total) {
    const long long id = (long long)blockIdx.x * 256 + threadIdx.x;
    if (id >= total) return;
    const int cpr = d / 8;  // 8-element pieces per row
    const int piece = (int)(id % cpr);
    const long long rowid = id / cpr;
    const int j = (int)(rowid % tn);
    const long long unit = rowid / tn;  // batch * heads + head
    const int b = (int)(unit / heads);
    const int64_t P0 = pos[b];
    // no valid position (a negative one, or one whose last token would pass
    // INT64_MAX and wrap to a negative ring row): the batch entry is a no-op
    if (P0 < 0 || P0 > INT64_MAX - tn) return;
    const int64_t P = P0 + j;
    const size_t src = ((size_t)unit * tn + j) * d + (size_t)piece * 8;  // element index
    float xk[8], xv[8];
    if constexpr (BF16) {
        const uint4 a = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(kn) + src);
        const uint4 c = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(vn) + src);
        const uint32_t ua[4] = {a.x, a.y, a.z, a.w}, uc[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xk[2 * i] = bf16lo(ua[i]);
            xk[2 * i + 1] = bf16hi(ua[i]);
            xv[2 * i] = bf16lo(uc[i]);
            xv[2 * i + 1] = bf16hi(uc[i]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i += 4) {
            const float4 a = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(kn) + src + i);
            const float4 c = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(vn) + src + i);
            xk[i] = a.x; xk[i + 1] = a.y; xk[i + 2] = a.z; xk[i + 3] = a.w;
            xv[i] = c.x; xv[i + 1] = c.y; xv[i + 2] = c.z; xv[i + 3] = c.w;
        }
    }
    const float sk = ksc[unit], sv = vsc[unit];
    uint32_t k8[2] = {0, 0}, v8[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        k8[i >> 2] |= e4m3_code(__fdiv_rn(xk[i], sk)) << (8 * (i & 3));
        v8[i >> 2] |= e4m3_code(__fdiv_rn(xv[i], sv)) << (8 * (i & 3));
    }
    const uint2 kk = make_uint2(k8[0], k8[1]), vv = make_uint2(v8[0], v8[1]);
    const size_t cache_base = (size_t)unit * (g + w) * d + (size_t)piece * 8;
    if (j >= tn - w) {
        const size_t dst = cache_base + (size_t)(g + (int)(P % w)) * d;
        *reinterpret_cast<uint2 *>(kc + dst) = kk;
        *reinterpret_cast<uint2 *>(vc + dst) = vv;
    }
    if (P < g) {
        const size_t dst = cache_base + (size_t)P * d;
        *reinterpret_cast<uint2 *>(kc + dst) = kk;
        *reinterpret_cast<uint2 *>(vc + dst) = vv;
    }
}

hipError_t launch_kv_append_fp8(void *kc, void *vc, const void *kn, const void *vn, const int64_t *pos,
                                const float *ksc, const float *vsc, int batch, int heads, int tn, int d, int w,
                                int g, bool bf16, hipStream_t stream) {
    const long long total = (long long)batch * heads * tn * (d / 8);
    const long long blocks = (total + 255) / 256;
    if (bf16)
        hipLaunchKernelGGL(kv_append_fp8_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, (uint8_t *)kc,
                           (uint8_t *)vc, kn, vn, pos, ksc, vsc, heads, tn, d, w, g, total);
    else
        hipLaunchKernelGGL(kv_append_fp8_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, (uint8_t *)kc,
                           (uint8_t *)vc, kn, vn, pos, ksc, vsc, heads, tn, d, w, g, total);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fixed device scratch for the decode entry point that allocates nothing: the
// split decode's partial (m, l, o) records go here instead of into a
// caller-supplied workspace.  Every device the library runs on holds its own
// copy until the process ends; calls that overlap on one device share it and
// race.  The kernels overwrite every record they later read, so nothing in it
// needs clearing between calls.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

size_t decode_scratch_bytes() { return kDecodeScratchBytes; }

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

// Device address of `scratch` on the device that owns `stream`, looked up once
// per device with that device current (the host-side name of the array is
// only a stand-in and is never passed to a kernel).
static hipError_t decode_scratch_address(hipStream_t stream, void **out) {
    int dev = -1;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// launch_decode with the partial records in the fixed scratch (the caller has
// checked that the launch needs at most kDecodeScratchBytes).
hipError_t launch_decode_noalloc(const void *q, const void *kc, const void *vc, const int64_t *pos, void *o,
                                 float *lse, int batch, int heads, int kv_heads, int d, int w, int g, float scale,
                                 float sink_bias, bool bf16, hipStream_t stream) {
    void *ws = nullptr;
    const hipError_t e = decode_scratch_address(stream, &ws);
    if (e != hipSuccess) return e;
    return launch_decode(q, kc, vc, pos, o, lse, batch, heads, kv_heads, d, w, g, scale, sink_bias, bf16, ws,
                         stream);
}

}  // namespace swa
