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
//      S^T = K Q^T    (A = K tile from LDS, B = the wave's Q held in VGPRs)
//      O^T += V^T P^T (A = V tile from LDS read transposed, B = P in VGPRs)
//    Computing the transposes makes the MFMA result layout put one query row
//    per lane (lanes l and l+32 share a row), so the online-softmax row max
//    and row sum are in-register reductions plus one permlane32 swap, the
//    probabilities P feed the second MFMA straight from the first one's
//    accumulators, and the output rescale needs no cross-lane traffic;
//  * tiles that the window edge, a sink or the end of the sequence cuts are
//    masked pair by pair (excluded scores -> -inf); the run of FULL tiles in
//    between skips masking in a loop of its own;
//  * scores stay in raw q.k units; exp2 with scale*log2(e) folded into one
//    FMA per score.  The reference max only moves when a score exceeds it by
//    more than 2^8 in probability, so the O rescale is rare.  A row with no
//    attended key yet keeps m = -inf and is guarded so that no -inf - -inf is
//    ever formed.  FULL tiles do not even take the row max first: their
//    probabilities are formed against the current reference, and only when
//    some lane's bf16 sum of them reaches 2^7 (a superset of the cases that
//    move the reference) is the exact update run and the tile's
//    probabilities formed again, so the result is the same bit for bit.
//
// bf16 path: K and V tiles go HBM -> LDS by buffer loads that write LDS
// directly (16 bytes per lane, out-of-range rows come back as zeros), so no
// VGPRs stage them.  K is stored in 64-byte column blocks with an XOR swizzle
// of its 16-byte chunks so that the 32 rows one MFMA operand read touches hit
// distinct banks; V is stored row-major and its transposed MFMA operand is
// read with ds_read_b64_tr_b16 (each 16-lane group of that instruction
// transposes 4x4 blocks of 16-bit values across lanes).
// fp32 path: tiles are staged through VGPRs and V is transposed on the way
// into LDS; it exists for fp32 parity, not for speed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.h"
#include "schedule.h"

namespace swa {

constexpr int kBK = 64;        // keys per tile (2 MFMA sub-blocks of 32)
constexpr int kBQ = 128;       // fp32 path: query rows per workgroup (4 waves x 32)
constexpr int kThreads = 256;  // fp32 path: threads per workgroup
constexpr int kWaves16 = 4;    // bf16 path: waves per workgroup (4 x 32 = 128 query rows)

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define SWA_LDS __attribute__((address_space(3)))

// 16-byte buffer load of every lane into LDS at lds + 16 * lane (one wave).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t *lds, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SWA_LDS void *)lds, 16, voff, 0, 0, 0);
}
// ds_read_b64_tr_b16 at an LDS address.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((SWA_LDS s16x4 *)p);
}

// Element offset of the key/value rows that query unit (batch * heads + head)
// reads: grouped-query attention maps heads / kv_heads consecutive query heads
// onto one key/value head (kv_heads == heads is plain multi-head attention).
__device__ __forceinline__ size_t kv_offset(int unit, int heads, int kv_heads, int n, int d) {
    const int b = unit / heads, h = unit - b * heads;
    return ((size_t)b * kv_heads + h / (heads / kv_heads)) * n * d;
}

// Chunked prefill against the rolling cache: the queries of a chunk are the
// positions p0 .. p0+T-1 of batch entry b (p0 = pos[b]); a key position s >=
// p0 is row s-p0 of the chunk's own K/V, a key position s < p0 is in the
// cache: ring row g + s mod w while s >= p0-w (the ring still holds it), else
// sink row s ("Sliding Window and Sparse Attention, from Longformer to CSA2",
// s2: rolling buffer, sinks; "Local and Sparse Attention: Reading Fewer Token
// Positions", Figure 4: circular overwrite, kept anchors).  Positions that are
// neither were evicted and are never attended; their loads land on some
// finite cache row or read as zero past the cache and are masked.
// part: 0 = every key, 1 = cache keys only (s < p0), 2 = chunk keys only.
//
// Strided fixed patterns on the same tiles ("Sliding Window and Sparse
// Attention, from Longformer to CSA2", s2 dilated windows and s4 block-sparse
// substrate; "Local and Sparse Attention: Reading Fewer Token Positions",
// Figure 2 landmarks):
//  * dilated (mode 1): query i reads keys i, i-r, ..., i-(w-1)r.  The rows of
//    one residue class c = i mod r form an ordinary causal window of w over
//    the subsequence c, c+r, c+2r, ...: the grid runs one unit per (batch,
//    head, class) on rows strided by r, with class-local positions.
//  * landmark part (mode 2): query i reads the landmarks j = k r that lie
//    below its window and are not sinks (g <= j <= i-w); over the K/V rows
//    strided by r that is the compact index range ceil(g/r) <= k <=
//    floor((i-w)/r).  The fp32 path runs it as a launch of its own and merges
//    it with the window-and-sinks launch by LSE.
//  * landmarks in one pass (kLandmark, bf16): each query block first streams
//    the tiles of that compact landmark range (K/V rows strided by r) and then
//    its window-and-sink tiles, all through one online softmax, so the union
//    of the three key sets is attended in a single launch.
enum { kPlain = 0, kChunk = 1, kStrided = 2, kLandmark = 3 };
struct PathArgs {
    const void *kc;        // chunk: K cache [batch][kv_heads][g + w][d]
    const void *vc;        // chunk: V cache, same layout
    const int64_t *pos;    // chunk: p0 of each batch entry
    int part;              // chunk: which keys
    int r;                 // strided, landmarks: the stride
    int mode;              // strided: 1 dilated, 2 landmark part
};
constexpr int kNoWindow = 1 << 30;  // a window wider than any sequence
// Chunk positions are accepted while pos + t stays this far below INT_MAX, so
// that every position sum of the tile arithmetic (a block's last row, a
// tile's last key, the next tile's first) is an int.
constexpr int kPosHeadroom = 1024;

// Byte offset of row `row` of a buffer of n rows, the row index formed in 64
// bits and clamped to n: a row at or past n reads as zero through the buffer
// range check, and no stride product can wrap round 2^32 back into range
// (n rows plus any 16-byte chunk of a row fit in 32 bits, n * row_bytes being
// below 2^32).
__device__ __forceinline__ uint32_t row_off(uint64_t row, int n, uint32_t row_bytes) {
    return (uint32_t)(row < (uint64_t)n ? row : (uint64_t)n) * row_bytes;
}

// Cache row of key position s < p0 (s >= 0).
__device__ __forceinline__ int cache_row(int s, int p0, int w, int g) {
    return (s >= p0 - w) ? g + s % w : s;
}

// ---------------------------------------------------------------------------
// Pieces shared by both paths.  s[sb][r] holds q_qi . k_j for the key
// j = k0 + 32 sb + 8 (r/4) + 4 lh + r%4 (the 32x32 MFMA result layout).

// Exact predicate on a cut tile.  A tile whose keys are all >= g and < n is
// cut only by the window and causality: 0 <= qi - j < w, one unsigned compare
// per score.  Tiles with sink keys or past the end of the sequence take the
// full predicate and the sink bias.  KLO: keys below klo are excluded too
// (a partial attention over the keys >= klo only).
template <bool KLO = false>
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int qi, int k0, int lh, int n, int w, int g,
                                          float bias_raw, int klo = 0) {
    if (k0 >= g && k0 + kBK <= n && (!KLO || k0 >= klo)) {
        const int diff = qi - k0 - 4 * lh;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dd = diff - (32 * sb + 8 * (r >> 2) + (r & 3));
                s[sb][r] = ((unsigned)dd < (unsigned)w) ? s[sb][r] : kNegInf;
            }
        return;
    }
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = k0 + 32 * sb + 8 * (r >> 2) + 4 * lh + (r & 3);
            const float x = s[sb][r] + (j < g ? bias_raw : 0.f);
            s[sb][r] = (pair_attended(qi, j, n, w, g) && (!KLO || j >= klo)) ? x : kNegInf;
        }
}

// Landmark tile of the single-pass landmark kernel: compact landmark index j
// (key row j r) is read by a row iff lk_lo <= j <= lq, lq being the row's last
// landmark below its window (-1 when it has none); landmarks are >= g, so no
// sink bias.
__device__ __forceinline__ void mask_landmark_tile(f32x16 (&s)[2], int lq, int k0, int lh, int lk_lo) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = k0 + 32 * sb + 8 * (r >> 2) + 4 * lh + (r & 3);
            s[sb][r] = (j >= lk_lo && j <= lq) ? s[sb][r] : kNegInf;
        }
}

// Row max of the tile; moves the reference max (and rescales O and l) only
// when some row of the wave would otherwise see a probability above 2^8.
template <int NACC>
__device__ __forceinline__ void update_max(const f32x16 (&s)[2], float &m_run, float &negm, float &l_run,
                                           f32x16 (&oacc)[NACC], float c2, float tau) {
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
        for (int cb = 0; cb < NACC; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[cb][r] *= alpha;
    }
}

// Normalise and store O (and LSE) of this lane's query row.
// Query row qi is row qi * rs of O and of lse.
template <typename T, int D>
__device__ __forceinline__ void store_rows(const f32x16 (&oacc)[D / 32], float m_run, float l_run, int qi, int n,
                                           int lh, T *O, float *lse, float scale, int rs = 1) {
    const float l_tot = half_swap_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
    if (qi >= n) return;
    T *orow = O + (size_t)qi * rs * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int c = 32 * cb + 8 * gq + 4 * lh;
            const float x0 = oacc[cb][4 * gq + 0] * inv, x1 = oacc[cb][4 * gq + 1] * inv;
            const float x2 = oacc[cb][4 * gq + 2] * inv, x3 = oacc[cb][4 * gq + 3] * inv;
            if constexpr (std::is_same<T, uint16_t>::value) {
                *reinterpret_cast<uint2 *>(orow + c) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
            } else {
                *reinterpret_cast<float4 *>(orow + c) = make_float4(x0, x1, x2, x3);
            }
        }
    if (lse != nullptr && lh == 0) lse[(size_t)qi * rs] = m_run * scale + logf(l_tot);
}


// bf16 output of one wave through LDS: the wave's 32 rows are written into
// its own 32 * 2D-byte region (16-byte chunk k of row r at chunk position
// k ^ (r % (2D/16)), so that the 32 rows of one column do not share banks),
// then read back row by row, 16 bytes per lane, and stored as whole rows
// (2D/16 lanes per row).  The region is LDS no other wave touches; a wave's
// own LDS writes and reads are ordered.
template <int D>
__device__ __forceinline__ void store_rows_lds(const f32x16 (&oacc)[D / 32], float m_run, float l_run, int qw0, int nq,
                                               int lr, int lh, int lane, uint16_t *O, float *lse, float scale,
                                               int rs, uint8_t *region) {
    constexpr int RB = 2 * D;      // bytes per row
    constexpr int CPR = RB / 16;   // 16-byte chunks per row
    const float l_tot = half_swap_sum(l_run);
    const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            // columns 32 cb + 8 gq + 4 lh .. +3: chunk 4 cb + gq, byte 8 lh in it
            const int ch = 4 * cb + gq;
            const float x0 = oacc[cb][4 * gq + 0] * inv, x1 = oacc[cb][4 * gq + 1] * inv;
            const float x2 = oacc[cb][4 * gq + 2] * inv, x3 = oacc[cb][4 * gq + 3] * inv;
            *reinterpret_cast<uint2 *>(region + lr * RB + ((ch ^ (lr % CPR)) * 16) + 8 * lh) =
                make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
        }
#pragma unroll
    for (int j = 0; j < 32 * CPR / 64; ++j) {
        const int idx = 64 * j + lane;
        const int r = idx / CPR, ch = idx % CPR;
        const uint4 v = *reinterpret_cast<const uint4 *>(region + r * RB + ((ch ^ (r % CPR)) * 16));
        if (qw0 + r < nq) *reinterpret_cast<uint4 *>(O + (size_t)(qw0 + r) * rs * D + 8 * ch) = v;
    }
    const int qi = qw0 + lr;
    if (lse != nullptr && lh == 0 && qi < nq) lse[(size_t)qi * rs] = m_run * scale + logf(l_tot);
}

// ---------------------------------------------------------------------------
// bf16 path.
template <int D, int WAVES>
struct Bf16Tile {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kTileBytes = kBK * kRowBytes;             // one K or V tile
    static constexpr int kStageBytes = 2 * kTileBytes;             // K then V
    static constexpr int kDmaPerWave = kTileBytes / 1024 / WAVES;  // 1 KB DMA loads per wave per tile
    static_assert(kTileBytes % (1024 * WAVES) == 0, "tile split over the waves");
    // LDS byte offset of K(key, 16-byte chunk c): 64-byte column block c/4,
    // 64 bytes per key inside it, chunk position (c%4) ^ ((key/4)%4).
    __device__ static constexpr uint32_t k_off(int key, int c) {
        return (uint32_t)((c >> 2) * (kBK * 64) + key * 64 + 16 * ((c & 3) ^ ((key >> 2) & 3)));
    }
    // V(key, 8-byte piece p of 4 columns): same column blocks, no swizzle.
    __device__ static constexpr uint32_t v_off(int key, int p) {
        return (uint32_t)((p >> 3) * (kBK * 64) + key * 64 + 8 * (p & 7));
    }
};

// KIND kChunk: the queries are a chunk of n positions starting at p0 =
// pos[b] and the keys come from the chunk and the cache; kStrided: a strided
// pattern (PathArgs); kLandmark: window, sinks and landmarks every ca.r in one
// pass; kPlain: q, k, v are whole sequences of n positions.
template <int D, int WAVES, int KIND>
__global__ __launch_bounds__(64 * WAVES, 8 / WAVES) void prefill_bf16_kernel(
    const uint16_t *__restrict__ qp, const uint16_t *__restrict__ kp, const uint16_t *__restrict__ vp,
    uint16_t *__restrict__ op, float *__restrict__ lsep, int n, int nqb, int w, int g, float c2, float scale,
    float bias_raw, int total_wg, int heads, int kv_heads, PathArgs ca) {
    constexpr bool CHUNK = (KIND == kChunk), STRIDED = (KIND == kStrided), LAND = (KIND == kLandmark);
    using L = Bf16Tile<D, WAVES>;
    constexpr int BQ = 32 * WAVES;
    // two K and two V tile buffers, as four arrays: the compiler can then see
    // that the LDS reads of one buffer do not alias the DMA into another and
    // does not wait for that DMA before them
    __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[L::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[L::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[L::kTileBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[L::kTileBytes];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 31;  // query row of this lane within the wave
    const int lh = lane >> 5;  // which half of the wave

    int unit, qb;
    // the query heads of one key/value head take each query block together
    // (strided launches interleave residue classes in their units: no grouping)
    workgroup_order(blockIdx.x, total_wg, nqb, STRIDED ? 1 : heads / kv_heads, &unit, &qb);
    // strided patterns: query row i of this unit is row oq + i sq of q and o,
    // key index k is row okv + k skv of k and v; nq query rows
    int nq = n, sq = 1, oq = 0, skv = 1, okv = 0;
    if constexpr (STRIDED) {
        if (ca.mode == 1) {
            const int cls = unit % ca.r;
            unit /= ca.r;
            nq = (n - cls + ca.r - 1) / ca.r;
            sq = ca.r;
            oq = cls;
            okv = cls;
        }
        skv = ca.r;
    }
    const size_t base = (size_t)unit * n * D;  // q and o of (batch, head)
    const uint16_t *Q = qp + base;
    const uint16_t *K = kp + kv_offset(unit, heads, kv_heads, n, D);
    const uint16_t *V = vp + kv_offset(unit, heads, kv_heads, n, D);

    const int q0 = qb * BQ;  // rows of this block: q0 .. q1 (< nq)
    const int q1 = min(q0 + BQ, nq) - 1;
    const int qi = q0 + wave * 32 + lr;
    if (STRIDED && q0 >= nq) return;  // a residue class shorter than the longest one
    // positions: query row r is at p0 + r; keys are attended in [klo, khi)
    int p0 = 0, klo = 0, khi = n, wq = w;
    const uint16_t *KC = nullptr, *VC = nullptr;
    if constexpr (CHUNK) {
        const int b = unit / heads;
        const int64_t pb = ca.pos[b];
        if (pb < 0 || pb > (int64_t)(0x7fffffff - kPosHeadroom - n)) {
            // no valid position: the rows are NaN
            if (qi < n) {
                uint16_t *orow = op + base + (size_t)qi * D;
                for (int c = 4 * lh; c < D; c += 8)
                    *reinterpret_cast<uint2 *>(orow + c) = make_uint2(0x7fc07fc0u, 0x7fc07fc0u);
                if (lsep != nullptr && lh == 0) lsep[(size_t)unit * n + qi] = __builtin_nanf("");
            }
            return;
        }
        p0 = (int)pb;
        klo = (ca.part == 2) ? p0 : 0;
        khi = (ca.part == 1) ? p0 : p0 + n;
        const size_t coff = kv_offset(unit, heads, kv_heads, g + w, D);
        KC = reinterpret_cast<const uint16_t *>(ca.kc) + coff;
        VC = reinterpret_cast<const uint16_t *>(ca.vc) + coff;
    }
    if constexpr (STRIDED) {
        if (ca.mode == 1) {
            khi = nq;  // class-local positions, an ordinary window
        } else {
            khi = (n + ca.r - 1) / ca.r;  // landmarks k r < n
            klo = (g + ca.r - 1) / ca.r;  // landmarks below g are sinks of the other part
            wq = kNoWindow;
            g = 0;
        }
    }
    // key position bound of query row r (the causal limit j <= qpos(r))
    auto qpos = [&](int r) -> int {
        if constexpr (STRIDED) {
            if (ca.mode == 2) return (r >= w) ? (r - w) / ca.r : -1;
        }
        return p0 + r;
    };
    const int qa = qpos(qi);  // position of this lane's query row
    const BandRange band = band_range(qpos(q0), qpos(q1), wq, g, kBK);
    // kLandmark: tiles 0 .. nl-1 hold compact landmark indices (lb0 + t) * kBK
    // .. +kBK-1 (K/V rows k * ca.r), covering lk_lo .. the block's last row's
    // last landmark; the window-and-sink tiles follow as tiles nl ..
    int nl = 0, lb0 = 0, lk_lo = 0;
    if constexpr (LAND) {
        lk_lo = (g + ca.r - 1) / ca.r;  // landmarks below g are sinks
        const int lq1 = (q1 >= w) ? (q1 - w) / ca.r : -1;
        if (lq1 >= lk_lo) {
            lb0 = lk_lo / kBK;
            nl = lq1 / kBK - lb0 + 1;
        }
    }
    const int ntiles = nl + band.count();
    const float tau = 8.f / c2;

    // ---- Q of this wave's 32 rows as the B operand (kept in VGPRs) ----
    bf16x8 qf[D / 16];
    {
        const int qr0 = oq + q0 * sq;  // first row of this block in q
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + (size_t)qr0 * D, (uint32_t)(n - qr0) * L::kRowBytes);
        const uint32_t rowoff = row_off((uint64_t)(wave * 32 + lr) * sq, n, L::kRowBytes);
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
            qf[c] = __builtin_bit_cast(bf16x8, buffer_load16(rq, rowoff + (16 * c + 8 * lh) * 2));
    }

    // ---- DMA of K and V tiles into LDS: each wave moves its share ----
    // LDS holds two K buffers and two V buffers.  DMA load i of this wave
    // fills bytes [1 KB m, 1 KB (m+1)) of a tile, m = wave * kDmaPerWave + i:
    // column block m/4, keys 16 (m%4) + lane/4, chunk position lane%4.  The
    // global chunk that belongs there undoes the swizzle (K) or is the same
    // chunk (V).
    uint32_t dma_k[L::kDmaPerWave], dma_v[L::kDmaPerWave];
#pragma unroll
    for (int i = 0; i < L::kDmaPerWave; ++i) {
        const int m = wave * L::kDmaPerWave + i;
        const int key = 16 * (m & 3) + (lane >> 2);
        const int pos = lane & 3;
        const int ck = (m >> 2) * 4 + (pos ^ ((key >> 2) & 3));
        const int cv = (m >> 2) * 4 + pos;
        // strided rows: the 64-bit, clamped offset (a stride can be as large
        // as n); otherwise key * row bytes, from which the chunk gather below
        // recovers the key
        const uint32_t rb = STRIDED ? row_off((uint64_t)key * skv, n, L::kRowBytes) : key * L::kRowBytes;
        dma_k[i] = rb + 16 * ck;
        dma_v[i] = rb + 16 * cv;
    }
    auto dma_rows = [&](const uint16_t *src, const uint32_t *offs, int r0, int nrows, uint8_t *dst) {
        // rows r0 .. of src, rows >= nrows read as zero
        const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (size_t)r0 * D, (uint32_t)(nrows - r0) * L::kRowBytes);
#pragma unroll
        for (int i = 0; i < L::kDmaPerWave; ++i) dma16(r, dst + (wave * L::kDmaPerWave + i) * 1024, offs[i]);
    };
    // landmark tile: compact indices k0 .. k0+63, rows k * ca.r (the offsets
    // above are key * row bytes + chunk; the row is re-formed in 64 bits and
    // clamped as for a strided launch)
    auto dma_land = [&](bool is_k, int k0, uint8_t *dst) {
        const uint16_t *src = is_k ? K : V;
        const uint32_t *offs = is_k ? dma_k : dma_v;
        const int r0 = k0 * ca.r;  // < n: tile nl-1 holds a landmark below n
        const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (size_t)r0 * D, (uint32_t)(n - r0) * L::kRowBytes);
#pragma unroll
        for (int i = 0; i < L::kDmaPerWave; ++i) {
            const uint32_t key = offs[i] / L::kRowBytes;
            const uint32_t part = offs[i] - key * L::kRowBytes;
            dma16(r, dst + (wave * L::kDmaPerWave + i) * 1024, row_off((uint64_t)key * ca.r, n, L::kRowBytes) + part);
        }
    };
    // tile of key positions k0 .. k0+63 of K (or V) into LDS at dst
    auto dma = [&](bool is_k, int k0, uint8_t *dst) {
        const uint16_t *src = is_k ? K : V;
        const uint32_t *offs = is_k ? dma_k : dma_v;
        if constexpr (!CHUNK) {
            dma_rows(src, offs, okv + k0 * skv, n, dst);
        } else {
            const uint16_t *cache = is_k ? KC : VC;
            if (k0 >= p0) {
                dma_rows(src, offs, k0 - p0, n, dst);  // all in the chunk
            } else if (k0 + kBK <= p0 && k0 >= p0 - w && k0 % w + kBK <= w) {
                dma_rows(cache, offs, g + k0 % w, g + w, dst);  // one unwrapped run of the ring
            } else {
                // row by row: chunk, ring or sink row of each key position
                const __amdgpu_buffer_rsrc_t rn = make_rsrc(src, (uint32_t)n * L::kRowBytes);
                const __amdgpu_buffer_rsrc_t rc = make_rsrc(cache, (uint32_t)(g + w) * L::kRowBytes);
#pragma unroll
                for (int i = 0; i < L::kDmaPerWave; ++i) {
                    const int key = (int)(offs[i] / L::kRowBytes);
                    const uint32_t part = offs[i] - (uint32_t)key * L::kRowBytes;
                    const int sp = k0 + key;
                    uint8_t *d = dst + (wave * L::kDmaPerWave + i) * 1024;
                    if (sp >= p0)
                        dma16(rn, d, (uint32_t)(sp - p0) * L::kRowBytes + part);
                    else
                        dma16(rc, d, (uint32_t)cache_row(sp, p0, w, g) * L::kRowBytes + part);
                }
            }
        }
    };

    // tile t of the block's sequence: landmark tiles first (kLandmark), then
    // the window-and-sink tiles.  MAYBE_LAND false: t is known to be past the
    // landmark tiles.
    auto key_block = [&](int t) -> int {
        if constexpr (LAND) {
            if (t < nl) return lb0 + t;
            return band.block(t - nl);
        }
        return band.block(t);
    };
    auto dma_t = [&](bool is_k, int t, uint8_t *dst, auto maybe_land_tag) __attribute__((always_inline)) {
        if constexpr (LAND && decltype(maybe_land_tag)::value) {
            if (t < nl) {
                dma_land(is_k, (lb0 + t) * kBK, dst);
                return;
            }
        }
        if constexpr (LAND) t -= nl;
        dma(is_k, band.block(t) * kBK, dst);
    };

    // Per-lane LDS read offsets within a buffer.
    // K operand: row 32 sb + lr, 16-byte chunk 2c + lh; even and odd c differ
    // in the chunk position, c/2 selects the column block.
    const uint32_t koff_even = L::k_off(lr, lh);
    const uint32_t koff_odd = L::k_off(lr, 2 + lh);
    // V operand (transposed read): lane j of 16-lane group G supplies key
    // 4 (G/2) + j/4 (on top of the chunk's key base) and the 8-byte piece of
    // columns 16 (G%2) + 4 (j%4) .. +3; the instruction hands lane j of the
    // group column 16 (G%2) + j of four consecutive keys.
    const int grp = lane >> 4, jj = lane & 15;
    const uint32_t voff = L::v_off(4 * (grp >> 1) + (jj >> 2), 4 * (grp & 1) + (jj & 3));

    // S^T = K Q^T of one tile whose K sits at kb
    auto scores = [&](const uint8_t *kb, f32x16 (&s)[2]) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
#pragma unroll
            for (int c = 0; c < D / 16; ++c) {
                const uint32_t off = ((c & 1) ? koff_odd : koff_even) + (c >> 1) * (kBK * 64) + sb * 32 * 64;
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kb + off);
                s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[sb], 0, 0, 0);
            }
        }
    };

    f32x16 oacc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
    float m_run = kNegInf, negm = 0.f, l_run = 0.f;

    // Key bounds of this wave's rows: a key after dead_hi, or below dead_lo
    // and not a sink, is attended by none of them.
    const int qw0 = q0 + wave * 32;  // this wave's first row
    const int qw_last = min(qw0 + 31, nq - 1);
    const int dead_hi = qpos(qw_last), dead_lo = qpos(qw0) - wq + 1;

    // Pipeline: tile t forms the probabilities of tile t, the scores of tile
    // t+1 and the PV product of tile t.  During tile t the DMA fills K(t+2)
    // into the K buffer that K(t) left and V(t+1) into the V buffer that
    // V(t-1) left, so every DMA has a whole tile of time to land.
    dma_t(true, 0, kbuf0, std::true_type{});
    dma_t(false, 0, vbuf0, std::true_type{});
    if (ntiles > 1) dma_t(true, 1, kbuf1, std::true_type{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 s_cur[2];
    {
        // tile 0's scores are not needed when no row of this wave attends it
        // (the window's first tile for the last two waves of a block)
        const int kk = key_block(0) * kBK;
        if (LAND || !(kk > dead_hi || (kk + kBK <= dead_lo && kk >= g))) {
            scores(kbuf0, s_cur);
        } else {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s_cur[sb][r] = 0.f;
        }
    }
    __syncthreads();  // every wave is done with K(0) before K(2) replaces it

    auto do_tile_p = [&](int t, auto masked_tag, auto par_tag, auto last_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        constexpr bool LAST = decltype(last_tag)::value;  // the block's last tile: no next tile to score
        constexpr int PAR = decltype(par_tag)::value;  // t & 1, or 2: from t at run time
        const int par = (PAR == 2) ? (t & 1) : PAR;
        uint8_t *const kcur = par ? kbuf1 : kbuf0;
        uint8_t *const knxt = par ? kbuf0 : kbuf1;
        uint8_t *const vcur = par ? vbuf1 : vbuf0;
        uint8_t *const vnxt = par ? vbuf0 : vbuf1;
        const int k0 = key_block(t) * kBK;
        // Wave priority over the tile: 1 while this wave issues its DMAs and
        // K fragment reads (its loads go out ahead of the other wave's vector
        // work), 0 over the vector phase, 1 over the score MFMAs and 2 over
        // the PV MFMAs (the wave nearest its barrier goes first).
        __builtin_amdgcn_s_setprio(1);
        // only cut tiles can be landmark tiles or precede one
        using ML = std::integral_constant<bool, MASKED>;
        if (t + 2 < ntiles) dma_t(true, t + 2, kcur, ML{});
        if (t + 1 < ntiles) dma_t(false, t + 1, vnxt, ML{});

        const uint8_t *kb = knxt;
        const uint8_t *vb = vcur + voff;
        constexpr int NC = D / 16;       // MFMAs per 32-key score sub-block
        constexpr int NS = 2 * NC;       // score MFMAs per tile
        constexpr int NP = 4 * (D / 32); // PV MFMAs per tile
        constexpr int VA = 3;            // V^T fragment read-ahead
        auto kfrag = [&](int j) -> bf16x8 {
            const int sb = j / NC, c = j % NC;
            const uint32_t off = ((c & 1) ? koff_odd : koff_even) + (c >> 1) * (kBK * 64) + sb * 32 * 64;
            return *reinterpret_cast<const bf16x8 *>(kb + off);
        };
        auto vfrag = [&](int j) -> bf16x8 {  // j = kc * (D/32) + cb
            const int kc = j / (D / 32), cb = j % (D / 32);
            // keys 16 kc + 4 lh + 0..3 (first read) and 16 kc + 8 + 4 lh + 0..3
            const uint8_t *p0 = vb + cb * (kBK * 64) + (16 * kc) * 64;
            const s16x4 lo = lds_read_tr16(p0);
            const s16x4 hi = lds_read_tr16(p0 + 8 * 64);
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        // Every K fragment of tile t+1 is read at the top of the tile; the
        // vector phase (on cut tiles also the mask and the row max) covers
        // the latency.
        bf16x8 kf[NS];
        if constexpr (!LAST) {
#pragma unroll
            for (int j = 0; j < NS; ++j) kf[j] = kfrag(j);
        }
        __builtin_amdgcn_s_setprio(0);

        // A cut tile none of whose pairs this wave's rows attend adds nothing
        // to them: its mask, exponentials and PV MFMAs are skipped (the score
        // MFMAs of the next tile still run).  Landmark tiles, whose keys are
        // compact indices, always run.
        bool dead = false;
        if constexpr (MASKED && !LAND) dead = (k0 > dead_hi) || (k0 + kBK <= dead_lo && k0 >= g);
        if constexpr (MASKED) {
            if (!dead) {
                if (LAND && t < nl)  // the row's last landmark below its window: (qi - w) / r
                    mask_landmark_tile(s_cur, (qa >= w) ? (qa - w) / ca.r : -1, k0, lh, lk_lo);
                else
                    mask_tile<CHUNK || STRIDED>(s_cur, qa, k0, lh, khi, wq, g, bias_raw, klo);
                update_max(s_cur, m_run, negm, l_run, oacc, c2, tau);
            }
        }

        // The rest of the tile is two phases, in a fixed order (sched_barrier
        // pins it):
        //  1. vector work: the exponentials of tile t, their bf16 packing and
        //     row-sum dot2s, and on FULL tiles the deferred max check;
        //  2. matrix work at raised wave priority: the score MFMAs of tile
        //     t+1 (none on the last tile), then the PV MFMAs of tile t, the
        //     V^T fragments read 3 MFMAs ahead.
        // The two waves of a SIMD belong to different workgroups at unrelated
        // points of their tiles: one wave's vector phase issues beside the
        // other's matrix phase, and the priorities let the wave that feeds
        // the matrix core issue first when both are ready.  (Spreading
        // the exponentials over the score MFMAs, or the PV MFMAs over both,
        // gives each wave a uniform mix and measured 2-5 % slower.)
        f32x16 s_nxt[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
            for (int r = 0; r < 16; ++r) s_nxt[sb][r] = 0.f;
        bf16x8 vf[VA];
        const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
        // probabilities of tile t as bf16 pairs: word i holds flat scores 2i, 2i+1
        // (flat e = 16 sb + r); the row-sum dot2s alternate between two sums
        uint32_t pw[16];
        float ls0 = 0.f, ls1 = 0.f;
        auto prob_pair = [&](int i) __attribute__((always_inline)) {
            const int e = 2 * i;
            const float a = fast_exp2(fmaf(s_cur[e >> 4][e & 15], c2, negm));
            const float b = fast_exp2(fmaf(s_cur[(e + 1) >> 4][(e + 1) & 15], c2, negm));
            const bf16x2 pr = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
            pw[i] = __builtin_bit_cast(uint32_t, pr);
            if (i & 1) ls1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls1, false);
            else ls0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls0, false);
        };
        if (dead) {
#pragma unroll
            for (int i = 0; i < 16; ++i) pw[i] = 0u;  // unread; left undefined, it costs spills
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) prob_pair(i);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!MASKED) {
            // The reference max moves only if some probability reached 2^8;
            // a lane whose bf16 row sum stays below 2^7 has none, so the
            // exact update (and a recomputation) runs only when a lane's sum
            // reaches 2^7, or the row has no reference yet.
            const float lsum = ls0 + ls1;
            if (__any(!(lsum < 128.f) || m_run == kNegInf)) {
                update_max(s_cur, m_run, negm, l_run, oacc, c2, tau);
                ls0 = 0.f;
                ls1 = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) prob_pair(i);
            }
        }

        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if (j >= NS - VA) vf[j - (NS - VA)] = vfrag(j - (NS - VA));
            if constexpr (!LAST)
                s_nxt[j / NC] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[j], qf[j % NC], s_nxt[j / NC], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(2);
        if (!dead) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                // probabilities of keys 16 kc + {4 lh + 0..3, 8 + 4 lh + 0..3}, rounded to bf16
                const bf16x8 pk =
                    __builtin_bit_cast(bf16x8, make_uint4(pw[4 * kc], pw[4 * kc + 1], pw[4 * kc + 2], pw[4 * kc + 3]));
#pragma unroll
                for (int cb = 0; cb < D / 32; ++cb) {
                    const int j = kc * (D / 32) + cb;
                    const bf16x8 a = vf[j % VA];
                    if (j + VA < NP) vf[j % VA] = vfrag(j + VA);
                    oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk, oacc[cb], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        l_run += ls0 + ls1;
        if constexpr (!LAST) {
            s_cur[0] = s_nxt[0];
            s_cur[1] = s_nxt[1];
        }
        __builtin_amdgcn_s_setprio(0);

        __builtin_amdgcn_s_waitcnt(0);  // K(t+2) and V(t+1) of this wave have landed
        __syncthreads();
    };

    // FULL tiles for this wave's own 32 rows: the band edges of the
    // workgroup's block cut a single wave's rows in fewer tiles.
    // (a wave entirely past n keeps all window tiles unmasked: it stores
    // nothing; landmark tiles always take the cut-tile body, whose DMA knows them)
    int t_lo = 0, t_hi = band.count();
    if (qw0 < nq) full_range(band, qpos(qw0), qpos(min(qw0 + 31, nq - 1)), khi, wq, g, kBK, &t_lo, &t_hi, klo);
    t_lo += nl;
    t_hi += nl;
    // The last tile runs on its own (no next tile to score) and with the
    // mask, which leaves a FULL tile's scores as they are.  (In the chunk
    // kernel this costs two spilled registers, reloaded on the cut tiles
    // before the FULL run; skipping the discarded score stream gains more.)
    if (t_hi > ntiles - 1) t_hi = ntiles - 1;
    if (t_lo > t_hi) t_lo = t_hi;
    // The FULL run is unrolled by two so that each tile body names its
    // buffers statically (parity 0 / 1); the cut tiles take the parity at run
    // time (2).
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using T = std::true_type;
    using F = std::false_type;
    // Scalar loads still in flight here (kernel arguments the epilogue
    // needs) would share the LDS counter inside the loop: every tile would
    // then wait for all its K fragment reads before its first MFMA.
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
    int t = 0;
    for (; t < t_lo; ++t) do_tile_p(t, T{}, P2{}, F{});
    if ((t & 1) && t < t_hi) {
        do_tile_p(t, F{}, P1{}, F{});
        ++t;
    }
    for (; t + 1 < t_hi; t += 2) {
        do_tile_p(t, F{}, P0{}, F{});
        do_tile_p(t + 1, F{}, P1{}, F{});
    }
    if (t < t_hi) {
        do_tile_p(t, F{}, P0{}, F{});
        ++t;
    }
    for (; t < ntiles - 1; ++t) do_tile_p(t, T{}, P2{}, F{});
    do_tile_p(ntiles - 1, T{}, P2{}, T{});

    // the loop's last barrier has every wave past its LDS reads; each wave
    // stages its rows in its own 32 * 2D bytes of the K buffers
    static_assert(2 * 32 * 2 * D <= L::kTileBytes, "two waves' rows per K buffer");
    uint8_t *const region = ((wave < 2) ? kbuf0 : kbuf1) + (wave & 1) * (32 * 2 * D);
    store_rows_lds<D>(oacc, m_run, l_run, q0 + wave * 32, nq, lr, lh, lane, op + base + (size_t)oq * D,
                      lsep ? lsep + (size_t)unit * n + oq : nullptr, scale, sq, region);
}

// ---------------------------------------------------------------------------
// fp32 path (parity): VGPR-staged tiles, V transposed on the way into LDS.
template <int D>
struct F32Cfg {
    static constexpr int kCPR = D / 4;        // 16-byte chunks per row
    static constexpr int kKStride = D + 4;    // K row stride (floats)
    static constexpr int kVStride = kBK + 4;  // V^T row stride (floats)
    static constexpr int kKElems = kBK * kKStride;
    static constexpr int kVElems = D * kVStride;
    static constexpr int kStage = kKElems + kVElems;
    static constexpr int kKChunks = kBK * kCPR / kThreads;
    static constexpr int kVBlocks = (kBK / 4) * kCPR / kThreads;
    static_assert(kBK * kCPR % kThreads == 0 && (kBK / 4) * kCPR % kThreads == 0, "tile split");
};

// Where the fp32 loader finds key index s: row okv + s skv of the sequence
// (rows >= n read as zero), or chunk / cache rows as in the bf16 path.
struct F32KeyRows {
    const float *k, *v;    // sequence or chunk rows
    const float *kc, *vc;  // cache rows (chunked prefill only)
    int n, p0, w, g;
    bool chunk;
    int skv, okv;          // strided patterns
    __device__ __forceinline__ uint4 load(bool is_k, int s, int col_byte, int d) const {
        if (!chunk || s >= p0) {
            const __amdgpu_buffer_rsrc_t r = make_rsrc(is_k ? k : v, (uint32_t)n * d * 4);
            return buffer_load16(r, row_off((uint64_t)okv + (uint64_t)(s - p0) * skv, n, d * 4) + col_byte);
        }
        const __amdgpu_buffer_rsrc_t r = make_rsrc(is_k ? kc : vc, (uint32_t)(g + w) * d * 4);
        return buffer_load16(r, (uint32_t)cache_row(s, p0, w, g) * d * 4 + col_byte);
    }
};

template <int D>
struct F32TileLoader {
    using C = F32Cfg<D>;
    uint4 k[C::kKChunks];
    uint4 v[C::kVBlocks][4];

    __device__ __forceinline__ void load(const F32KeyRows &src, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < C::kKChunks; ++i) {
            const int id = tid + kThreads * i;
            k[i] = src.load(true, k0 + id / C::kCPR, (id % C::kCPR) * 16, D);
        }
#pragma unroll
        for (int i = 0; i < C::kVBlocks; ++i) {
            const int id = tid + kThreads * i;
            const int kg = id % (kBK / 4), cg = id / (kBK / 4);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) v[i][rr] = src.load(false, k0 + 4 * kg + rr, cg * 16, D);
        }
    }
    __device__ __forceinline__ void store(float *ks, float *vts, int tid) const {
#pragma unroll
        for (int i = 0; i < C::kKChunks; ++i) {
            const int id = tid + kThreads * i;
            *reinterpret_cast<uint4 *>(ks + (id / C::kCPR) * C::kKStride + (id % C::kCPR) * 4) = k[i];
        }
#pragma unroll
        for (int i = 0; i < C::kVBlocks; ++i) {
            const int id = tid + kThreads * i;
            const int kg = id % (kBK / 4), cg = id / (kBK / 4);
            const uint32_t *r0 = reinterpret_cast<const uint32_t *>(&v[i][0]);
            const uint32_t *r1 = reinterpret_cast<const uint32_t *>(&v[i][1]);
            const uint32_t *r2 = reinterpret_cast<const uint32_t *>(&v[i][2]);
            const uint32_t *r3 = reinterpret_cast<const uint32_t *>(&v[i][3]);
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
                *reinterpret_cast<uint4 *>(vts + (cg * 4 + cc) * C::kVStride + 4 * kg) =
                    make_uint4(r0[cc], r1[cc], r2[cc], r3[cc]);
        }
    }
};

template <int D, int KIND>
__global__ __launch_bounds__(kThreads, 1) void prefill_f32_kernel(
    const float *__restrict__ qp, const float *__restrict__ kp, const float *__restrict__ vp,
    float *__restrict__ op, float *__restrict__ lsep, int n, int nqb, int w, int g, float c2, float scale,
    float bias_raw, int total_wg, int heads, int kv_heads, PathArgs ca) {
    constexpr bool CHUNK = (KIND == kChunk), STRIDED = (KIND == kStrided);
    using C = F32Cfg<D>;
    __shared__ __attribute__((aligned(16))) float smem[2 * C::kStage];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 31;
    const int lh = lane >> 5;

    int unit, qb;
    workgroup_order(blockIdx.x, total_wg, nqb, STRIDED ? 1 : heads / kv_heads, &unit, &qb);
    int nq = n, sq = 1, oq = 0, skv = 1, okv = 0;  // strided patterns, as in the bf16 kernel
    if constexpr (STRIDED) {
        if (ca.mode == 1) {
            const int cls = unit % ca.r;
            unit /= ca.r;
            nq = (n - cls + ca.r - 1) / ca.r;
            sq = ca.r;
            oq = cls;
            okv = cls;
        }
        skv = ca.r;
    }
    const size_t base = (size_t)unit * n * D;  // q and o of (batch, head)
    const float *Q = qp + base;
    const float *K = kp + kv_offset(unit, heads, kv_heads, n, D);
    const float *V = vp + kv_offset(unit, heads, kv_heads, n, D);

    const int q0 = qb * kBQ;
    const int q1 = min(q0 + kBQ, nq) - 1;
    const int qi = q0 + wave * 32 + lr;
    if (STRIDED && q0 >= nq) return;
    F32KeyRows src{K, V, nullptr, nullptr, n, 0, w, g, CHUNK, skv, okv};
    int p0 = 0, klo = 0, khi = n, wq = w;
    if constexpr (CHUNK) {
        const int b = unit / heads;
        const int64_t pb = ca.pos[b];
        if (pb < 0 || pb > (int64_t)(0x7fffffff - kPosHeadroom - n)) {
            if (qi < n) {
                float *orow = op + base + (size_t)qi * D;
                for (int c = 4 * lh; c < D; c += 8) {
                    const float nan = __builtin_nanf("");
                    *reinterpret_cast<float4 *>(orow + c) = make_float4(nan, nan, nan, nan);
                }
                if (lsep != nullptr && lh == 0) lsep[(size_t)unit * n + qi] = __builtin_nanf("");
            }
            return;
        }
        p0 = (int)pb;
        klo = (ca.part == 2) ? p0 : 0;
        khi = (ca.part == 1) ? p0 : p0 + n;
        const size_t coff = kv_offset(unit, heads, kv_heads, g + w, D);
        src.kc = reinterpret_cast<const float *>(ca.kc) + coff;
        src.vc = reinterpret_cast<const float *>(ca.vc) + coff;
        src.p0 = p0;
    }
    if constexpr (STRIDED) {
        if (ca.mode == 1) {
            khi = nq;
        } else {
            khi = (n + ca.r - 1) / ca.r;
            klo = (g + ca.r - 1) / ca.r;
            wq = kNoWindow;
            g = 0;
        }
    }
    auto qpos = [&](int r) -> int {
        if constexpr (STRIDED) {
            if (ca.mode == 2) return (r >= w) ? (r - w) / ca.r : -1;
        }
        return p0 + r;
    };
    const int qa = qpos(qi);
    const BandRange band = band_range(qpos(q0), qpos(q1), wq, g, kBK);
    const int ntiles = band.count();
    const float tau = 8.f / c2;

    // Q as the B operand of 32x32x2 MFMAs: lane half lh holds d = 2c + lh
    float qf[D / 2];
    {
        const int qr0 = oq + q0 * sq;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + (size_t)qr0 * D, (uint32_t)(n - qr0) * D * 4);
        const uint32_t rowoff = row_off((uint64_t)(wave * 32 + lr) * sq, n, D * 4);
#pragma unroll
        for (int c4 = 0; c4 < D / 8; ++c4) {
            const uint4 a = buffer_load16(rq, rowoff + (8 * c4) * 4);
            const uint4 b = buffer_load16(rq, rowoff + (8 * c4 + 4) * 4);
            const uint32_t e[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) qf[4 * c4 + j] = __uint_as_float(lh ? e[2 * j + 1] : e[2 * j]);
        }
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[cb][r] = 0.f;
    float m_run = kNegInf, negm = 0.f, l_run = 0.f;

    F32TileLoader<D> ld;
    ld.load(src, band.block(0) * kBK, tid);
    ld.store(smem, smem + C::kKElems, tid);
    __syncthreads();

    auto do_tile = [&](int t, int stage, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const float *Ks = smem + stage * C::kStage;
        const float *Vts = Ks + C::kKElems;
        const int k0 = band.block(t) * kBK;
        const bool has_next = (t + 1 < ntiles);
        if (has_next) ld.load(src, band.block(t + 1) * kBK, tid);

        f32x16 s[2];
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[sb][r] = 0.f;
            const float *krow = Ks + (32 * sb + lr) * C::kKStride + lh;
#pragma unroll
            for (int c = 0; c < D / 2; ++c)
                s[sb] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * c], qf[c], s[sb], 0, 0, 0);
        }
        if constexpr (MASKED) mask_tile<CHUNK || STRIDED>(s, qa, k0, lh, khi, wq, g, bias_raw, klo);
        update_max(s, m_run, negm, l_run, oacc, c2, tau);

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
            const float *vrow = Vts + (32 * cb + lr) * C::kVStride + 4 * lh;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    oacc[cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * sb + 8 * (r >> 2) + (r & 3)], s[sb][r],
                                                                    oacc[cb], 0, 0, 0);
        }

        if (has_next) {
            float *nxt = smem + (stage ^ 1) * C::kStage;
            ld.store(nxt, nxt + C::kKElems, tid);
        }
        __syncthreads();
    };

    int t_lo, t_hi;
    full_range(band, qpos(q0), qpos(q1), khi, wq, g, kBK, &t_lo, &t_hi, klo);
    int t = 0, stage = 0;
    for (; t < t_lo; ++t, stage ^= 1) do_tile(t, stage, std::true_type{});
    for (; t < t_hi; ++t, stage ^= 1) do_tile(t, stage, std::false_type{});
    for (; t < ntiles; ++t, stage ^= 1) do_tile(t, stage, std::true_type{});

    store_rows<float, D>(oacc, m_run, l_run, qi, nq, lh, op + base + (size_t)oq * D,
                         lsep ? lsep + (size_t)unit * n + oq : nullptr, scale, sq);
}

// ---------------------------------------------------------------------------
// Query rows per workgroup (the prefill grid is units x ceil(n / rows)).
int prefill_rows_per_workgroup(bool bf16) { return bf16 ? 32 * kWaves16 : kBQ; }

// Host launchers (validated arguments only).  units_mul: grid units per
// (batch, head) (the residue classes of a dilated launch); nq_max: query rows
// of the longest unit.
template <int KIND>
static hipError_t launch_prefill_t(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                                   int heads, int kv_heads, int n, int d, int w, int g, float scale,
                                   float sink_bias, bool bf16, PathArgs ca, int units_mul, int nq_max,
                                   hipStream_t stream) {
    const int units = batch * heads * units_mul;
    const float c2 = (float)((double)scale * kLog2e);
    const float bias_raw = (float)((double)sink_bias / (double)scale);
    if (bf16) {
        const int bq = 32 * kWaves16;
        const int nqb = (nq_max + bq - 1) / bq;
        const int total = units * nqb;
        const dim3 grid(total), block(64 * kWaves16);
        const uint16_t *qq = (const uint16_t *)q, *kk = (const uint16_t *)k, *vv = (const uint16_t *)v;
        uint16_t *oo = (uint16_t *)o;
        if (d == 128)
            hipLaunchKernelGGL((prefill_bf16_kernel<128, kWaves16, KIND>), grid, block, 0, stream, qq, kk, vv, oo,
                               lse, n, nqb, w, g, c2, scale, bias_raw, total, heads, kv_heads, ca);
        else
            hipLaunchKernelGGL((prefill_bf16_kernel<64, kWaves16, KIND>), grid, block, 0, stream, qq, kk, vv, oo,
                               lse, n, nqb, w, g, c2, scale, bias_raw, total, heads, kv_heads, ca);
    } else if constexpr (KIND == kLandmark) {
        return hipErrorInvalidValue;  // bf16 only: fp32 runs the landmark part as a launch of its own
    } else {
        const int nqb = (nq_max + kBQ - 1) / kBQ;
        const int total = units * nqb;
        const dim3 grid(total), block(kThreads);
        const float *qq = (const float *)q, *kk = (const float *)k, *vv = (const float *)v;
        float *oo = (float *)o;
        if (d == 128)
            hipLaunchKernelGGL((prefill_f32_kernel<128, KIND>), grid, block, 0, stream, qq, kk, vv, oo, lse, n, nqb,
                               w, g, c2, scale, bias_raw, total, heads, kv_heads, ca);
        else
            hipLaunchKernelGGL((prefill_f32_kernel<64, KIND>), grid, block, 0, stream, qq, kk, vv, oo, lse, n, nqb,
                               w, g, c2, scale, bias_raw, total, heads, kv_heads, ca);
    }
    return hipGetLastError();
}

hipError_t launch_prefill(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int heads,
                          int kv_heads, int n, int d, int w, int g, float scale, float sink_bias, bool bf16,
                          hipStream_t stream) {
    return launch_prefill_t<kPlain>(q, k, v, o, lse, batch, heads, kv_heads, n, d, w, g, scale, sink_bias, bf16,
                                    PathArgs{nullptr, nullptr, nullptr, 0, 1, 0}, 1, n, stream);
}

hipError_t launch_chunk_prefill(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                                const void *v_cache, const int64_t *pos, void *o, float *lse, int batch, int heads,
                                int kv_heads, int t, int d, int w, int g, float scale, float sink_bias, int part,
                                bool bf16, hipStream_t stream) {
    return launch_prefill_t<kChunk>(q, k_new, v_new, o, lse, batch, heads, kv_heads, t, d, w, g, scale, sink_bias,
                                    bf16, PathArgs{k_cache, v_cache, pos, part, 1, 0}, 1, t, stream);
}

// Dilated window: r residue classes per (batch, head), each an ordinary
// window of w over its strided rows (no sinks).
hipError_t launch_dilated_prefill(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                                  int heads, int kv_heads, int n, int d, int w, int r, float scale, bool bf16,
                                  hipStream_t stream) {
    return launch_prefill_t<kStrided>(q, k, v, o, lse, batch, heads, kv_heads, n, d, w, 0, scale, 0.f, bf16,
                                      PathArgs{nullptr, nullptr, nullptr, 0, r, 1}, r, (n + r - 1) / r, stream);
}

// Landmark part of window + sinks + landmarks every r: the landmarks below
// the window and not below g (lse of rows without one: -inf, o = 0).
hipError_t launch_landmark_part(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                                int heads, int kv_heads, int n, int d, int w, int g, int r, float scale, bool bf16,
                                hipStream_t stream) {
    return launch_prefill_t<kStrided>(q, k, v, o, lse, batch, heads, kv_heads, n, d, w, g, scale, 0.f, bf16,
                                      PathArgs{nullptr, nullptr, nullptr, 0, r, 2}, 1, n, stream);
}

// Window + sinks + landmarks every r in one bf16 launch (landmark tiles, then
// the window-and-sink tiles of each query block, one online softmax).
hipError_t launch_landmark_prefill(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                                   int heads, int kv_heads, int n, int d, int w, int g, int r, float scale,
                                   float sink_bias, hipStream_t stream) {
    return launch_prefill_t<kLandmark>(q, k, v, o, lse, batch, heads, kv_heads, n, d, w, g, scale, sink_bias, true,
                                       PathArgs{nullptr, nullptr, nullptr, 0, r, 0}, 1, n, stream);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of two partial attentions over disjoint key sets of the
// same query rows ("Sliding Window and Sparse Attention, from Longformer to
// CSA2", s10 glossary, LSE): with M = max(lse_a, lse_b),
//   o = (e^(lse_a - M) o_a + e^(lse_b - M) o_b) / (e^(lse_a - M) + e^(lse_b - M)),
//   lse = M + ln(e^(lse_a - M) + e^(lse_b - M)).
// A part with lse = -inf (no key) has weight 0; two empty parts give o = 0
// and lse = -inf.  One thread per 4 columns of a row.
template <typename T>
__global__ __launch_bounds__(256) void lse_merge_kernel(const T *__restrict__ oa, const float *__restrict__ la,
                                                       const T *__restrict__ ob, const float *__restrict__ lb,
                                                       T *__restrict__ o, float *__restrict__ lse, long rows,
                                                       int d) {
    const long idx = (long)blockIdx.x * 256 + threadIdx.x;
    const int per_row = d / 4;
    const long row = idx / per_row;
    if (row >= rows) return;
    const int c = (int)(idx - row * per_row) * 4;
    const float a = la[row], b = lb[row];
    const float M = fmaxf(a, b);
    float wa = 0.f, wb = 0.f;
    if (M != kNegInf) {
        wa = fast_exp2((a - M) * (float)kLog2e);
        wb = fast_exp2((b - M) * (float)kLog2e);
    }
    const float sum = wa + wb;
    const float inv = (sum > 0.f) ? 1.f / sum : 0.f;
    wa *= inv;
    wb *= inv;
    float xa[4], xb[4];
    const size_t off = (size_t)row * d + c;
    if constexpr (std::is_same<T, uint16_t>::value) {
        const uint2 ua = *reinterpret_cast<const uint2 *>(oa + off), ub = *reinterpret_cast<const uint2 *>(ob + off);
        xa[0] = bf16lo(ua.x); xa[1] = bf16hi(ua.x); xa[2] = bf16lo(ua.y); xa[3] = bf16hi(ua.y);
        xb[0] = bf16lo(ub.x); xb[1] = bf16hi(ub.x); xb[2] = bf16lo(ub.y); xb[3] = bf16hi(ub.y);
        float r[4];
        for (int e = 0; e < 4; ++e) r[e] = (wa > 0.f ? wa * xa[e] : 0.f) + (wb > 0.f ? wb * xb[e] : 0.f);
        *reinterpret_cast<uint2 *>(o + off) = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
    } else {
        const float4 fa = *reinterpret_cast<const float4 *>(oa + off), fb = *reinterpret_cast<const float4 *>(ob + off);
        xa[0] = fa.x; xa[1] = fa.y; xa[2] = fa.z; xa[3] = fa.w;
        xb[0] = fb.x; xb[1] = fb.y; xb[2] = fb.z; xb[3] = fb.w;
        float r[4];
        for (int e = 0; e < 4; ++e) r[e] = (wa > 0.f ? wa * xa[e] : 0.f) + (wb > 0.f ? wb * xb[e] : 0.f);
        *reinterpret_cast<float4 *>(o + off) = make_float4(r[0], r[1], r[2], r[3]);
    }
    if (lse != nullptr && c == 0) lse[row] = (sum > 0.f) ? M + logf(sum) : kNegInf;
}

hipError_t launch_lse_merge(const void *oa, const float *la, const void *ob, const float *lb, void *o, float *lse,
                            long rows, int d, bool bf16, hipStream_t stream) {
    const long threads = rows * (d / 4);
    const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
    if (bf16)
        hipLaunchKernelGGL(lse_merge_kernel<uint16_t>, grid, block, 0, stream, (const uint16_t *)oa, la,
                           (const uint16_t *)ob, lb, (uint16_t *)o, lse, rows, d);
    else
        hipLaunchKernelGGL(lse_merge_kernel<float>, grid, block, 0, stream, (const float *)oa, la, (const float *)ob,
                           lb, (float *)o, lse, rows, d);
    return hipGetLastError();
}

}  // namespace swa
