// api.cpp -- the C ABI of libswa.so (declared in include/swa.h): argument
// validation, dispatch to the HIP launchers, status codes, test hooks.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "../../include/swa.h"
#include "schedule.h"

namespace swa {
hipError_t launch_prefill(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int heads,
                          int kv_heads, int n, int d, int w, int g, float scale, float sink_bias, bool bf16,
                          hipStream_t stream);
hipError_t launch_decode(const void *q, const void *kc, const void *vc, const int64_t *pos, void *o, float *lse,
                         int batch, int heads, int kv_heads, int d, int w, int g, float scale, float sink_bias,
                         bool bf16, void *ws, hipStream_t stream);
hipError_t launch_kv_append(void *kc, void *vc, const void *kn, const void *vn, const int64_t *pos, int batch,
                            int heads, int tn, int d, int w, int g, bool bf16, hipStream_t stream);
size_t decode_workspace_bytes(int batch, int heads, int kv_heads, int d, int rows, int kind);
int decode_kind(bool bf16, bool fp8, int heads, int kv_heads);
hipError_t launch_chunk_prefill(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                                const void *v_cache, const int64_t *pos, void *o, float *lse, int batch, int heads,
                                int kv_heads, int t, int d, int w, int g, float scale, float sink_bias, int part,
                                bool bf16, hipStream_t stream);
hipError_t launch_dilated_prefill(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                                  int heads, int kv_heads, int n, int d, int w, int r, float scale, bool bf16,
                                  hipStream_t stream);
hipError_t launch_landmark_part(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                                int heads, int kv_heads, int n, int d, int w, int g, int r, float scale, bool bf16,
                                hipStream_t stream);
hipError_t launch_landmark_prefill(const void *q, const void *k, const void *v, void *o, float *lse, int batch,
                                   int heads, int kv_heads, int n, int d, int w, int g, int r, float scale,
                                   float sink_bias, hipStream_t stream);
hipError_t launch_kv_append_fp8(void *kc, void *vc, const void *kn, const void *vn, const int64_t *pos,
                                const float *ksc, const float *vsc, int batch, int heads, int tn, int d, int w,
                                int g, bool bf16, hipStream_t stream);
hipError_t launch_decode_fp8(const void *q, const void *kc, const void *vc, const float *ksc, const float *vsc,
                             const int64_t *pos, void *o, float *lse, int batch, int heads, int kv_heads, int d,
                             int w, int g, float scale, float sink_bias, bool bf16, void *ws, hipStream_t stream);
hipError_t launch_lse_merge(const void *oa, const float *la, const void *ob, const float *lb, void *o, float *lse,
                            long rows, int d, bool bf16, hipStream_t stream);
int prefill_rows_per_workgroup(bool bf16);
hipError_t launch_decode_noalloc(const void *q, const void *kc, const void *vc, const int64_t *pos, void *o,
                                 float *lse, int batch, int heads, int kv_heads, int d, int w, int g, float scale,
                                 float sink_bias, bool bf16, hipStream_t stream);
size_t decode_scratch_bytes();
// keys per prefill tile (prefill.hip)
constexpr int kPrefillBK = 64;
inline int prefill_bq(bool bf16) { return prefill_rows_per_workgroup(bf16); }
}  // namespace swa

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_dtype_d(swa_dtype_t dtype, int d) {
    if (dtype != SWA_F32 && dtype != SWA_BF16) return SWA_EUNSUPPORTED;
    if (d != 64 && d != 128) return SWA_EUNSUPPORTED;
    return SWA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? SWA_OK : SWA_EHIP; }

// Whether a prefill grid of units x query blocks fits in INT_MAX workgroups
// (each product checked before it is formed: batch x heads alone can pass
// 2^62).
bool prefill_grid_fits(int batch, int heads, int units_mul, long long nqb) {
    long long units = (long long)batch * heads;  // < 2^62
    if (units > INT_MAX / units_mul) return false;
    units *= units_mul;
    return units <= INT_MAX / nqb;
}

// Whether the append grid (one thread per 16-byte chunk of each appended row,
// 256 threads per workgroup) fits in INT_MAX workgroups: batch x heads x
// tokens x chunks, each product checked before it is formed.
bool append_grid_fits(int batch, int heads, int t_new, int chunks_per_row) {
    const long long limit = (long long)INT_MAX * 256;  // chunks that INT_MAX workgroups cover
    long long chunks = (long long)batch * heads;        // < 2^62
    if (chunks > limit / t_new) return false;
    chunks *= t_new;
    return chunks <= limit / chunks_per_row;
}

}  // namespace

extern "C" {

const char *swa_strerror(int status) {
    switch (status) {
        case SWA_OK: return "ok";
        case SWA_EINVAL: return "invalid argument (size, count, scale or null pointer)";
        case SWA_EUNSUPPORTED: return "unsupported head dimension or dtype (d must be 64 or 128; f32 or bf16)";
        case SWA_EALIGN: return "pointer not aligned (tensors need 16 bytes, lse 4 bytes)";
        case SWA_EHIP: return "the HIP runtime rejected a launch";
        case SWA_EWORKSPACE: return "decode workspace missing or too small";
        case SWA_ESCRATCH: return "the shape needs more than the library's fixed decode scratch";
        default: return "unknown status";
    }
}

int swa_prefill_fwd_gqa(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int heads,
                        int kv_heads, int n, int d, int w, int g, float scale, float sink_bias, swa_dtype_t dtype,
                        hipStream_t stream) {
    if (!q || !k || !v || !o) return SWA_EINVAL;
    if (batch < 1 || heads < 1 || n < 1 || w < 1 || g < 0) return SWA_EINVAL;
    if (g > n) g = n;  // every position a sink either way (and the tile arithmetic stays in int)
    if (kv_heads < 1 || kv_heads > heads || heads % kv_heads != 0) return SWA_EINVAL;
    if (!std::isfinite(scale) || !(scale > 0.f) || !std::isfinite(sink_bias)) return SWA_EINVAL;
    int st = check_dtype_d(dtype, d);
    if (st != SWA_OK) return st;
    const int bq = swa::prefill_bq(dtype == SWA_BF16);
    if (n > INT_MAX - bq) return SWA_EINVAL;
    if (!prefill_grid_fits(batch, heads, 1, (n + bq - 1) / bq)) return SWA_EINVAL;
    // byte offsets within one (batch, head)'s rows stay below 2^32 for the buffer loads
    if ((long long)n * d * (dtype == SWA_BF16 ? 2 : 4) >= (1LL << 32)) return SWA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned4(lse)))
        return SWA_EALIGN;
    return status_of(swa::launch_prefill(q, k, v, o, lse, batch, heads, kv_heads, n, d, w, g, scale, sink_bias,
                                         dtype == SWA_BF16, stream));
}

int swa_prefill_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int heads, int n,
                    int d, int w, int g, float scale, float sink_bias, swa_dtype_t dtype, hipStream_t stream) {
    return swa_prefill_fwd_gqa(q, k, v, o, lse, batch, heads, heads, n, d, w, g, scale, sink_bias, dtype, stream);
}

int swa_kv_append(void *k_cache, void *v_cache, const void *k_new, const void *v_new, const int64_t *pos,
                  int batch, int heads, int t_new, int d, int w, int g, swa_dtype_t dtype, hipStream_t stream) {
    if (!k_cache || !v_cache || !k_new || !v_new || !pos) return SWA_EINVAL;
    if (batch < 1 || heads < 1 || t_new < 0 || w < 1 || g < 0) return SWA_EINVAL;
    if ((long long)g + w > INT_MAX) return SWA_EINVAL;
    int st = check_dtype_d(dtype, d);
    if (st != SWA_OK) return st;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new) ||
        (reinterpret_cast<uintptr_t>(pos) & 7u))
        return SWA_EALIGN;
    if (t_new == 0) return SWA_OK;
    if (!append_grid_fits(batch, heads, t_new, d * (dtype == SWA_BF16 ? 2 : 4) / 16)) return SWA_EINVAL;
    return status_of(swa::launch_kv_append(k_cache, v_cache, k_new, v_new, pos, batch, heads, t_new, d, w, g,
                                           dtype == SWA_BF16, stream));
}

// shared checks of the whole-sequence prefill forms
static int check_prefill(const void *q, const void *k, const void *v, const void *o, const float *lse, int batch,
                         int heads, int kv_heads, int n, int d, int w, int g, float scale, float sink_bias,
                         swa_dtype_t dtype, int units_mul) {
    if (!q || !k || !v || !o) return SWA_EINVAL;
    if (batch < 1 || heads < 1 || n < 1 || w < 1 || g < 0) return SWA_EINVAL;
    if (kv_heads < 1 || kv_heads > heads || heads % kv_heads != 0) return SWA_EINVAL;
    if (!std::isfinite(scale) || !(scale > 0.f) || !std::isfinite(sink_bias)) return SWA_EINVAL;
    int st = check_dtype_d(dtype, d);
    if (st != SWA_OK) return st;
    const int bq = swa::prefill_bq(dtype == SWA_BF16);
    if (n > INT_MAX - bq) return SWA_EINVAL;
    if (!prefill_grid_fits(batch, heads, units_mul, (n + bq - 1) / bq)) return SWA_EINVAL;
    const long long row_bytes = (long long)d * (dtype == SWA_BF16 ? 2 : 4);
    if ((long long)n * row_bytes >= (1LL << 32)) return SWA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned4(lse)))
        return SWA_EALIGN;
    return SWA_OK;
}

int swa_dilated_prefill_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int heads,
                            int kv_heads, int n, int d, int w, int r, float scale, swa_dtype_t dtype,
                            hipStream_t stream) {
    if (r < 1) return SWA_EINVAL;
    if (n >= 1 && r > n) r = n;  // every stride >= n reads the same keys (each query only itself)
    int st = check_prefill(q, k, v, o, lse, batch, heads, kv_heads, n, d, w, 0, scale, 0.f, dtype, r);
    if (st != SWA_OK) return st;
    return status_of(swa::launch_dilated_prefill(q, k, v, o, lse, batch, heads, kv_heads, n, d, w, r, scale,
                                                 dtype == SWA_BF16, stream));
}

size_t swa_landmark_workspace_bytes(int batch, int heads, int n, int d, swa_dtype_t dtype) {
    if (batch < 1 || heads < 1 || n < 1 || (d != 64 && d != 128) || (dtype != SWA_F32 && dtype != SWA_BF16))
        return 0;
    if (dtype == SWA_BF16) return 0;  // one launch over landmark, window and sink tiles
    const size_t rows = (size_t)batch * heads * n;
    const size_t lb = (rows * 4 + 255) / 256 * 256;
    const size_t ob = (rows * d * 4 + 255) / 256 * 256;
    return ob + 2 * lb;  // fp32: the landmark part's o and both LSEs, merged by a third launch
}

int swa_landmark_prefill_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int batch, int heads,
                             int kv_heads, int n, int d, int w, int g, int r, float scale, float sink_bias,
                             swa_dtype_t dtype, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (r < 1) return SWA_EINVAL;
    if (n >= 1 && r > n) r = n;  // every stride >= n has the one landmark 0
    int st = check_prefill(q, k, v, o, lse, batch, heads, kv_heads, n, d, w, g, scale, sink_bias, dtype, 1);
    if (st != SWA_OK) return st;
    if (g > n) g = n;  // every position a sink (and no landmark) either way
    const size_t need = swa_landmark_workspace_bytes(batch, heads, n, d, dtype);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return SWA_EWORKSPACE;
        if (!aligned16(workspace)) return SWA_EALIGN;
    }
    const bool bf16 = dtype == SWA_BF16;
    if (bf16)
        return status_of(swa::launch_landmark_prefill(q, k, v, o, lse, batch, heads, kv_heads, n, d, w, g, r, scale,
                                                      sink_bias, stream));
    const size_t rows = (size_t)batch * heads * n;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    void *o_b = ws;
    float *lse_a = reinterpret_cast<float *>(ws + (rows * d * (bf16 ? 2 : 4) + 255) / 256 * 256);
    float *lse_b = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(lse_a) + (rows * 4 + 255) / 256 * 256);
    // window and sinks into o, landmarks into the workspace, then the LSE merge into o
    hipError_t e = swa::launch_prefill(q, k, v, o, lse_a, batch, heads, kv_heads, n, d, w, g, scale, sink_bias, bf16,
                                       stream);
    if (e == hipSuccess)
        e = swa::launch_landmark_part(q, k, v, o_b, lse_b, batch, heads, kv_heads, n, d, w, g, r, scale, bf16,
                                      stream);
    if (e == hipSuccess) e = swa::launch_lse_merge(o, lse_a, o_b, lse_b, o, lse, (long)rows, d, bf16, stream);
    return status_of(e);
}

int swa_chunk_prefill_fwd(const void *q, const void *k_new, const void *v_new, const void *k_cache,
                          const void *v_cache, const int64_t *pos, void *o, float *lse, int batch, int heads,
                          int kv_heads, int t, int d, int w, int g, float scale, float sink_bias, int keys,
                          swa_dtype_t dtype, hipStream_t stream) {
    if (!q || !k_new || !v_new || !k_cache || !v_cache || !pos || !o) return SWA_EINVAL;
    if (batch < 1 || heads < 1 || t < 1 || w < 1 || g < 0) return SWA_EINVAL;
    if (kv_heads < 1 || kv_heads > heads || heads % kv_heads != 0) return SWA_EINVAL;
    if (keys != SWA_KEYS_ALL && keys != SWA_KEYS_CACHE && keys != SWA_KEYS_CHUNK) return SWA_EINVAL;
    if ((long long)g + w > INT_MAX / 2) return SWA_EINVAL;
    if (!std::isfinite(scale) || !(scale > 0.f) || !std::isfinite(sink_bias)) return SWA_EINVAL;
    int st = check_dtype_d(dtype, d);
    if (st != SWA_OK) return st;
    const int bq = swa::prefill_bq(dtype == SWA_BF16);
    if (t > INT_MAX - bq) return SWA_EINVAL;
    if (!prefill_grid_fits(batch, heads, 1, (t + bq - 1) / bq)) return SWA_EINVAL;
    // byte offsets of one (batch, head)'s rows stay below 2^32 for the buffer loads
    const long long row_bytes = (long long)d * (dtype == SWA_BF16 ? 2 : 4);
    if ((long long)t * row_bytes >= (1LL << 32) || ((long long)g + w) * row_bytes >= (1LL << 32)) return SWA_EINVAL;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache) ||
        !aligned16(o) || (reinterpret_cast<uintptr_t>(pos) & 7u) || (lse && !aligned4(lse)))
        return SWA_EALIGN;
    return status_of(swa::launch_chunk_prefill(q, k_new, v_new, k_cache, v_cache, pos, o, lse, batch, heads,
                                               kv_heads, t, d, w, g, scale, sink_bias, keys, dtype == SWA_BF16,
                                               stream));
}

int swa_lse_merge(const void *o_a, const float *lse_a, const void *o_b, const float *lse_b, void *o, float *lse,
                  long long rows, int d, swa_dtype_t dtype, hipStream_t stream) {
    if (!o_a || !lse_a || !o_b || !lse_b || !o) return SWA_EINVAL;
    if (rows < 1) return SWA_EINVAL;
    int st = check_dtype_d(dtype, d);
    if (st != SWA_OK) return st;
    // one thread per 4 columns of a row, 256 per workgroup: at most INT_MAX - 1
    // workgroups (rows x (d/4) is not formed: rows can be near LLONG_MAX)
    if (rows > ((long long)INT_MAX - 1) * 256 / (d / 4)) return SWA_EINVAL;
    if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o) || !aligned4(lse_a) || !aligned4(lse_b) ||
        (lse && !aligned4(lse)))
        return SWA_EALIGN;
    return status_of(swa::launch_lse_merge(o_a, lse_a, o_b, lse_b, o, lse, (long)rows, d, dtype == SWA_BF16, stream));
}

int swa_kv_append_fp8(void *k_cache, void *v_cache, const void *k_new, const void *v_new, const int64_t *pos,
                      const float *k_scale, const float *v_scale, int batch, int heads, int t_new, int d, int w,
                      int g, swa_dtype_t dtype, hipStream_t stream) {
    if (!k_cache || !v_cache || !k_new || !v_new || !pos || !k_scale || !v_scale) return SWA_EINVAL;
    if (batch < 1 || heads < 1 || t_new < 0 || w < 1 || g < 0) return SWA_EINVAL;
    if ((long long)g + w > INT_MAX) return SWA_EINVAL;
    int st = check_dtype_d(dtype, d);
    if (st != SWA_OK) return st;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new) ||
        (reinterpret_cast<uintptr_t>(pos) & 7u) || !aligned4(k_scale) || !aligned4(v_scale))
        return SWA_EALIGN;
    if (t_new == 0) return SWA_OK;
    if (!append_grid_fits(batch, heads, t_new, d / 8)) return SWA_EINVAL;
    return status_of(swa::launch_kv_append_fp8(k_cache, v_cache, k_new, v_new, pos, k_scale, v_scale, batch, heads,
                                               t_new, d, w, g, dtype == SWA_BF16, stream));
}

int swa_decode_fwd_fp8(const void *q, const void *k_cache, const void *v_cache, const float *k_scale,
                       const float *v_scale, const int64_t *pos, void *o, float *lse, int batch, int heads,
                       int kv_heads, int d, int w, int g, float scale, float sink_bias, swa_dtype_t dtype,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !k_scale || !v_scale || !pos || !o) return SWA_EINVAL;
    if (batch < 1 || heads < 1 || w < 1 || g < 0) return SWA_EINVAL;
    if (kv_heads < 1 || kv_heads > heads || heads % kv_heads != 0) return SWA_EINVAL;
    if ((long long)g + w > INT_MAX / 2) return SWA_EINVAL;
    if ((long long)batch * heads > INT_MAX / 64) return SWA_EINVAL;
    if (((long long)g + w) * d * 4 >= (1LL << 32)) return SWA_EINVAL;  // cache bytes of one head, buffer offsets
    if (!std::isfinite(scale) || !(scale > 0.f) || !std::isfinite(sink_bias)) return SWA_EINVAL;
    int st = check_dtype_d(dtype, d);
    if (st != SWA_OK) return st;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
        (reinterpret_cast<uintptr_t>(pos) & 7u) || (lse && !aligned4(lse)) || !aligned4(k_scale) ||
        !aligned4(v_scale))
        return SWA_EALIGN;
    const size_t need = swa::decode_workspace_bytes(batch, heads, kv_heads, d, g + w, 1);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return SWA_EWORKSPACE;
        if (!aligned16(workspace)) return SWA_EALIGN;
    }
    return status_of(swa::launch_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, pos, o, lse, batch, heads,
                                            kv_heads, d, w, g, scale, sink_bias, dtype == SWA_BF16, workspace,
                                            stream));
}

size_t swa_decode_workspace_bytes_gqa(int batch, int heads, int kv_heads, int d, int w, int g) {
    if (batch < 1 || heads < 1 || w < 1 || g < 0 || (d != 64 && d != 128)) return 0;
    if (kv_heads < 1 || kv_heads > heads || heads % kv_heads != 0) return 0;
    if ((long long)g + w > INT_MAX / 2 || (long long)batch * heads > INT_MAX / 64) return 0;
    return swa::decode_workspace_bytes(batch, heads, kv_heads, d, g + w, -1);
}

size_t swa_decode_workspace_bytes(int batch, int heads, int d, int w, int g) {
    return swa_decode_workspace_bytes_gqa(batch, heads, heads, d, w, g);
}

int swa_decode_fwd_gqa(const void *q, const void *k_cache, const void *v_cache, const int64_t *pos, void *o,
                       float *lse, int batch, int heads, int kv_heads, int d, int w, int g, float scale,
                       float sink_bias, swa_dtype_t dtype, void *workspace, size_t workspace_bytes,
                       hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !pos || !o) return SWA_EINVAL;
    if (batch < 1 || heads < 1 || w < 1 || g < 0) return SWA_EINVAL;
    if (kv_heads < 1 || kv_heads > heads || heads % kv_heads != 0) return SWA_EINVAL;
    if ((long long)g + w > INT_MAX / 2) return SWA_EINVAL;
    if ((long long)batch * heads > INT_MAX / 64) return SWA_EINVAL;
    if (((long long)g + w) * d * 4 >= (1LL << 32)) return SWA_EINVAL;  // cache bytes of one head, buffer offsets
    if (!std::isfinite(scale) || !(scale > 0.f) || !std::isfinite(sink_bias)) return SWA_EINVAL;
    int st = check_dtype_d(dtype, d);
    if (st != SWA_OK) return st;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
        (reinterpret_cast<uintptr_t>(pos) & 7u) || (lse && !aligned4(lse)))
        return SWA_EALIGN;
    const size_t need = swa::decode_workspace_bytes(batch, heads, kv_heads, d, g + w,
                                                    swa::decode_kind(dtype == SWA_BF16, false, heads, kv_heads));
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return SWA_EWORKSPACE;
        if (!aligned16(workspace)) return SWA_EALIGN;
    }
    return status_of(swa::launch_decode(q, k_cache, v_cache, pos, o, lse, batch, heads, kv_heads, d, w, g, scale,
                                        sink_bias, dtype == SWA_BF16, workspace, stream));
}

int swa_decode_fwd_gqa_noalloc(const void *q, const void *k_cache, const void *v_cache, const int64_t *pos, void *o,
                               float *lse, int batch, int heads, int kv_heads, int d, int w, int g, float scale,
                               float sink_bias, swa_dtype_t dtype, hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !pos || !o) return SWA_EINVAL;
    if (batch < 1 || heads < 1 || w < 1 || g < 0) return SWA_EINVAL;
    if (kv_heads < 1 || kv_heads > heads || heads % kv_heads != 0) return SWA_EINVAL;
    if ((long long)g + w > INT_MAX / 2) return SWA_EINVAL;
    if ((long long)batch * heads > INT_MAX / 64) return SWA_EINVAL;
    if (((long long)g + w) * d * 4 >= (1LL << 32)) return SWA_EINVAL;
    if (!std::isfinite(scale) || !(scale > 0.f) || !std::isfinite(sink_bias)) return SWA_EINVAL;
    int st = check_dtype_d(dtype, d);
    if (st != SWA_OK) return st;
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
        (reinterpret_cast<uintptr_t>(pos) & 7u) || (lse && !aligned4(lse)))
        return SWA_EALIGN;
    const size_t need = swa::decode_workspace_bytes(batch, heads, kv_heads, d, g + w,
                                                    swa::decode_kind(dtype == SWA_BF16, false, heads, kv_heads));
    if (need > swa::decode_scratch_bytes()) return SWA_ESCRATCH;
    return status_of(swa::launch_decode_noalloc(q, k_cache, v_cache, pos, o, lse, batch, heads, kv_heads, d, w, g,
                                                scale, sink_bias, dtype == SWA_BF16, stream));
}

size_t swa_decode_scratch_bytes(void) { return swa::decode_scratch_bytes(); }

int swa_decode_fwd(const void *q, const void *k_cache, const void *v_cache, const int64_t *pos, void *o, float *lse,
                   int batch, int heads, int d, int w, int g, float scale, float sink_bias, swa_dtype_t dtype,
                   void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return swa_decode_fwd_gqa(q, k_cache, v_cache, pos, o, lse, batch, heads, heads, d, w, g, scale, sink_bias, dtype,
                              workspace, workspace_bytes, stream);
}

long swa_band_tiles(int n, int w, int g, int bq, int bk, int *out, long cap) {
    if (n < 1 || w < 1 || g < 0 || bq < 1 || bk < 1 || cap < 0 || (cap > 0 && !out)) return SWA_EINVAL;
    // the block and tile arithmetic (q0 + bq, the last key of a tile) stays within int
    if (n > INT_MAX - bq || n > INT_MAX - bk) return SWA_EINVAL;
    if (g > n) g = n;  // the same tiles and FULL tests (every position a sink)
    long count = 0;
    const int nqb = (n + bq - 1) / bq;
    for (int qb = 0; qb < nqb; ++qb) {
        const int q0 = qb * bq;
        const int q1 = (q0 + bq < n ? q0 + bq : n) - 1;
        const swa::BandRange r = swa::band_range(q0, q1, w, g, bk);
        int t_lo, t_hi;  // the kernels' closed form; the per-tile test must agree with it
        swa::full_range(r, q0, q1, n, w, g, bk, &t_lo, &t_hi);
        for (int t = 0; t < r.count(); ++t) {
            const int kb = r.block(t);
            const int full = swa::tile_full(q0, q1, kb * bk, kb * bk + bk - 1, n, w, g) ? 1 : 0;
            if (full != ((t >= t_lo && t < t_hi) ? 1 : 0)) return SWA_EINVAL;
            if (count < cap) {
                out[3 * count + 0] = qb;
                out[3 * count + 1] = kb;
                out[3 * count + 2] = full;
            }
            ++count;
        }
    }
    return count;
}

int swa_prefill_tile_shape(swa_dtype_t dtype, int d, int *bq, int *bk) {
    int st = check_dtype_d(dtype, d);
    if (st != SWA_OK) return st;
    if (!bq || !bk) return SWA_EINVAL;
    *bq = swa::prefill_bq(dtype == SWA_BF16);
    *bk = swa::kPrefillBK;
    return SWA_OK;
}

long swa_prefill_order(int units, int nqb, int group, int *out, long cap) {
    if (units < 1 || nqb < 1 || group < 1 || units % group != 0 || cap < 0 || (cap > 0 && !out)) return SWA_EINVAL;
    const long long total = (long long)units * nqb;
    if (total > INT_MAX) return SWA_EINVAL;
    for (long long bid = 0; bid < total; ++bid) {
        int u, qb;
        swa::workgroup_order((int)bid, (int)total, nqb, group, &u, &qb);
        if (bid < cap) {
            out[2 * bid] = u;
            out[2 * bid + 1] = qb;
        }
    }
    return (long)total;
}

}  // extern "C"
