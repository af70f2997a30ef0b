// Host-only stand-ins for the kernel launchers that api.cpp calls (the real
// ones are in the HIP sources and launch GPU work).  Each records the call;
// the sizing hooks return fixed, plausible values.  Test infrastructure only:
// linked into the sanitizer build of the C ABI by tests/test_host_sanitizers.py.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

int g_launches = 0;  // launcher calls since the last reset
int g_last_batch = -1, g_last_heads = -1, g_last_n = -1, g_last_r = -1;

namespace swa {
static hipError_t record(int batch, int heads, int n, int r = -1) {
    ++g_launches;
    g_last_batch = batch;
    g_last_heads = heads;
    g_last_n = n;
    g_last_r = r;
    return hipSuccess;
}
hipError_t launch_prefill(const void *, const void *, const void *, void *, float *, int batch, int heads, int,
                          int n, int, int, int, float, float, bool, hipStream_t) {
    return record(batch, heads, n);
}
hipError_t launch_decode(const void *, const void *, const void *, const int64_t *, void *, float *, int batch,
                         int heads, int, int, int w, int, float, float, bool, void *, hipStream_t) {
    return record(batch, heads, w);
}
hipError_t launch_kv_append(void *, void *, const void *, const void *, const int64_t *, int batch, int heads,
                            int tn, int, int, int, bool, hipStream_t) {
    return record(batch, heads, tn);
}
// the decode launch of the given kind splits when it has few (batch, head) jobs
size_t decode_workspace_bytes(int batch, int heads, int, int d, int, int) {
    return (batch * (size_t)heads < 64) ? (size_t)batch * heads * 4 * (2 + d) * sizeof(float) : 0;
}
int decode_kind(bool bf16, bool fp8, int heads, int kv_heads) {
    if (fp8) return 1;
    return (bf16 && heads / kv_heads >= 2) ? 2 : 0;
}
hipError_t launch_chunk_prefill(const void *, const void *, const void *, const void *, const void *,
                                const int64_t *, void *, float *, int batch, int heads, int, int t, int, int, int,
                                float, float, int, bool, hipStream_t) {
    return record(batch, heads, t);
}
hipError_t launch_dilated_prefill(const void *, const void *, const void *, void *, float *, int batch, int heads, int,
                                  int n, int, int, int r, float, bool, hipStream_t) {
    return record(batch, heads, n, r);
}
hipError_t launch_landmark_part(const void *, const void *, const void *, void *, float *, int batch, int heads,
                                int, int n, int, int, int, int r, float, bool, hipStream_t) {
    return record(batch, heads, n, r);
}
hipError_t launch_landmark_prefill(const void *, const void *, const void *, void *, float *, int batch, int heads,
                                   int, int n, int, int, int, int r, float, float, hipStream_t) {
    return record(batch, heads, n, r);
}
hipError_t launch_kv_append_fp8(void *, void *, const void *, const void *, const int64_t *, const float *,
                                const float *, int batch, int heads, int tn, int, int, int, bool, hipStream_t) {
    return record(batch, heads, tn);
}
hipError_t launch_decode_fp8(const void *, const void *, const void *, const float *, const float *,
                             const int64_t *, void *, float *, int batch, int heads, int, int, int w, int, float,
                             float, bool, void *, hipStream_t) {
    return record(batch, heads, w);
}
hipError_t launch_lse_merge(const void *, const float *, const void *, const float *, void *, float *, long rows,
                            int d, bool, hipStream_t) {
    return record((int)(rows > 0x7fffffff ? -2 : rows), d, 0);
}
int prefill_rows_per_workgroup(bool) { return 128; }
hipError_t launch_decode_noalloc(const void *, const void *, const void *, const int64_t *, void *, float *,
                                 int batch, int heads, int, int, int w, int, float, float, bool, hipStream_t) {
    return record(batch, heads, w);
}
size_t decode_scratch_bytes() { return (size_t)16 << 20; }
}  // namespace swa
