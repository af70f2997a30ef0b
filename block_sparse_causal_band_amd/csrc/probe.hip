// probe.hip -- measurement kernels: the rates the attention kernels are also
// compared against, measured on the chip that runs them (the datasheet peaks
// assume the top clock, which a power-limited dense load does not hold).
//  * probe_mfma_kernel: v_mfma_f32_32x32x16_bf16 back to back on register
//    operands, four independent accumulator chains per wave, so the matrix
//    core never waits on a result; no memory traffic inside the loop.
//  * probe_read_kernel: each workgroup streams one contiguous range of a
//    buffer as `streams` interleaved sub-ranges (as a decode workgroup reads
//    its K and V rows), 16-byte non-temporal loads, 8 per lane in flight;
//    every wave load instruction covers 1 KB of consecutive bytes.
#include "common.h"
#include "swa.h"
#include "swa_probe.h"

namespace swa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeChains = 4;  // independent accumulators per wave
constexpr int kReadDepth = 8;    // 16-byte loads per lane per round

__global__ __launch_bounds__(kProbeThreads) void probe_mfma_kernel(float *__restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        // small values: iters * 16 * 4 products of at most 5e-5 stay far from overflow
        a[e] = static_cast<__bf16>(1e-3f * (float)((lane + e) & 7));
        b[e] = static_cast<__bf16>(1e-3f * (float)((3 * lane + e) & 7));
    }
    f32x16 acc[kProbeChains];
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    for (int i = 0; i < iters; ++i)  // the loop's scalar work issues beside the 4 MFMAs
#pragma unroll
        for (int j = 0; j < kProbeChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[(size_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// per_wg bytes per workgroup, split into `streams` equal sub-ranges; one
// round reads kReadDepth 4 KB blocks (256 lanes x 16 bytes), spread over the
// streams round-robin.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint8_t *__restrict__ buf, size_t per_wg,
                                                                   int streams, uint32_t *__restrict__ sink) {
    const size_t per_stream = per_wg / streams;
    const uint8_t *base = buf + (size_t)blockIdx.x * per_wg + 16 * threadIdx.x;
    const int per_round = kReadDepth / streams;  // blocks of each stream per round
    const size_t rounds = per_stream / ((size_t)4096 * per_round);
    uint32_t x = 0;
    for (size_t rd = 0; rd < rounds; ++rd) {
        uint4 v[kReadDepth];
#pragma unroll
        for (int u = 0; u < kReadDepth; ++u) {
            const int s = u % streams, blk = u / streams;
            v[u] = load_stream16(base + s * per_stream + (rd * per_round + blk) * 4096);
        }
#pragma unroll
        for (int u = 0; u < kReadDepth; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    // every lane's loads stay live through the compare; the store is rare
    if (x == 0x9e3779b9u) sink[blockIdx.x] = x;
}

}  // namespace
}  // namespace swa

extern "C" {

int swa_probe_mfma_bf16(float *out, int workgroups, int iters, hipStream_t stream) {
    if (!out || workgroups < 1 || iters < 1) return SWA_EINVAL;
    if ((reinterpret_cast<uintptr_t>(out) & 3u) != 0) return SWA_EALIGN;
    hipLaunchKernelGGL(swa::probe_mfma_kernel, dim3(workgroups), dim3(swa::kProbeThreads), 0, stream, out, iters);
    return hipGetLastError() == hipSuccess ? SWA_OK : SWA_EHIP;
}

double swa_probe_mfma_bf16_flops(int workgroups, int iters) {
    if (workgroups < 1 || iters < 1) return 0.0;
    return (double)workgroups * (swa::kProbeThreads / 64) * iters * swa::kProbeChains * 32.0 * 32.0 * 16.0 * 2.0;
}

int swa_probe_hbm_read(const void *buf, size_t bytes, int workgroups, int streams, uint32_t *sink,
                       hipStream_t stream) {
    if (!buf || !sink || workgroups < 1 || bytes == 0) return SWA_EINVAL;
    if (streams != 1 && streams != 2 && streams != 4 && streams != 8) return SWA_EINVAL;
    const size_t round = (size_t)16 * swa::kProbeThreads * swa::kReadDepth;  // 32 KB per workgroup round
    if (bytes % ((size_t)workgroups * round) != 0) return SWA_EINVAL;
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return SWA_EALIGN;
    hipLaunchKernelGGL(swa::probe_read_kernel, dim3(workgroups), dim3(swa::kProbeThreads), 0, stream,
                       static_cast<const uint8_t *>(buf), bytes / workgroups, streams, sink);
    return hipGetLastError() == hipSuccess ? SWA_OK : SWA_EHIP;
}

}  // extern "C"
