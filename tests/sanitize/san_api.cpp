// Host-only run of the C ABI's argument validation and size arithmetic
// (block_sparse_causal_band_amd/csrc/api.cpp), built with AddressSanitizer and
// UndefinedBehaviorSanitizer against the launcher stand-ins of api_stubs.cpp
// by tests/test_host_sanitizers.py, as an executable of its own.  Test
// infrastructure only.
//
// Every entry point is called on valid arguments (it must return SWA_OK and
// reach its launcher with the caller's sizes), on each kind of invalid
// argument (the documented status, no launch), and on sizes at the edges of
// the int and size_t ranges, where any intermediate product that overflowed
// would be undefined behaviour and stop the run.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "swa.h"

extern int g_launches;
extern int g_last_batch, g_last_heads, g_last_n, g_last_r;

static int failures = 0;
#define CHECK(cond, ...)                                              \
    do {                                                              \
        if (!(cond)) {                                                \
            std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                        \
            std::fprintf(stderr, "\n");                               \
            ++failures;                                               \
        }                                                             \
    } while (0)

// status of a call and whether it launched
#define EXPECT(call, want, launched)                                                                   \
    do {                                                                                               \
        const int before = g_launches;                                                                 \
        const int st = (call);                                                                         \
        CHECK(st == (want), "%s -> %d, want %d", #call, st, (int)(want));                              \
        CHECK((g_launches != before) == (launched), "%s launched %d times", #call, g_launches - before); \
    } while (0)

// stand-ins for device pointers: never dereferenced on the host path
alignas(256) static unsigned char arena[4096];
static void *P = arena;
static void *P8 = arena + 8;  // 8-byte aligned only
static const int64_t *POS = reinterpret_cast<const int64_t *>(arena + 64);
static const int64_t *POS4 = reinterpret_cast<const int64_t *>(arena + 68);  // not 8-byte aligned
static float *F = reinterpret_cast<float *>(arena + 128);
static hipStream_t S = nullptr;

static void prefill_cases() {
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 2, 4, 300, 128, 70, 4, 0.125f, 1.f, SWA_BF16, S), SWA_OK, true);
    CHECK(g_last_batch == 2 && g_last_heads == 4 && g_last_n == 300, "prefill launch sizes");
    EXPECT(swa_prefill_fwd(P, P, P, P, nullptr, 1, 1, 1, 64, 1, 0, 1.f, 0.f, SWA_F32, S), SWA_OK, true);
    EXPECT(swa_prefill_fwd_gqa(P, P, P, P, F, 1, 32, 8, 16384, 128, 4096, 0, 0.088f, 0.f, SWA_BF16, S), SWA_OK, true);
    // invalid
    EXPECT(swa_prefill_fwd(nullptr, P, P, P, F, 1, 1, 16, 128, 4, 0, 1.f, 0.f, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 0, 1, 16, 128, 4, 0, 1.f, 0.f, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 1, 1, 16, 128, 0, 0, 1.f, 0.f, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 1, 1, 16, 128, 4, -1, 1.f, 0.f, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 1, 1, 16, 96, 4, 0, 1.f, 0.f, SWA_BF16, S), SWA_EUNSUPPORTED, false);
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 1, 1, 16, 128, 4, 0, 1.f, 0.f, (swa_dtype_t)7, S), SWA_EUNSUPPORTED, false);
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 1, 1, 16, 128, 4, 0, NAN, 0.f, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 1, 1, 16, 128, 4, 0, -1.f, 0.f, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 1, 1, 16, 128, 4, 0, 1.f, INFINITY, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_prefill_fwd(P8, P, P, P, F, 1, 1, 16, 128, 4, 0, 1.f, 0.f, SWA_BF16, S), SWA_EALIGN, false);
    EXPECT(swa_prefill_fwd_gqa(P, P, P, P, F, 1, 6, 4, 16, 128, 4, 0, 1.f, 0.f, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_prefill_fwd_gqa(P, P, P, P, F, 1, 4, 8, 16, 128, 4, 0, 1.f, 0.f, SWA_BF16, S), SWA_EINVAL, false);
    // sizes at the edges: n near INT_MAX, batch x heads x blocks past INT_MAX, rows past 4 GiB
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 1, 1, INT_MAX, 128, 4, 0, 1.f, 0.f, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_prefill_fwd(P, P, P, P, F, INT_MAX, INT_MAX, 1024, 128, 4, 0, 1.f, 0.f, SWA_BF16, S), SWA_EINVAL,
           false);
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 1, 1, 1 << 24, 128, 4, 0, 1.f, 0.f, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 1, 1, (1 << 24) - 128, 128, INT_MAX, INT_MAX, 1.f, 0.f, SWA_BF16, S),
           SWA_OK, true);
    // more sinks than positions: read as g = n (the tile arithmetic on g stays within int)
    EXPECT(swa_prefill_fwd(P, P, P, P, F, 1, 1, 300, 128, 16, INT_MAX, 1.f, 0.f, SWA_BF16, S), SWA_OK, true);
    EXPECT(swa_landmark_prefill_fwd(P, P, P, P, F, 1, 1, 1, 300, 128, 16, INT_MAX, 7, 1.f, 0.f, SWA_BF16, nullptr, 0,
                                    S),
           SWA_OK, true);
}

static void pattern_cases() {
    // dilated: a stride at or past n is clamped to n before any offset is formed
    EXPECT(swa_dilated_prefill_fwd(P, P, P, P, F, 1, 2, 2, 300, 128, 16, INT_MAX, 0.125f, SWA_BF16, S), SWA_OK,
           true);
    CHECK(g_last_r == 300, "dilated stride clamped to n: %d", g_last_r);
    EXPECT(swa_dilated_prefill_fwd(P, P, P, P, F, 1, 2, 2, 300, 128, 16, 0, 0.125f, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_dilated_prefill_fwd(P, P, P, P, F, INT_MAX, INT_MAX, 1, 4096, 128, 16, 4, 0.125f, SWA_BF16, S),
           SWA_EINVAL, false);
    // landmarks: bf16 needs no workspace; fp32 needs its workspace
    CHECK(swa_landmark_workspace_bytes(1, 2, 64, 128, SWA_BF16) == 0, "bf16 landmark workspace");
    const size_t lw = swa_landmark_workspace_bytes(1, 2, 64, 128, SWA_F32);
    CHECK(lw == 1 * 2 * 64 * 128 * 4 + 2 * 512, "fp32 landmark workspace %zu", lw);
    CHECK(swa_landmark_workspace_bytes(INT_MAX, INT_MAX, INT_MAX, 128, SWA_F32) > 0, "huge landmark workspace");
    CHECK(swa_landmark_workspace_bytes(1, 1, 1, 96, SWA_F32) == 0, "unsupported d");
    EXPECT(swa_landmark_prefill_fwd(P, P, P, P, F, 1, 2, 2, 300, 128, 64, 4, INT_MAX, 0.125f, 1.f, SWA_BF16, nullptr,
                                    0, S),
           SWA_OK, true);
    CHECK(g_last_r == 300, "landmark stride clamped to n: %d", g_last_r);
    EXPECT(swa_landmark_prefill_fwd(P, P, P, P, F, 1, 2, 2, 64, 128, 16, 4, 8, 0.125f, 1.f, SWA_F32, nullptr, 0, S),
           SWA_EWORKSPACE, false);
    EXPECT(swa_landmark_prefill_fwd(P, P, P, P, F, 1, 2, 2, 64, 128, 16, 4, 8, 0.125f, 1.f, SWA_F32, P8, lw, S),
           SWA_EALIGN, false);
    EXPECT(swa_landmark_prefill_fwd(P, P, P, P, F, 1, 2, 2, 64, 128, 16, 4, 8, 0.125f, 1.f, SWA_F32, P, lw, S),
           SWA_OK, true);
}

static void append_cases() {
    EXPECT(swa_kv_append(P, P, P, P, POS, 64, 32, 1, 128, 4096, 4, SWA_BF16, S), SWA_OK, true);
    EXPECT(swa_kv_append(P, P, P, P, POS, 64, 32, 0, 128, 4096, 4, SWA_BF16, S), SWA_OK, false);
    EXPECT(swa_kv_append(P, P, P, P, POS4, 1, 1, 1, 128, 16, 0, SWA_BF16, S), SWA_EALIGN, false);
    EXPECT(swa_kv_append(P, P, P, P, POS, 1, 1, 1, 128, INT_MAX, 1, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_kv_append(P, P, P, P, nullptr, 1, 1, 1, 128, 16, 0, SWA_BF16, S), SWA_EINVAL, false);
    // the grid size of a huge append: batch x heads x tokens x chunks, not formed in one product
    EXPECT(swa_kv_append(P, P, P, P, POS, INT_MAX, INT_MAX, INT_MAX, 128, 16, 0, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_kv_append(P, P, P, P, POS, INT_MAX, INT_MAX, 1, 128, 16, 0, SWA_F32, S), SWA_EINVAL, false);
    EXPECT(swa_kv_append_fp8(P, P, P, P, POS, F, F, 64, 32, 1, 128, 4096, 4, SWA_BF16, S), SWA_OK, true);
    EXPECT(swa_kv_append_fp8(P, P, P, P, POS, F, F, INT_MAX, INT_MAX, INT_MAX, 128, 16, 0, SWA_BF16, S), SWA_EINVAL,
           false);
    EXPECT(swa_kv_append_fp8(P, P, P, P, POS, nullptr, F, 1, 1, 1, 128, 16, 0, SWA_BF16, S), SWA_EINVAL, false);
}

static void decode_cases() {
    const size_t need = swa_decode_workspace_bytes(1, 8, 128, 4096, 4);
    CHECK(need > 0, "a small decode splits");
    EXPECT(swa_decode_fwd(P, P, P, POS, P, F, 1, 8, 128, 4096, 4, 0.088f, 1.f, SWA_BF16, P, need, S), SWA_OK, true);
    EXPECT(swa_decode_fwd(P, P, P, POS, P, F, 1, 8, 128, 4096, 4, 0.088f, 1.f, SWA_BF16, P, need - 1, S),
           SWA_EWORKSPACE, false);
    EXPECT(swa_decode_fwd(P, P, P, POS, P, F, 1, 8, 128, 4096, 4, 0.088f, 1.f, SWA_BF16, P8, need, S), SWA_EALIGN,
           false);
    EXPECT(swa_decode_fwd(P, P, P, POS, P, F, 64, 32, 128, 4096, 4, 0.088f, 1.f, SWA_BF16, nullptr, 0, S), SWA_OK,
           true);
    EXPECT(swa_decode_fwd_gqa(P, P, P, POS, P, F, 64, 32, 8, 128, 4096, 4, 0.088f, 0.f, SWA_BF16, nullptr, 0, S),
           SWA_OK, true);
    EXPECT(swa_decode_fwd_gqa(P, P, P, POS, P, F, 64, 32, 5, 128, 4096, 4, 0.088f, 0.f, SWA_BF16, nullptr, 0, S),
           SWA_EINVAL, false);
    EXPECT(swa_decode_fwd(P, P, P, POS, P, F, 1, 1, 128, INT_MAX, INT_MAX, 1.f, 0.f, SWA_BF16, nullptr, 0, S),
           SWA_EINVAL, false);
    EXPECT(swa_decode_fwd(P, P, P, POS, P, F, INT_MAX, INT_MAX, 128, 16, 0, 1.f, 0.f, SWA_BF16, nullptr, 0, S),
           SWA_EINVAL, false);
    CHECK(swa_decode_workspace_bytes(INT_MAX, INT_MAX, 128, INT_MAX, INT_MAX) == 0, "huge decode workspace");
    CHECK(swa_decode_workspace_bytes_gqa(1, 8, 3, 128, 16, 0) == 0, "kv heads not dividing");
    // allocation-free form: the fixed scratch bounds the split workspace
    CHECK(swa_decode_scratch_bytes() == ((size_t)16 << 20), "scratch size");
    EXPECT(swa_decode_fwd_gqa_noalloc(P, P, P, POS, P, F, 1, 8, 2, 128, 4096, 4, 0.088f, 0.f, SWA_BF16, S), SWA_OK,
           true);
    // fp8 decode
    EXPECT(swa_decode_fwd_fp8(P, P, P, F, F, POS, P, F, 64, 32, 32, 128, 4096, 4, 0.088f, 0.f, SWA_BF16, nullptr, 0,
                              S),
           SWA_OK, true);
    EXPECT(swa_decode_fwd_fp8(P, P, P, nullptr, F, POS, P, F, 64, 32, 32, 128, 4096, 4, 0.088f, 0.f, SWA_BF16,
                              nullptr, 0, S),
           SWA_EINVAL, false);
}

static void chunk_and_merge_cases() {
    EXPECT(swa_chunk_prefill_fwd(P, P, P, P, P, POS, P, F, 4, 32, 8, 4096, 128, 4096, 4, 0.088f, 4.f, SWA_KEYS_ALL,
                                 SWA_BF16, S),
           SWA_OK, true);
    EXPECT(swa_chunk_prefill_fwd(P, P, P, P, P, POS, P, F, 4, 32, 8, 4096, 128, 4096, 4, 0.088f, 4.f, 9, SWA_BF16, S),
           SWA_EINVAL, false);
    EXPECT(swa_chunk_prefill_fwd(P, P, P, P, P, POS, P, F, 1, 1, 1, INT_MAX, 128, 16, 0, 1.f, 0.f, SWA_KEYS_ALL,
                                 SWA_BF16, S),
           SWA_EINVAL, false);
    EXPECT(swa_chunk_prefill_fwd(P, P, P, P, P, POS, P, F, 1, 1, 1, 16, 128, INT_MAX, INT_MAX, 1.f, 0.f,
                                 SWA_KEYS_ALL, SWA_BF16, S),
           SWA_EINVAL, false);
    EXPECT(swa_lse_merge(P, F, P, F, P, F, 1000, 128, SWA_BF16, S), SWA_OK, true);
    EXPECT(swa_lse_merge(P, F, P, F, P, F, 0, 128, SWA_BF16, S), SWA_EINVAL, false);
    // a row count whose grid would not fit: rejected without forming rows x d
    EXPECT(swa_lse_merge(P, F, P, F, P, F, LLONG_MAX, 128, SWA_BF16, S), SWA_EINVAL, false);
    EXPECT(swa_lse_merge(P, F, P, F, P, F, LLONG_MAX / 2, 64, SWA_F32, S), SWA_EINVAL, false);
}

static void hook_cases() {
    const int statuses[] = {SWA_OK, SWA_EINVAL, SWA_EUNSUPPORTED, SWA_EALIGN, SWA_EHIP, SWA_EWORKSPACE, SWA_ESCRATCH, -99};
    for (int st : statuses)
        CHECK(swa_strerror(st) != nullptr && std::strlen(swa_strerror(st)) > 0, "strerror %d", st);
    // the tile enumeration: a count-only call, a call into a buffer, a buffer too small
    const long count = swa_band_tiles(1000, 127, 65, 128, 64, nullptr, 0);
    CHECK(count > 0, "tile count %ld", count);
    std::vector<int> tiles(3 * count);
    CHECK(swa_band_tiles(1000, 127, 65, 128, 64, tiles.data(), count) == count, "tiles written");
    CHECK(swa_band_tiles(1000, 127, 65, 128, 64, tiles.data(), count - 1) == count, "count past a short buffer");
    CHECK(swa_band_tiles(0, 1, 0, 128, 64, tiles.data(), count) < 0, "n = 0 refused");
    CHECK(swa_band_tiles(1000, 127, 65, 128, 64, nullptr, 4) < 0, "null buffer with room refused");
    // block and tile sizes that would carry the row arithmetic past INT_MAX are refused
    CHECK(swa_band_tiles(INT_MAX, 4096, 4, INT_MAX, 64, nullptr, 0) < 0, "n + bq past INT_MAX refused");
    CHECK(swa_band_tiles(INT_MAX - 64, 4096, 4, 64, INT_MAX, nullptr, 0) < 0, "n + bk past INT_MAX refused");
    CHECK(swa_band_tiles(INT_MAX - (1 << 30), INT_MAX, INT_MAX, 1 << 30, 1 << 30, nullptr, 0) > 0,
          "a schedule near INT_MAX");
    int bq = 0, bk = 0;
    CHECK(swa_prefill_tile_shape(SWA_BF16, 128, &bq, &bk) == SWA_OK && bq == 128 && bk == 64, "tile shape");
    CHECK(swa_prefill_tile_shape(SWA_BF16, 96, &bq, &bk) != SWA_OK, "tile shape of d = 96");
    // the workgroup order: a permutation, refused when the group does not divide the units
    std::vector<int> order(2 * 32 * 128);
    CHECK(swa_prefill_order(32, 128, 4, order.data(), 32 * 128) == 32 * 128, "order written");
    std::vector<char> seen(32 * 128, 0);
    for (int i = 0; i < 32 * 128; ++i) seen[order[2 * i] * 128 + order[2 * i + 1]] = 1;
    int covered = 0;
    for (char c : seen) covered += c;
    CHECK(covered == 32 * 128, "order is a permutation (%d)", covered);
    CHECK(swa_prefill_order(6, 4, 4, order.data(), 24) < 0, "group not dividing the units refused");
    CHECK(swa_prefill_order(INT_MAX, INT_MAX, 1, nullptr, 0) != 0, "huge order handled");
}

int main() {
    prefill_cases();
    pattern_cases();
    append_cases();
    decode_cases();
    chunk_and_merge_cases();
    hook_cases();
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("sanitized C ABI checks: ok (%d launches)\n", g_launches);
    return 0;
}
