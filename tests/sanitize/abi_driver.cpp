// Host driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of
// the C ABI (include/sa_indexer.h): argument validation and workspace sizing
// of every entry point.  Every call here is rejected before any launch (or is
// a size query), so it runs without a GPU; the sanitizers abort on any memory
// or undefined-behaviour error in the host code, e.g. an overflowing size
// computation for a very large shape.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "sa_indexer.h"

static int failures = 0;

static void expect(int got, int want, const char* what, int line) {
    if (got != want) {
        std::fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", line, what, got, want,
                     sa_last_error());
        ++failures;
    }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

int main() {
    // Never dereferenced: every call below is rejected before any launch.
    auto* q = reinterpret_cast<const uint16_t*>(uintptr_t(0x1000));
    auto* w = reinterpret_cast<const float*>(uintptr_t(0x2000));
    auto* k = reinterpret_cast<const uint16_t*>(uintptr_t(0x3000));
    auto* oi = reinterpret_cast<int32_t*>(uintptr_t(0x4000));
    auto* os = reinterpret_cast<float*>(uintptr_t(0x5000));
    auto* c8 = reinterpret_cast<const uint8_t*>(uintptr_t(0x6000));
    auto* sc = reinterpret_cast<const float*>(uintptr_t(0x7000));
    void* ws = reinterpret_cast<void*>(uintptr_t(0x8000));
    size_t n = 0;

    const sa_shape dec{8, 1, 64, 128, 131072, 131071, 2048};
    const sa_shape pre{1, 4096, 64, 128, 32768, 28672, 2048};
    // size queries, including the largest shapes the checks accept
    EXPECT(indexer_score_topk_ws(&dec, &n), SA_OK);
    EXPECT(indexer_score_topk_ws(&pre, &n), SA_OK);
    const sa_shape big{65535, 1, 64, 128, 1 << 30, (1 << 30) - 1, 1};
    EXPECT(indexer_score_topk_ws(&big, &n), SA_OK);
    const sa_shape bigpre{1, 1 << 20, 64, 128, 1 << 30, (1 << 30) - (1 << 20), 1 << 20};
    EXPECT(indexer_score_topk_ws(&bigpre, &n), SA_OK);
    EXPECT(misa_route_ws(&big, 1, 64, 0, 0, &n), SA_OK);
    EXPECT(misa_route_ws(&dec, 1024, 8, 8192, 1, &n), SA_OK);
    EXPECT(hisa_coarse_fine_ws(&big, 1, 1, 0, &n), SA_OK);
    EXPECT(hisa_coarse_fine_ws(&dec, 128, 64, 1, &n), SA_OK);
    EXPECT(misa_hisa_ws(&dec, 1024, 8, 128, 64, 0, 0, &n), SA_OK);
    EXPECT(lisa_score_topk_ws(&pre, &n), SA_OK);
    EXPECT(resmisa_route_ws(&dec, 128, 7, 0, &n), SA_OK);
    EXPECT(resmisa_route_ws(&big, 1, 60, 0, &n), SA_OK);
    EXPECT(indexer_score_topk_fp8_ws(&dec, &n), SA_OK);
    EXPECT(indexer_score_topk_fp8q_ws(&dec, &n), SA_OK);
    EXPECT(indexer_score_topk_ragged_ws(&pre, &n), SA_OK);

    // shape checks
    EXPECT(indexer_score_topk_ws(nullptr, &n), SA_EINVAL);
    sa_shape s = dec;
    s.d = 64;
    EXPECT(indexer_score_topk_ws(&s, &n), SA_EUNSUPPORTED);
    s = dec;
    s.H = 65;
    EXPECT(indexer_score_topk_ws(&s, &n), SA_EUNSUPPORTED);
    s = dec;
    s.causal_offset = dec.L;
    EXPECT(indexer_score_topk_ws(&s, &n), SA_EINVAL);
    s = dec;
    s.topk = 0;
    EXPECT(indexer_score_topk_ws(&s, &n), SA_EINVAL);
    s = dec;
    s.batch = 70000;
    EXPECT(indexer_score_topk_ws(&s, &n), SA_EUNSUPPORTED);
    s = dec;
    s.L = 2147483647;
    s.causal_offset = s.L - 1;
    EXPECT(indexer_score_topk_ws(&s, &n), SA_EUNSUPPORTED);
    s = dec;
    s.causal_offset = 2147483647;
    EXPECT(indexer_score_topk_ws(&s, &n), SA_EINVAL);
    EXPECT(indexer_score_topk_ws(&dec, nullptr), SA_EINVAL);

    // pointers and workspace
    EXPECT(indexer_score_topk(nullptr, w, k, &dec, oi, os, ws, 1 << 30, nullptr), SA_EINVAL);
    EXPECT(indexer_score_topk(q, w, k, &dec, nullptr, os, ws, 1 << 30, nullptr), SA_EINVAL);
    EXPECT(indexer_score_topk(q, w, k, &dec, oi, os, ws, 1, nullptr), SA_EWORKSPACE);
    EXPECT(indexer_score_topk(q, w, k, &dec, oi, os, nullptr, 1ull << 40, nullptr), SA_EWORKSPACE);
    EXPECT(indexer_score_topk_ragged(q, w, k, nullptr, 0, &pre, oi, os, ws, 1, nullptr),
           SA_EINVAL);
    EXPECT(indexer_score_topk_ragged(q, w, k, oi, -1, &pre, oi, os, ws, 1, nullptr), SA_EINVAL);
    EXPECT(indexer_score_topk_noalloc(q, w, k, &pre, oi, os, nullptr), SA_EWORKSPACE);
    EXPECT(indexer_score_topk_noalloc(q, w, nullptr, &dec, oi, os, nullptr), SA_EINVAL);

    // DSA with block pooling
    EXPECT(indexer_score_topk_pooled_ws(&dec, 128, 1024, &n), SA_OK);
    EXPECT(indexer_score_topk_pooled_ws(&pre, 128, 1024, &n), SA_EUNSUPPORTED);
    EXPECT(indexer_score_topk_pooled_ws(&dec, 64, 1024, &n), SA_EINVAL);
    EXPECT(indexer_score_topk_pooled_ws(&dec, 128, 1000, &n), SA_EINVAL);
    EXPECT(indexer_score_topk_pooled_ws(&dec, 1024, 8192, &n), SA_EUNSUPPORTED);
    EXPECT(indexer_score_topk_pooled(q, w, k, &dec, 128, 1024, nullptr, nullptr, oi, os, ws,
                                     1 << 30, nullptr, nullptr), SA_EINVAL);
    EXPECT(indexer_score_topk_pooled(q, w, k, &dec, 128, 1024, reinterpret_cast<uint16_t*>(oi),
                                     reinterpret_cast<uint16_t*>(oi), oi, os, ws, 1, nullptr,
                                     nullptr), SA_EWORKSPACE);

    // MISA / HISA arguments
    EXPECT(misa_route_ws(&dec, 0, 8, 0, 0, &n), SA_EINVAL);
    EXPECT(misa_route_ws(&dec, 1024, 0, 0, 0, &n), SA_EINVAL);
    EXPECT(misa_route_ws(&dec, 1024, 65, 0, 0, &n), SA_EINVAL);
    EXPECT(misa_route_ws(&dec, 1024, 8, 100, 0, &n), SA_EINVAL);
    EXPECT(misa_route(q, w, k, &dec, 1024, 8, 0, nullptr, nullptr, nullptr, oi, os, ws, 1,
                      nullptr), SA_EWORKSPACE);
    EXPECT(hisa_coarse_fine_ws(&dec, 128, 8, 0, &n), SA_EINVAL);   // r * b < k
    EXPECT(hisa_coarse_fine_ws(&dec, 0, 64, 0, &n), SA_EINVAL);
    EXPECT(hisa_coarse_fine_ws(&dec, 1 << 20, 1 << 20, 0, &n), SA_EUNSUPPORTED);
    EXPECT(hisa_coarse_fine(q, w, k, &dec, 128, 64, nullptr, nullptr, oi, os, ws, 1, nullptr),
           SA_EWORKSPACE);
    EXPECT(misa_hisa(q, w, k, &dec, 1024, 8, 128, 8, nullptr, nullptr, nullptr, nullptr, oi, os,
                     ws, 1 << 30, nullptr), SA_EINVAL);
    EXPECT(resmisa_route_ws(&dec, 128, 61, 0, &n), SA_EUNSUPPORTED);
    EXPECT(resmisa_route_ws(&dec, 0, 7, 0, &n), SA_EINVAL);
    EXPECT(lisa_score_topk(q, w, k, &dec, oi, os, ws, 1, nullptr), SA_EWORKSPACE);

    // FP8 cache
    EXPECT(sa_quantize_keys_fp8(k, 8, 131072, 64, nullptr, nullptr, nullptr), SA_EINVAL);
    EXPECT(sa_quantize_keys_fp8(k, 8, 131072, 64, const_cast<uint8_t*>(c8),
                                const_cast<float*>(sc), nullptr), SA_EUNSUPPORTED);
    EXPECT(indexer_score_topk_fp8(q, w, c8, sc, &pre, oi, os, ws, 1 << 30, nullptr),
           SA_EUNSUPPORTED);
    EXPECT(indexer_score_topk_fp8(q, w, c8, nullptr, &dec, oi, os, ws, 1 << 30, nullptr),
           SA_EINVAL);
    EXPECT(indexer_score_topk_fp8q(q, w, c8, sc, &dec, oi, os, ws, 1, nullptr), SA_EWORKSPACE);
    EXPECT(misa_route_fp8(q, w, c8, sc, &dec, 1024, 8, 8192, nullptr, nullptr, nullptr, oi, os,
                          ws, 1, nullptr), SA_EWORKSPACE);
    EXPECT(hisa_coarse_fine_fp8(q, w, nullptr, sc, &dec, 128, 64, nullptr, nullptr, oi, os, ws,
                                1 << 30, nullptr), SA_EINVAL);

    // pooling, extrema, tidy-up
    EXPECT(sa_pool_blocks(k, 8, 131072, 128, 0, nullptr, nullptr), SA_EINVAL);
    EXPECT(sa_pool_blocks2(k, 8, 131072, 128, 128, 1000, nullptr, nullptr, nullptr), SA_EINVAL);
    EXPECT(sa_block_extrema(k, 8, 131072, 96, 128, reinterpret_cast<uint16_t*>(oi), nullptr),
           SA_EUNSUPPORTED);
    EXPECT(sa_tidy_indices(oi, 8, 3, 2048, nullptr, 0, 64, 0, oi, nullptr, nullptr), SA_EINVAL);
    EXPECT(sa_tidy_indices(oi, 8, 1, 5000, nullptr, 0, 64, 0, oi, nullptr, nullptr),
           SA_EUNSUPPORTED);
    EXPECT(sa_tidy_indices(oi, 8, 1, 2048, nullptr, 0, 0, 0, oi, nullptr, nullptr), SA_EINVAL);

    // diagnostics
    EXPECT(sa_profile_read(-1, nullptr, nullptr), SA_EINVAL);
    if (sa_kernel_count() < 1 || std::strlen(sa_kernel_name(0)) == 0) ++failures;
    if (std::strlen(sa_kernel_name(10000)) != 0) ++failures;

    if (failures) {
        std::fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    std::printf("abi sanitizer driver ok\n");
    return 0;
}
