// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point with arguments that the
// library must refuse before any HIP call, and the host-only size queries
// over a seeded sweep of problem descriptors, extreme sizes and strides
// included.  Device pointers are fake, non-null values that are never
// dereferenced: no call here reaches a kernel launch (a valid problem is only
// given to the host-only queries, or to an entry point together with one
// invalid argument).  Exit status 0 when every expectation holds.
#include "csa_index.h"

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>

namespace {

int g_failures = 0;

void expect(bool ok, const char *what, int line)
{
    if (!ok) {
        std::fprintf(stderr, "line %d: expectation failed: %s (last error: %s)\n", line, what, csa_last_error());
        ++g_failures;
    }
}
#define EXPECT(c) expect((c), #c, __LINE__)

void *fake(uintptr_t v) { return reinterpret_cast<void *>(v); }
const uintptr_t kFake = 0x100000; // 256-byte aligned, never dereferenced

csa_index_problem problem(int B, int S, int H, int D, int W, int m = 4)
{
    csa_index_problem p{};
    p.B = B;
    p.S = S;
    p.H = H;
    p.D = D;
    p.W = W;
    p.compress_rate = m;
    p.scale = 1.0f;
    p.plan = CSA_PLAN_AUTO;
    p.q_sb = (int64_t)H * S * D;
    p.q_sh = (int64_t)S * D;
    p.q_ss = D;
    p.k_sb = (int64_t)W * D;
    p.k_sw = D;
    p.w_sb = (int64_t)S * H;
    p.w_ss = H;
    return p;
}

// splitmix64
uint64_t g_state = 0x243F6A8885A308D3ull;
uint64_t next()
{
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int32_t pick_i32()
{
    static const int32_t edge[] = {0, 1, 2, 3, 7, 8, 31, 32, 33, 63, 64, 127, 128, 129, 255, 256, 4096, 65536, 65537,
                                   1 << 30, (1 << 30) + 1, std::numeric_limits<int32_t>::max(), -1,
                                   std::numeric_limits<int32_t>::min()};
    const uint64_t r = next();
    if (r % 3 == 0)
        return edge[(r >> 8) % (sizeof edge / sizeof edge[0])];
    return (int32_t)((r >> 8) % 70000);
}

int64_t pick_i64()
{
    static const int64_t edge[] = {0, 8, 16, 64, 128, 136, 1 << 20, (int64_t)1 << 24, ((int64_t)1 << 24) - 8,
                                   (int64_t)1 << 40, std::numeric_limits<int64_t>::max() / 2 * 2, -8};
    const uint64_t r = next();
    if (r % 2 == 0)
        return edge[(r >> 8) % (sizeof edge / sizeof edge[0])];
    return (int64_t)((r >> 8) % (1 << 22)) * 8;
}

void refused_before_any_launch()
{
    csa_index_problem p = problem(2, 64, 8, 64, 40);
    size_t n = 0;
    EXPECT(csa_index_workspace_size(&p, 16, &n) == CSA_OK);
    EXPECT(csa_index_backward_workspace_size(&p, &n) == CSA_OK);
    EXPECT(csa_index_resolve_plan(&p) >= CSA_PLAN_ROW_TILES);
    csa_index_masks m{};
    int32_t *idx = static_cast<int32_t *>(fake(kFake));
    float *f = static_cast<float *>(fake(kFake));
    // null / misaligned inputs
    EXPECT(csa_index_score(&p, nullptr, fake(kFake), fake(kFake), &m, f, nullptr) == CSA_ERR_INVALID_ARG);
    EXPECT(csa_index_score(&p, fake(kFake + 2), fake(kFake), fake(kFake), &m, f, nullptr) == CSA_ERR_INVALID_ARG);
    EXPECT(csa_index_score(&p, fake(kFake), fake(kFake + 8), fake(kFake), &m, f, nullptr) == CSA_ERR_INVALID_ARG);
    EXPECT(csa_index_score(nullptr, fake(kFake), fake(kFake), fake(kFake), &m, f, nullptr) == CSA_ERR_INVALID_ARG);
    // top_k outside [1, 2048]: an unsupported size
    EXPECT(csa_index_select(&p, fake(kFake), fake(kFake), fake(kFake), &m, 0, idx, nullptr, nullptr, 0, nullptr) ==
           CSA_ERR_UNSUPPORTED);
    EXPECT(csa_index_select(&p, fake(kFake), fake(kFake), fake(kFake), &m, 4096, idx, nullptr, nullptr, 0, nullptr) ==
           CSA_ERR_UNSUPPORTED);
    EXPECT(csa_index_select(&p, fake(kFake), fake(kFake), fake(kFake), &m, 16, nullptr, nullptr, nullptr, 0,
                            nullptr) == CSA_ERR_INVALID_ARG);
    EXPECT(csa_index_select_noalloc(&p, fake(kFake), fake(kFake), fake(kFake), &m, 16, nullptr, nullptr, nullptr) ==
           CSA_ERR_INVALID_ARG);
    // mask pairs: q_seg without k_seg
    csa_index_masks bad{};
    bad.q_seg = static_cast<const int32_t *>(fake(kFake));
    EXPECT(csa_index_select(&p, fake(kFake), fake(kFake), fake(kFake), &bad, 16, idx, nullptr, nullptr, 0, nullptr) ==
           CSA_ERR_INVALID_ARG);
    // unsupported shapes
    csa_index_problem q = problem(1, 8, 4, 40, 8);
    EXPECT(csa_index_score(&q, fake(kFake), fake(kFake), fake(kFake), &m, f, nullptr) == CSA_ERR_UNSUPPORTED);
    q = problem(1, 8, 130, 32, 8);
    EXPECT(csa_index_score(&q, fake(kFake), fake(kFake), fake(kFake), &m, f, nullptr) == CSA_ERR_UNSUPPORTED);
    q = problem(1, 8, 4, 32, 8);
    q.k_sw = 12;
    EXPECT(csa_index_score(&q, fake(kFake), fake(kFake), fake(kFake), &m, f, nullptr) == CSA_ERR_UNSUPPORTED);
    q = problem(1, 8, 4, 32, 8);
    q.scale = std::numeric_limits<float>::quiet_NaN();
    EXPECT(csa_index_score(&q, fake(kFake), fake(kFake), fake(kFake), &m, f, nullptr) == CSA_ERR_INVALID_ARG);
    // top-k entry point
    EXPECT(csa_index_topk(4, 100, 0, f, idx, nullptr, 0, nullptr) == CSA_ERR_UNSUPPORTED);
    EXPECT(csa_index_topk(-1, 100, 5, f, idx, nullptr, 0, nullptr) == CSA_ERR_INVALID_ARG);
    EXPECT(csa_index_topk(4, 100, 5, nullptr, idx, nullptr, 0, nullptr) == CSA_ERR_INVALID_ARG);
    EXPECT(csa_index_topk_workspace_size(4, 100, 5, &n) == CSA_OK);
    // backward: gradient, outputs and workspace
    size_t need = 0;
    EXPECT(csa_index_backward_workspace_size(&p, &need) == CSA_OK);
    EXPECT(csa_index_score_backward(&p, fake(kFake), fake(kFake), fake(kFake), &m, nullptr, f, f, f, fake(kFake), need,
                                    nullptr) == CSA_ERR_INVALID_ARG);
    EXPECT(csa_index_score_backward(&p, fake(kFake), fake(kFake), fake(kFake), &m, f, f, f, f, nullptr, need,
                                    nullptr) == CSA_ERR_WORKSPACE);
    EXPECT(csa_index_score_backward(&p, fake(kFake), fake(kFake), fake(kFake), &m, f, f, f, f, fake(kFake), need - 1,
                                    nullptr) == CSA_ERR_WORKSPACE);
    EXPECT(csa_index_score_backward(&p, fake(kFake), fake(kFake), fake(kFake), &m, f, f, static_cast<float *>(fake(kFake + 4)), f,
                                    fake(kFake), need, nullptr) == CSA_ERR_INVALID_ARG);
    // KL loss: target and output
    EXPECT(csa_index_kl_loss(&p, fake(kFake), fake(kFake), fake(kFake), &m, nullptr, f, nullptr, nullptr) ==
           CSA_ERR_INVALID_ARG);
    EXPECT(csa_index_kl_loss(&p, fake(kFake), fake(kFake), fake(kFake), &m, f, nullptr, nullptr, nullptr) ==
           CSA_ERR_INVALID_ARG);
    // status strings
    for (int s = -1; s <= 5; ++s)
        EXPECT(csa_status_string(static_cast<csa_status>(s)) != nullptr);
    EXPECT(csa_index_abi_version() == CSA_INDEX_ABI_VERSION);
}

// Random descriptors through the host-only queries: whatever the fields, the
// queries return a status (no overflow, no out-of-bounds access) and, for
// problems they accept, sizes that are consistent between calls.
void descriptor_sweep(int iters)
{
    for (int it = 0; it < iters; ++it) {
        csa_index_problem p{};
        p.B = pick_i32();
        p.S = pick_i32();
        p.H = (int32_t)(next() % 3 == 0 ? pick_i32() : (int32_t)(1 + next() % 130));
        static const int32_t ds[] = {32, 64, 128, 16, 0, 256};
        p.D = ds[next() % 6];
        p.W = pick_i32();
        p.compress_rate = next() % 4 == 0 ? pick_i32() : (int32_t)(1 + next() % 8);
        p.scale = next() % 16 == 0 ? std::numeric_limits<float>::infinity() : 0.5f;
        p.plan = (int32_t)(next() % 4) - (next() % 8 == 0 ? 1 : 0);
        p.q_sb = pick_i64();
        p.q_sh = pick_i64();
        p.q_ss = pick_i64();
        p.k_sb = pick_i64();
        p.k_sw = pick_i64();
        p.w_sb = pick_i64();
        p.w_ss = pick_i64();
        const int32_t top_k = pick_i32();
        size_t a = 1, b = 2;
        const csa_status s1 = csa_index_workspace_size(&p, top_k, &a);
        const csa_status s2 = csa_index_workspace_size(&p, top_k, &b);
        EXPECT(s1 == s2);
        if (s1 == CSA_OK)
            EXPECT(a == b);
        const int32_t plan = csa_index_resolve_plan(&p);
        EXPECT(plan == -1 || plan == CSA_PLAN_ROW_TILES || plan == CSA_PLAN_SPLIT_ROWS);
        const csa_status s3 = csa_index_backward_workspace_size(&p, &a);
        EXPECT(s3 >= CSA_OK && s3 <= CSA_ERR_DEVICE);
        (void)csa_index_topk_workspace_size((int64_t)p.B * p.S, p.W, top_k, &a);
        // the compute entry points with a null output must refuse on the host
        csa_index_masks m{};
        EXPECT(csa_index_select(&p, fake(kFake), fake(kFake), fake(kFake), &m, top_k, nullptr, nullptr, nullptr, 0,
                                nullptr) != CSA_OK || (int64_t)p.B * p.S == 0);
    }
}

} // namespace

int main(int argc, char **argv)
{
    const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
    refused_before_any_launch();
    descriptor_sweep(iters);
    if (g_failures) {
        std::fprintf(stderr, "%d expectation(s) failed\n", g_failures);
        return 1;
    }
    std::printf("api driver: all expectations hold (%d descriptors)\n", iters);
    return 0;
}
