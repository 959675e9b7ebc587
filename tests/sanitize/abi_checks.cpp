// Host-only driver for the C ABI's argument validation, built with the host
// address and undefined-behaviour sanitizers (no kernel is compiled or
// launched: every call below fails validation before any HIP call).  Exits 0
// when every status matches; the sanitizers abort on the first finding.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "finch_wkv.h"

static int g_fail = 0;
#define EXPECT(call, want)                                                                  \
    do {                                                                                    \
        const wkv_status_t got_ = (call);                                                   \
        if (got_ != (want)) {                                                               \
            std::printf("FAIL line %d: %s -> %d (want %d): %s\n", __LINE__, #call, (int)got_, \
                        (int)(want), wkv_last_error());                                     \
            ++g_fail;                                                                       \
        }                                                                                   \
    } while (0)

// distinct, aligned fake device addresses, far apart (never dereferenced)
static void *fake(int n) { return reinterpret_cast<void *>(uintptr_t(n + 1) << 40); }

int main() {
    void *r = fake(0), *k = fake(1), *v = fake(2), *w = fake(3), *ws = fake(8), *u2 = fake(9);
    const float *u = static_cast<const float *>(fake(4)), *s_in = static_cast<const float *>(fake(5));
    float *o = static_cast<float *>(fake(6)), *s_out = static_cast<float *>(fake(7));
    const size_t need = wkv_prefill_workspace_bytes(1, 4096, 32, 64, WKV_BF16);
    if (need == 0) { std::printf("FAIL: no workspace for a split plan\n"); ++g_fail; }

    EXPECT(wkv_prefill(r, k, v, w, u, s_in, o, s_out, 1, 128, 4, 32, WKV_BF16, ws, need, nullptr), WKV_EUNSUPPORTED);
    EXPECT(wkv_prefill(r, k, v, w, u, s_in, o, s_out, 1, 128, 0, 64, WKV_BF16, ws, need, nullptr), WKV_EINVAL);
    EXPECT(wkv_prefill(r, k, v, w, u, s_in, o, s_out, 0, 128, 4, 64, WKV_BF16, ws, need, nullptr), WKV_EINVAL);
    EXPECT(wkv_prefill(r, k, v, w, u, s_in, o, s_out, 1, -1, 4, 64, WKV_BF16, ws, need, nullptr), WKV_EINVAL);
    EXPECT(wkv_prefill(r, k, v, w, u, s_in, o, s_out, 70000, 70000, 4, 64, WKV_BF16, ws, need, nullptr), WKV_EINVAL);
    EXPECT(wkv_prefill(r, k, v, w, u, s_in, o, s_out, 300, 17, 65536, 64, WKV_BF16, ws, need, nullptr), WKV_EUNSUPPORTED);
    EXPECT(wkv_prefill(nullptr, k, v, w, u, s_in, o, s_out, 1, 128, 4, 64, WKV_BF16, ws, need, nullptr), WKV_EINVAL);
    EXPECT(wkv_prefill(static_cast<char *>(r) + 2, k, v, w, u, s_in, o, s_out, 1, 128, 4, 64, WKV_BF16, ws, need,
                       nullptr), WKV_EINVAL);
    EXPECT(wkv_prefill(r, k, v, w, u, s_in, o, s_out, 1, 4096, 32, 64, WKV_BF16, nullptr, need, nullptr),
           WKV_EWORKSPACE);
    EXPECT(wkv_prefill(r, k, v, w, u, s_in, o, s_out, 1, 4096, 32, 64, WKV_BF16, ws, need - 1, nullptr),
           WKV_EWORKSPACE);
    EXPECT(wkv_prefill(r, k, v, w, u, s_in, static_cast<float *>(r) + 16, s_out, 1, 128, 4, 64, WKV_BF16, ws, need,
                       nullptr), WKV_EINVAL);                                      // o overlaps r
    EXPECT(wkv_prefill_ex(r, k, v, w, u, u2, s_in, o, s_out, 1, 128, 4, 64, WKV_BF16, 0, ws, need, nullptr),
           WKV_EINVAL);                                                            // u' without Finch-C2
    EXPECT(wkv_prefill_ex(r, k, v, w, u, nullptr, s_in, o, s_out, 1, 128, 4, 64, WKV_BF16, 64, ws, need, nullptr),
           WKV_EUNSUPPORTED);                                                      // unknown flag
    EXPECT(wkv_prefill_noalloc(r, k, v, w, u, nullptr, s_in, o, s_out, 1, 4096, 32, 32, WKV_BF16, 0, nullptr),
           WKV_EUNSUPPORTED);
    EXPECT(wkv_prefill_noalloc(nullptr, k, v, w, u, nullptr, s_in, o, s_out, 1, 4096, 32, 64, WKV_BF16, 0, nullptr),
           WKV_EINVAL);
    int marked = -1;
    EXPECT(wkv_workspace_errors(ws, need, 0, nullptr, nullptr), WKV_EINVAL);                  // no count
    EXPECT(wkv_workspace_errors(ws, WKV_WORKSPACE_CONTROL_BYTES - 64, 1, &marked, nullptr), WKV_EWORKSPACE);
    EXPECT(wkv_workspace_errors(ws, 0, 0, &marked, nullptr), WKV_OK);                         // no records
    if (marked != 0) {
        std::printf("FAIL: a workspace of 0 bytes reported %d marks\n", marked);
        ++g_fail;
    }

    // ragged offsets: host copies of every shape the planner reads
    std::vector<int32_t> bad_start = {1, 5, 9}, decreasing = {0, 5, 3}, good = {0, 100, 300};
    EXPECT(wkv_prefill_varlen(r, k, v, w, u, static_cast<int32_t *>(fake(10)), bad_start.data(), 2, s_in, o, s_out,
                              4, 64, WKV_BF16, ws, need, nullptr), WKV_EINVAL);
    EXPECT(wkv_prefill_varlen(r, k, v, w, u, static_cast<int32_t *>(fake(10)), decreasing.data(), 2, s_in, o, s_out,
                              4, 64, WKV_BF16, ws, need, nullptr), WKV_EINVAL);
    EXPECT(wkv_prefill_varlen(r, k, v, w, u, nullptr, good.data(), 2, s_in, o, s_out, 4, 64, WKV_BF16, ws, need,
                              nullptr), WKV_EINVAL);
    EXPECT(wkv_prefill_varlen(r, k, v, w, u, static_cast<int32_t *>(fake(10)), nullptr, 2, s_in, o, s_out, 4, 64,
                              WKV_BF16, ws, need, nullptr), WKV_EINVAL);
    std::vector<int32_t> many(100001);
    for (size_t i = 0; i < many.size(); ++i) many[i] = int32_t(i * 3);
    if (wkv_prefill_varlen_workspace_bytes(many.data(), 100000, 32, 64, WKV_BF16) == 0) {
        std::printf("FAIL: no workspace for 100000 short sequences\n");
        ++g_fail;
    }
    EXPECT(wkv_prefill_varlen_ex(r, k, v, w, u, nullptr, static_cast<int32_t *>(fake(10)), good.data(), 2, s_in, o,
                                 s_out, 4, 64, WKV_BF16, 16, ws, need, nullptr), WKV_EUNSUPPORTED);

    // epilogue entry points
    EXPECT(wkv_layernorm_heads(static_cast<const float *>(r), u, s_in, 1e-5f, o, WKV_BF16, 4096, 2048 + 512, nullptr),
           WKV_EUNSUPPORTED);
    EXPECT(wkv_layernorm_heads(static_cast<const float *>(r), u, s_in, -1.f, o, WKV_BF16, 4096, 2048, nullptr),
           WKV_EINVAL);
    EXPECT(wkv_gold_compress(r, w, o, WKV_F32, 4096, 512, nullptr), WKV_EUNSUPPORTED);
    EXPECT(wkv_gold_compress(r, w, static_cast<char *>(static_cast<void *>(o)) + 2, WKV_F32, 4096, 2048, nullptr),
           WKV_EINVAL);

    // status strings and the query functions never fail
    for (int s = 0; s < 6; ++s)
        if (!wkv_status_string(static_cast<wkv_status_t>(s))[0]) ++g_fail;
    if (wkv_abi_version() != FINCH_WKV_ABI_VERSION) ++g_fail;
    std::printf("%s (%d failure(s))\n", g_fail ? "FAILED" : "all checks passed", g_fail);
    return g_fail ? 1 : 0;
}
