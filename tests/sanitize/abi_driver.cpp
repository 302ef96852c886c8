// Drives every entry point of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer against the launch stubs: valid calls on fake
// device addresses (which must validate and reach the stubbed launch) and
// invalid ones (which must be refused with the documented status).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "path_attn.h"

static int failures = 0;
static void expect(const char *what, int got, int want) {
    if (got != want) {
        std::printf("FAIL %s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}
static void *P(uint64_t i) { return (void *)(uintptr_t)((i + 1) << 40); }  // far apart: no accidental overlap
static float *F(uint64_t i) { return (float *)P(i); }

int main() {
    const path_dtype_t BF = PATH_DTYPE_BF16, F32 = PATH_DTYPE_F32;
    expect("abi version", path_abi_version(), PATH_ABI_VERSION);
    for (int s = 0; s <= 5; ++s) (void)path_status_string((path_status_t)s);
    for (int d : {64, 128})
        for (path_dtype_t t : {BF, F32})
            for (int L : {1, 63, 64, 65, 4096}) {
                const size_t ws = path_attn_fwd_workspace_size(2, 3, L, d, t);
                expect("fwd ws size", ws > 0, 1);
                expect("fwd", path_attn_fwd(P(0), P(1), P(2), P(3), F(4), nullptr, P(5), F(6), 2, 3, L, d, t, 0.f,
                                            P(7), ws, nullptr), PATH_OK);
                expect("fwd_ex gate skip", path_attn_fwd_ex(P(0), P(1), P(2), P(3), F(4), F(8), P(5), nullptr, 2, 3,
                                                            L, d, t, 0.25f, P(7), ws, PATH_FWD_SKIP_NEGLIGIBLE,
                                                            nullptr), PATH_OK);
                expect("fwd small ws", path_attn_fwd(P(0), P(1), P(2), P(3), F(4), nullptr, P(5), F(6), 2, 3, L, d,
                                                     t, 0.f, P(7), ws - 1, nullptr), PATH_EINVAL);
                expect("fused", path_attn_fwd_fused(P(0), P(1), P(2), P(3), F(9), F(4), 1.98f, nullptr, P(5), F(6), 2,
                                                    3, L, d, t, 0.f, P(7), ws, nullptr), PATH_OK);
                expect("prep", path_attn_fwd_prep(P(0), P(1), P(2), P(3), F(4), F(8), P(5), F(6), 2, 3, L, d, t, 0.f,
                                                  P(7), ws, nullptr), PATH_OK);
                expect("scan", path_attn_fwd_scan(P(5), F(6), 1, 2, 3, L, d, t, 0.f, P(7), ws, nullptr), PATH_OK);
                expect("cache", path_decode_cache_from_fwd(P(7), ws, P(2), F(8), P(10), P(11), F(12), L + 5, 2, 3, L,
                                                           d, t, nullptr), PATH_OK);
                const size_t dws = path_decode_workspace_size(2, 3, L + 1, d, t);
                expect("decode", path_decode_step(P(10), P(11), L, L + 1, P(0), P(3), F(4), P(1), P(2), P(5), F(6), 2,
                                                  3, d, t, 0.f, P(7), dws, nullptr), PATH_OK);
                expect("decode_ex", path_decode_step_ex(P(10), P(11), L, L + 1, P(0), P(3), F(4), F(8), F(12), P(1),
                                                        P(2), P(5), F(6), 2, 3, d, t, 0.f, P(7), dws, nullptr),
                       PATH_OK);
                const size_t fws = path_decode_fused_workspace_size(2, 3, L + 1, d, t);
                expect("decode fused", path_decode_step_fused(P(10), P(11), L, L + 1, P(0), P(21), F(9), F(4), 1.98f,
                                                              P(22), F(8), F(12), P(1), P(2), P(5), F(6), 2, 3, d, t,
                                                              0.f, P(7), fws, nullptr), PATH_OK);
                expect("decode fused small ws",
                       path_decode_step_fused(P(10), P(11), L, L + 1, P(0), P(21), F(9), F(4), 0.f, P(22), nullptr,
                                              nullptr, P(1), P(2), P(5), F(6), 2, 3, d, t, 0.f, P(7), fws - 1, nullptr),
                       PATH_EINVAL);
                expect("decode noalloc (no device here)",
                       path_decode_step_noalloc(P(10), P(11), L, L + 1, P(0), P(3), F(4), nullptr, nullptr, nullptr,
                                                nullptr, P(5), F(6), 2, 3, d, t, 0.f, nullptr),
                       PATH_EHIP);
                const size_t bws = path_attn_bwd_workspace_size(2, 3, L, d, t);
                if (bws > 0)
                    expect("bwd", path_attn_bwd(P(0), P(1), P(2), P(3), F(4), F(8), P(5), F(6), P(13), F(14), P(15),
                                                P(16), P(17), P(18), F(19), F(20), 2, 3, L, d, t, 0.f, P(7), bws,
                                                nullptr), PATH_OK);
            }
    // refusals
    expect("fwd d96", path_attn_fwd(P(0), P(1), P(2), P(3), F(4), nullptr, P(5), nullptr, 1, 1, 64, 96, BF, 0.f, P(7),
                                    1u << 30, nullptr), PATH_EUNSUPPORTED);
    expect("fwd nan scale", path_attn_fwd(P(0), P(1), P(2), P(3), F(4), nullptr, P(5), nullptr, 1, 1, 64, 64, BF, NAN,
                                          P(7), 1u << 30, nullptr), PATH_EINVAL);
    expect("fwd alias", path_attn_fwd(P(0), P(1), P(2), P(3), F(4), nullptr, P(0), nullptr, 1, 1, 64, 64, BF, 0.f,
                                      P(7), 1u << 30, nullptr), PATH_EINVAL);
    expect("fwd huge", path_attn_fwd(P(0), P(1), P(2), P(3), F(4), nullptr, P(5), nullptr, 1 << 30, 1 << 30, 1 << 30,
                                     64, BF, 0.f, P(7), 1u << 30, nullptr), PATH_EINVAL);
    expect("decode n > ncap", path_decode_step(P(10), P(11), 11, 10, P(0), P(3), F(4), nullptr, nullptr, P(5), nullptr,
                                               1, 1, 64, BF, 0.f, P(7), 1u << 20, nullptr), PATH_EINVAL);
    expect("noalloc too big", path_decode_step_noalloc(P(10), P(11), 100, 100, P(0), P(3), F(4), nullptr, nullptr,
                                                       nullptr, nullptr, P(5), nullptr, 1000, 100, 128, BF, 0.f,
                                                       nullptr), PATH_ESCRATCH);
    expect("decode fused state over the cache",
           path_decode_step_fused(P(10), P(11), 10, 11, P(0), P(21), F(9), F(4), 0.f, P(10), nullptr, nullptr, nullptr,
                                  nullptr, P(5), nullptr, 1, 1, 64, BF, 0.f, P(7), 1u << 20, nullptr), PATH_EINVAL);
    expect("decode fused negative cap",
           path_decode_step_fused(P(10), P(11), 10, 11, P(0), P(21), F(9), F(4), -1.f, P(22), nullptr, nullptr, nullptr,
                                  nullptr, P(5), nullptr, 1, 1, 64, BF, 0.f, P(7), 1u << 20, nullptr), PATH_EINVAL);
    expect("fwd_ex bad flag", path_attn_fwd_ex(P(0), P(1), P(2), P(3), F(4), nullptr, P(5), nullptr, 1, 1, 64, 64, BF,
                                               0.f, P(7), 1u << 30, 4u, nullptr), PATH_EINVAL);
    std::printf("%s: %d failures\n", failures ? "FAILED" : "abi ok", failures);
    return failures ? 1 : 0;
}
