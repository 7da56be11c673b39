/* Drives the host side of the C ABI (include/moe.h) under AddressSanitizer and
 * UndefinedBehaviorSanitizer without a GPU: the host helpers over a grid of valid and
 * invalid descriptors, and every device entry point with arguments that the host-side
 * validation rejects before any HIP call (so nothing is launched).  Exit 0 and "ok" on
 * success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

#define CHECK(c, ...) do { if (!(c)) { printf("FAIL: " __VA_ARGS__); printf("\n"); exit(1); } } while (0)

static void expect_error(moe_status st, moe_status want, const char* what) {
    CHECK(st == want, "%s: status %d, expected %d (%s)", what, st, want, moe_last_error());
    CHECK(strlen(moe_last_error()) > 0, "%s: empty error message", what);
}

int main(void) {
    CHECK(moe_abi_version() == MOE_ABI_VERSION, "abi version");
    CHECK(moe_capacity(4096, 2, 8, 1.0) == 1024 && moe_capacity(4096, 8, 64, 1.0) == 512, "capacity");
    CHECK(moe_capacity(8, 2, 4, -1.0) == -1 && moe_capacity(-1, 2, 4, 1.0) == -1, "capacity");

    /* host helpers over a grid of descriptors, valid and not */
    const int Ts[] = {-1, 0, 1, 255, 4096, 65536};
    const int Es[] = {0, 1, 8, 64, 65};
    const int Ks[] = {0, 1, 2, 8, 9};
    const int Ss[] = {0, 1, 64, 4096};
    const int caps[] = {-2, -1, 0, 1, 1024};
    long valid = 0;
    for (size_t a = 0; a < sizeof(Ts) / sizeof(Ts[0]); ++a)
    for (size_t b = 0; b < sizeof(Es) / sizeof(Es[0]); ++b)
    for (size_t c = 0; c < sizeof(Ks) / sizeof(Ks[0]); ++c)
    for (size_t s = 0; s < sizeof(Ss) / sizeof(Ss[0]); ++s)
    for (size_t q = 0; q < sizeof(caps) / sizeof(caps[0]); ++q)
    for (int dt = -1; dt <= 2; ++dt) {
        moe_desc d = {Ts[a], 6144, Es[b], Ks[c], 16384, Ss[s], caps[q], dt, 0};
        int64_t R = moe_max_rows(&d);
        if (R < 0) {
            CHECK(strlen(moe_last_error()) > 0, "message for an invalid desc");
            CHECK(moe_workspace_size(&d, MOE_WS_ROUTE) == (size_t)-1, "ws of an invalid desc");
            continue;
        }
        ++valid;
        CHECK(R <= (int64_t)d.T * d.K, "max rows bound");
        for (int w = 0; w <= 4; ++w) CHECK(moe_workspace_size(&d, w) != (size_t)-1, "ws kind %d", w);
        CHECK(moe_workspace_size(&d, 5) == (size_t)-1, "unknown ws kind");
    }
    CHECK(valid > 0, "some descriptors are valid");
    CHECK(moe_max_rows(NULL) == -1, "null desc");

    /* device entry points, rejected before any HIP call */
    moe_desc d = {256, 64, 4, 2, 128, 256, -1, MOE_F32, 0};
    moe_desc bad = d;
    bad.K = 9;
    moe_routing r0;
    memset(&r0, 0, sizeof(r0));
    moe_routing rf;
    void** slots = (void**)&rf;
    for (size_t i = 0; i < sizeof(rf) / sizeof(void*); ++i) slots[i] = (void*)(uintptr_t)(4096 * (i + 1));
    void* p = (void*)(uintptr_t)4096;
    expect_error(moe_route(&bad, p, p, NULL, NULL, p, NULL, &rf, p, 1 << 20, NULL), MOE_ERR_INVALID_ARG, "route desc");
    expect_error(moe_route(&d, p, p, NULL, NULL, p, NULL, &r0, p, 1 << 20, NULL), MOE_ERR_INVALID_ARG, "route routing");
    expect_error(moe_route(&d, NULL, p, NULL, NULL, p, NULL, &rf, p, 1 << 20, NULL), MOE_ERR_INVALID_ARG, "route x");
    expect_error(moe_route(&d, p, p, NULL, p, p, NULL, &rf, p, 1 << 20, NULL), MOE_ERR_INVALID_ARG, "route w_sg");
    expect_error(moe_route(&d, p, p, NULL, NULL, p, NULL, &rf, p, 1, NULL), MOE_ERR_WORKSPACE, "route ws");
    expect_error(moe_route_noalloc(NULL, p, p, NULL, NULL, p, NULL, &rf, NULL), MOE_ERR_INVALID_ARG, "noalloc desc");
    moe_desc big = {65536, 6144, 64, 8, 2048, 65536, 4096, MOE_BF16, 0};
    expect_error(moe_route_noalloc(&big, p, p, NULL, NULL, p, NULL, &rf, NULL), MOE_ERR_UNSUPPORTED, "noalloc size");
    expect_error(moe_route_from_logits(&d, NULL, &rf, p, 1 << 20, NULL), MOE_ERR_INVALID_ARG, "from_logits");
    expect_error(moe_route_from_logits(&d, p, &rf, NULL, 1 << 20, NULL), MOE_ERR_INVALID_ARG, "from_logits ws");
    expect_error(moe_permute(&d, NULL, &rf, p, NULL), MOE_ERR_INVALID_ARG, "permute");
    expect_error(moe_expert_ffn_fwd(&d, p, p, p, p, p, p, p, p, NULL, NULL, 0, NULL), MOE_ERR_INVALID_ARG, "ffn_fwd");
    expect_error(moe_unpermute(&d, p, &rf, p, NULL, p, NULL), MOE_ERR_INVALID_ARG, "unpermute");
    expect_error(moe_unpermute_bwd(&d, p, p, &rf, NULL, NULL, p, NULL, NULL, NULL, NULL), MOE_ERR_INVALID_ARG, "unpermute_bwd");
    expect_error(moe_expert_ffn_bwd(&d, p, p, p, p, p, p, p, p, p, p, p, p, p, p, 1, NULL), MOE_ERR_WORKSPACE, "ffn_bwd ws");
    expect_error(moe_expert_ffn_bwd(&d, p, p, p, p, p, p, p, NULL, p, p, p, p, p, p, 1 << 30, NULL), MOE_ERR_INVALID_ARG, "ffn_bwd offsets");
    expect_error(moe_route_bwd(&d, p, &rf, p, p, p, p, NULL, p, 1 << 30, NULL), MOE_ERR_INVALID_ARG, "route_bwd dw_sg");
    expect_error(moe_route_bwd(&d, p, &rf, p, NULL, p, p, NULL, p, 1, NULL), MOE_ERR_WORKSPACE, "route_bwd ws");
    expect_error(moe_permute_bwd(&d, p, &rf, p, NULL, NULL, NULL, NULL, p, NULL, 0, NULL), MOE_ERR_INVALID_ARG, "permute_bwd w_router");
    moe_desc part = d;
    part.dtype = MOE_BF16;
    part.flags = MOE_FLAG_F32_PARTIAL;
    expect_error(moe_unpermute(&part, p, &rf, NULL, NULL, p, NULL), MOE_ERR_INVALID_ARG, "partial flag");
    moe_desc flags = d;
    flags.flags = 4;
    expect_error(moe_permute(&flags, p, &rf, p, NULL), MOE_ERR_INVALID_ARG, "unknown flag");
    printf("ok (%ld valid descriptors of the grid)\n", valid);
    return 0;
}
