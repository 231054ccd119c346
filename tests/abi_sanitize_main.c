/* Drives every argument check of the moe_w4 C ABI with fake device pointers:
 * none of these calls may reach the device (each returns its status before
 * any HIP call), so the program runs without a GPU.  Built against a library
 * whose host code has AddressSanitizer and UndefinedBehaviorSanitizer
 * instrumentation (tests/test_abi_sanitize.py); any report aborts it. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moe_w4.h"

static int failures = 0;
#define EXPECT(call, want)                                                                        \
    do {                                                                                          \
        const int got_ = (call);                                                                  \
        if (got_ != (want)) {                                                                     \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, got_, \
                    (int)(want));                                                                 \
            ++failures;                                                                           \
        }                                                                                         \
    } while (0)

#define P(a) ((void *)(uintptr_t)(a))

int main(void) {
    const int64_t Ts[] = {0, 1, 7, 8, 9, 48, 49, 127, 128, 2048, 3000, MOE_W4_MAX_TOKENS};
    for (size_t i = 0; i < sizeof(Ts) / sizeof(Ts[0]); ++i) {
        moe_w4_ws_layout L;
        EXPECT(moe_w4_workspace_layout(Ts[i], &L), MOE_W4_OK);
        if (L.total != moe_w4_workspace_bytes(Ts[i])) ++failures;
        if (moe_w4_stack_workspace_bytes(Ts[i]) < L.total) ++failures;
    }
    EXPECT(moe_w4_workspace_layout(-1, NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_workspace_layout(MOE_W4_MAX_TOKENS + 1, NULL), MOE_W4_EINVAL);
    if (moe_w4_workspace_bytes(MOE_W4_MAX_TOKENS + 1) != 0) ++failures;

    const size_t ws4 = moe_w4_workspace_bytes(4);
    /* forward: T, pointers, alignment, workspace size, aliasing */
    EXPECT(moe_w4_forward(P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000), 0,
                          P(0x60000000), NULL, P(0x70000000), ws4, NULL), MOE_W4_OK);
    EXPECT(moe_w4_forward(P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000), -3,
                          P(0x60000000), NULL, P(0x70000000), ws4, NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_forward(NULL, P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000), 4, P(0x60000000),
                          NULL, P(0x70000000), ws4, NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_forward(P(0x10000008), P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000), 4,
                          P(0x60000000), NULL, P(0x70000000), ws4, NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_forward(P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000), 4,
                          P(0x60000000), (const float *)P(0x80000002), P(0x70000000), ws4, NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_forward(P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000), 4,
                          P(0x60000000), NULL, P(0x70000000), ws4 - 1, NULL), MOE_W4_EWORKSPACE);
    EXPECT(moe_w4_forward(P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000), 4,
                          P(0x10000000 + 4096), NULL, P(0x70000000), ws4, NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_forward_policy(P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000), 4,
                                 P(0x60000000), NULL, 3, P(0x70000000), ws4, NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_forward_nvfp4(P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000), NULL,
                                P(0x50000000), 4, P(0x60000000), NULL, P(0x70000000), ws4, NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_forward_profiled(P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000), 4,
                                   P(0x60000000), NULL, P(0x70000000), ws4, NULL, NULL, 2), MOE_W4_EINVAL);
    EXPECT(moe_w4_forward_static(P(0x10000000), P(0x20000000), P(0x30000000), P(0x40000000), P(0x50000000),
                                 MOE_W4_STATIC_MAX_TOKENS + 1, P(0x60000000), NULL, NULL), MOE_W4_EWORKSPACE);
    EXPECT(moe_w4_forward_static(NULL, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL), MOE_W4_OK);

    /* stack: layer array contents are read and checked */
    moe_w4_layer layers[3];
    for (int l = 0; l < 3; ++l) {
        layers[l].router_w = P(0x10000000 + 0x100000 * l);
        layers[l].codes = P(0x10010000 + 0x100000 * l);
        layers[l].scales = P(0x10020000 + 0x100000 * l);
        layers[l].shared_w = P(0x10030000 + 0x100000 * l);
    }
    const size_t sws = moe_w4_stack_workspace_bytes(8);
    EXPECT(moe_w4_stack_forward((float *)P(0x40000000), layers, 3, 8, NULL, P(0x60000000), sws - 1, NULL),
           MOE_W4_EWORKSPACE);
    EXPECT(moe_w4_stack_forward((float *)P(0x40000000), layers, MOE_W4_STACK_MAX_LAYERS + 1, 8, NULL,
                                P(0x60000000), sws, NULL), MOE_W4_EINVAL);
    layers[2].scales = P(0x10020008);
    EXPECT(moe_w4_stack_forward((float *)P(0x40000000), layers, 3, 8, NULL, P(0x60000000), sws, NULL),
           MOE_W4_EINVAL);
    layers[2].scales = NULL;
    EXPECT(moe_w4_stack_forward((float *)P(0x40000000), layers, 3, 8, NULL, P(0x60000000), sws, NULL),
           MOE_W4_EINVAL);
    EXPECT(moe_w4_stack_forward((float *)P(0x40000000), NULL, 3, 8, NULL, P(0x60000000), sws, NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_stack_forward((float *)P(0x40000000), layers, 0, 8, NULL, P(0x60000000), sws, NULL), MOE_W4_OK);
    EXPECT(moe_w4_stack_layer(NULL, P(0x2000), P(0x3000), P(0x4000), P(0x5000), 4, P(0x6000), P(0x7000), P(0x8000),
                              1u << 30, NULL), MOE_W4_EINVAL);

    /* generators, packer, dense block, diagnostics */
    EXPECT(moe_w4_generate_normal_bf16(0, 1, -1, 1.0, P(0x1000), NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_generate_normal_bf16(0, 1, 16, -1.0, P(0x1000), NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_generate_normal_bf16(0, 1, 16, 1.0, P(0x1001), NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_generate_x(0, 0, -1, P(0x1000), NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_generate_layer(0, -1, NULL, NULL, NULL, NULL, NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_pack_experts(P(0x10000000), -1, P(0x20000000), P(0x30000000), NULL), MOE_W4_EINVAL);
    EXPECT(moe_w4_pack_experts(P(0x10000000), 0, NULL, NULL, NULL), MOE_W4_OK);
    EXPECT(moe_w4_dense_mlp(P(0x10000000), P(0x20000000), 4, P(0x60000000), P(0x70000000),
                            moe_w4_dense_mlp_workspace_bytes(4) - 1, NULL), MOE_W4_EWORKSPACE);
    EXPECT(moe_w4_set_fused_wait(-1, 0), MOE_W4_EINVAL);
    EXPECT(moe_w4_set_fused_wait(0, 0), MOE_W4_OK);
    for (int st = -5; st <= 1; ++st)
        if (!moe_w4_status_string(st)) ++failures;
    for (int i = -1; i <= moe_w4_profile_points(); ++i) (void)moe_w4_profile_point_name(i);
    if (moe_w4_last_device_error() != 0) ++failures;

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("abi validation under the sanitizers: ok\n");
    return 0;
}
