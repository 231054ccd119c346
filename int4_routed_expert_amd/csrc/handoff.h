// Hand-offs between the workgroups of one launch: data written and read with
// a cache policy that is coherent across the XCDs' L2s, and completion
// counters that the consumers poll with a time bound.
#pragma once

#include "common.h"
#include "launch.h"

namespace moe_w4 {

// Cache policy of a hand-off: device scope (sc1) plus the volatile bit, which
// keeps the accesses in program order around the counter and barriers (the
// compiler adds sc0: system scope, also coherent across XCDs).
constexpr int kHandOff = 16 | (int)(1u << 31);

// Poll one replica of a completion counter until it reaches `target` or
// `ticks` of the 100 MHz real-time clock pass; returns whether it was reached.
__device__ __forceinline__ bool wait_count(const int *counter, int target, uint32_t ticks) {
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
    for (;;) {
        if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) return true;
        if (__builtin_amdgcn_s_memrealtime() - t_start > ticks) return false;
        __builtin_amdgcn_s_sleep(8);
    }
}

// Add 1 to every replica of a counter (lanes 0..15 of the calling wave).
__device__ __forceinline__ void count_done(int *counters, int lane) {
    if (lane < kFusedCounters)
        __hip_atomic_fetch_add(counters + lane * kFusedCounterStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moe_w4
