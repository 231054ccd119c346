// Seeded synthetic inputs on the device: the counter-based SplitMix64
// generator (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014), written from its published definition.
//   r(key, i) = mix64(key + (i + 1) * G),  key = mix64(seed * G + tid)
// int4 code = (r >> 60) - 8.  "Normal" bf16 = bf16_rne(f32(S) * mult) with S
// the centred sum of the four 16-bit lanes of r (an Irwin-Hall variate):
// integer work plus one fp32 multiply, so it matches a CPU implementation bit
// for bit.  This is input generation, not part of the layer.
#include "common.h"
#include "launch.h"

namespace moe_w4 {

constexpr uint64_t kGolden = 0x9E3779B97F4A7C15ull;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z ^= z >> 30;
    z *= 0xBF58476D1CE4E5B9ull;
    z ^= z >> 27;
    z *= 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z;
}

__device__ __forceinline__ uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * kGolden); }

__device__ __forceinline__ int irwin_hall(uint64_t r) {
    return (int)(r & 0xffff) + (int)((r >> 16) & 0xffff) + (int)((r >> 32) & 0xffff) + (int)(r >> 48) - 131070;
}

__global__ void k_gen_normal_bf16(uint64_t key, int64_t n, float mult, int absval, uint16_t *out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    int s = irwin_hall(draw(key, (uint64_t)i));
    if (absval) s = s < 0 ? -s : s;
    const float v = __fmul_rn((float)s, mult);   // one rounded fp32 multiply
    out[i] = f32_to_bf16(v);
}

// One thread writes one dword = 8 consecutive codes of a row.
__global__ void k_gen_codes(uint64_t key, int rows, int k, int experts, int64_t expert_elems,
                            int64_t expert_stride_bytes, uint8_t *out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int dw_per_row = k / 8;
    const int64_t total = (int64_t)experts * rows * dw_per_row;
    if (g >= total) return;
    const int d = (int)(g % dw_per_row);
    const int64_t er = g / dw_per_row;
    const int row = (int)(er % rows);
    const int e = (int)(er / rows);
    const uint64_t base = (uint64_t)e * expert_elems + (uint64_t)row * k + (uint64_t)d * 8;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int c = (int)(draw(key, base + i) >> 60) - 8;
        word |= ((uint32_t)c & 0xfu) << (4 * i);
    }
    *reinterpret_cast<uint32_t *>(out + e * expert_stride_bytes + (int64_t)row * (k / 2) + 4 * d) = word;
}

__global__ void k_gen_scales(uint64_t key, int groups_per_row, int rows, int experts, int64_t expert_stride,
                             float mult, uint16_t *out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_expert = (int64_t)rows * groups_per_row;
    if (g >= per_expert * experts) return;
    const int64_t e = g / per_expert, w = g % per_expert;
    int s = irwin_hall(draw(key, (uint64_t)g));
    s = s < 0 ? -s : s;
    out[e * expert_stride + w] = f32_to_bf16(__fmul_rn((float)s, mult));
}

void launch_gen_normal_bf16(uint64_t key, int64_t n, float mult, int absval, uint16_t *out, hipStream_t s) {
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL(k_gen_normal_bf16, dim3(blocks), dim3(256), 0, s, key, n, mult, absval, out);
}

void launch_gen_codes(uint64_t key, int rows, int k, int experts, int64_t expert_elems,
                      int64_t expert_stride_bytes, uint8_t *out, hipStream_t s) {
    const int64_t total = (int64_t)experts * rows * (k / 8);
    hipLaunchKernelGGL(k_gen_codes, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, key, rows, k,
                       experts, expert_elems, expert_stride_bytes, out);
}

void launch_gen_scales(uint64_t key, int groups_per_row, int rows, int experts, int64_t expert_stride,
                       float mult, uint16_t *out, hipStream_t s) {
    const int64_t total = (int64_t)experts * rows * groups_per_row;
    hipLaunchKernelGGL(k_gen_scales, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, key,
                       groups_per_row, rows, experts, expert_stride, mult, out);
}

}  // namespace moe_w4
