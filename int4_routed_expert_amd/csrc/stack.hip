// The two element-wise steps of a layer stack: x_l = bf16(rmsnorm(resid)) with
// unit gain and eps 1e-6, and resid += f32(y_l).
#include "common.h"
#include "launch.h"

namespace moe_w4 {

// x = bf16(resid / sqrt(mean(resid^2) + 1e-6)), one workgroup per token.
__global__ __launch_bounds__(256) void k_rmsnorm_bf16(const float *__restrict__ resid, int T,
                                                      uint16_t *__restrict__ x) {
    __shared__ float part[4];
    const int t = blockIdx.x;
    const int c = threadIdx.x * 8;
    const float4 *rp = reinterpret_cast<const float4 *>(resid + (size_t)t * kH + c);
    const float4 a = rp[0], b = rp[1];
    float ss = a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w + b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float tot = part[0] + part[1] + part[2] + part[3];
    const float inv = 1.0f / sqrtf(tot / (float)kH + 1e-6f);
    uint4 out;
    out.x = (uint32_t)f32_to_bf16(a.x * inv) | ((uint32_t)f32_to_bf16(a.y * inv) << 16);
    out.y = (uint32_t)f32_to_bf16(a.z * inv) | ((uint32_t)f32_to_bf16(a.w * inv) << 16);
    out.z = (uint32_t)f32_to_bf16(b.x * inv) | ((uint32_t)f32_to_bf16(b.y * inv) << 16);
    out.w = (uint32_t)f32_to_bf16(b.z * inv) | ((uint32_t)f32_to_bf16(b.w * inv) << 16);
    reinterpret_cast<uint4 *>(x + (size_t)t * kH + c)[0] = out;
}

void launch_rmsnorm_bf16(const float *resid, int T, uint16_t *x, hipStream_t s) {
    hipLaunchKernelGGL(k_rmsnorm_bf16, dim3(T), dim3(256), 0, s, resid, T, x);
}

__global__ __launch_bounds__(256) void k_residual_add(float *__restrict__ resid,
                                                      const uint16_t *__restrict__ y, int64_t n) {
    const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i >= n) return;
    const uint4 q = *reinterpret_cast<const uint4 *>(y + i);
    float4 *rp = reinterpret_cast<float4 *>(resid + i);
    float4 a = rp[0], b = rp[1];
    a.x += bf16lo(q.x); a.y += bf16hi(q.x); a.z += bf16lo(q.y); a.w += bf16hi(q.y);
    b.x += bf16lo(q.z); b.y += bf16hi(q.z); b.z += bf16lo(q.w); b.w += bf16hi(q.w);
    rp[0] = a;
    rp[1] = b;
}

void launch_residual_add(float *resid, const uint16_t *y, int T, hipStream_t s) {
    const int64_t n = (int64_t)T * kH;
    hipLaunchKernelGGL(k_residual_add, dim3((unsigned)((n / 8 + 255) / 256)), dim3(256), 0, s, resid, y, n);
}

}  // namespace moe_w4
