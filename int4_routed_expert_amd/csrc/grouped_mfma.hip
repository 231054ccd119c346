// Routed experts at prefill sizes: grouped int4 x fp16 products on the MFMA
// units (v_mfma_f32_32x32x16_f16), one launch for gate/up and one for down.
//
// Format (Flint model card, Aijuus/flint-w4exp, table row "weights"): signed
// int4 codes, one bf16 scale per 128 of K, in a fwht128-rotated basis; bank
// layout (NInfer README of Flint, "What is inside"): per expert, gate rows then
// up rows (2 x 512, K = 2048) and 2,048 down rows (K = 512).
//
// Work unit: a chunk of at most 64 sorted assignments of one expert (the chunk
// list comes from the sort) times a tile of weight rows.  Every code byte of
// the tile is read from HBM once per chunk and turned into exact fp16 values
// in registers: the mask trick of int4x8_to_q gives 1024+u and 1024+16u, and
// one packed fp16 add removes the bias, leaving c and 16c (exact).  The
// activations are the fp16 operands the rotation wrote (odd positions of each
// 8-group pre-divided by 16, exact), so each 8-group of codes is one MFMA B
// operand and the matching 16 bytes of activations one A operand.  Products
// are exact and the MFMA sums them in fp32; the partial sum of each 128-block
// is scaled by its bf16 scale in fp32, as the format defines.
//
// The K order inside an MFMA is free as long as A and B agree, so lane group
// g = lane / 32 of k-slice j in K-step q of a block takes 8-group 8g + 4q + j:
// a lane's codes for a whole block are 32 contiguous bytes of its row.
//
// gate/up: a workgroup owns 128 columns of a = silu(g) * u (the 128 gate rows
// and the 128 up rows behind them) for the chunk's tokens, i.e. exactly one
// Hadamard block of a, so its epilogue rotates a (fwht128 in LDS), picks the
// power-of-two prescale of each (row, block) and writes the fp16 operands of
// the down projection: the rotation costs no launch and no fp32 round trip.
//
// Work mapping: workgroups are dealt to the 8 XCDs round robin, so the tiles
// of one chunk are given consecutive per-XCD slots and share that XCD's L2
// for the chunk's activations.
#include "common.h"
#include "launch.h"

namespace moe_w4 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kChunkRows = 64;   // assignments per chunk (two 32-row MFMA tiles)
constexpr int kXcds = 8;

__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
}

// Eight codes -> the exact fp16 B operand (c0, c4, 16c1, 16c5, c2, c6, 16c3, 16c7).
__device__ __forceinline__ uint4 codes_to_f16(uint32_t w) {
    const Q4 q = int4x8_to_q(w);
    const half2_t even = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2_t odd = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q.q0) + even);
    r.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q.q1) + odd);
    r.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q.q2) + even);
    r.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q.q3) + odd);
    return r;
}

__device__ __forceinline__ uint32_t word(const uint4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Wait states between the last MFMA writing an accumulator and the first
// non-MFMA reader, made explicit: the compiler does not always cover them at
// the end of a loop.
__device__ __forceinline__ void mfma_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
}

// An offset the compiler cannot see through: reads addressed with it inside
// a loop are not hoisted out of it (the A operands in LDS are the same for
// every tile of the down kernel; keeping them all in registers would not fit).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm volatile("" : "+v"(v));
    return v;
}

// chunk index and tile index of this workgroup (XCD-aware deal, see above)
__device__ __forceinline__ void chunk_tile(int tiles, int &chunk, int &tile) {
    const int b = blockIdx.x, xcd = b % kXcds, k = b / kXcds;
    chunk = (k / tiles) * kXcds + xcd;
    tile = k % tiles;
}

// =========================================================================
// gate/up + SwiGLU + rotation of a
// =========================================================================
constexpr int kGuBuf = kChunkRows * 256;          // one A block: 64 rows x 128 fp16, swizzled
constexpr int kGuRing = 3;                          // A blocks in LDS: current and two in flight

// vmcnt-only wait (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and
// lgkmcnt at their maxima, i.e. not waited for)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// the same, and every LDS access of this wave completed (lgkmcnt 0)
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Workgroup barrier without the release/acquire fences of __syncthreads:
// those make every wave wait for all of its direct global->LDS loads
// (vmcnt 0), which would drain the prefetch.  The callers wait for exactly
// the loads the next block reads (wait_vmcnt) before arriving; the empty asm
// statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The A block of the chunk's 64 rows lives in LDS as [row][16 groups of 16 B]
// with group position grp ^ (row & 15): unpadded rows (so one wave's direct
// global->LDS load fills 4 whole rows) whose MFMA reads still hit 16
// different 4-bank slots for 16 consecutive rows.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gateup_mfma(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales, const uint32_t *__restrict__ xt,
    const float *__restrict__ xt_scale, const int *__restrict__ perm, const int4 *__restrict__ chunks,
    const int *__restrict__ n_chunks, uint32_t *__restrict__ at, float *__restrict__ at_scale) {
    // three separate arrays rather than one: the compiler then knows that a
    // block's reads do not alias the direct loads in flight into the other two
    // slots and does not wait for those loads before every LDS read
    __shared__ __attribute__((aligned(16))) uint8_t ring0[kGuBuf], ring1[kGuBuf], ring2[kGuBuf];
    __shared__ float row_p[kChunkRows];
    auto slot_ptr = [&](int slot) -> uint8_t * { return slot == 0 ? ring0 : slot == 1 ? ring1 : ring2; };
    int chunk, nt;
    chunk_tile(kI / kG, chunk, nt);
    if (chunk >= *n_chunks) return;
    const int4 ch = chunks[chunk];
    const int e = uniform(ch.x), row0 = uniform(ch.y), rows = uniform(ch.z);
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int n = lane & 31, g = lane >> 5;
    constexpr int kBlocks = kH / kG;

    if (tid < kChunkRows) row_p[tid] = xt_scale[perm[row0 + min(tid, rows - 1)] / kTopK];
    // A loads: wave w fills rows 16w..16w+15 of a block, 4 rows (1 KB) per
    // instruction; lane l writes position l & 15 of row 16w + 4i + (l >> 4)
    const uint8_t *asrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 16 * wave + 4 * i + (lane >> 4);
        const int tok = perm[row0 + min(r, rows - 1)] / kTopK;
        asrc[i] = reinterpret_cast<const uint8_t *>(xt + (size_t)tok * (kH / 2)) + ((lane & 15) ^ (r & 15)) * 16;
    }
    auto issue_a = [&](int slot, int blk) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_global_load_lds(asrc[i] + blk * 256,
                                             (lds_void_t *)(slot_ptr(slot) + (16 * wave + 4 * i) * 256), 16, 0, 0);
    };

    // this lane's gate and up rows; codes stream two blocks ahead
    const int gr = kG * nt + 32 * wave + n;
    const __amdgpu_buffer_rsrc_t cres = make_buf(codes + (size_t)e * kCodeBytesPerExpert, (uint32_t)kCodeBytesGu);
    const __amdgpu_buffer_rsrc_t sres = make_buf(scales + (size_t)e * kScalesPerExpert, (uint32_t)kScalesGu * 2);
    const uint32_t goff = (uint32_t)gr * (kH / 2) + 32 * g, uoff = goff + (uint32_t)kPlaneGateBytes;
    const uint32_t gsoff = (uint32_t)gr * 32, usoff = gsoff + (uint32_t)kScalesGate * 2;
    uint4 cb[3][4];
    auto fetch = [&](int slot, int blk) {
        const uint32_t o = (uint32_t)blk * 64;
        cb[slot][0] = bload16(cres, goff + o, 0);
        cb[slot][1] = bload16(cres, goff + o + 16, 0);
        cb[slot][2] = bload16(cres, uoff + o, 0);
        cb[slot][3] = bload16(cres, uoff + o + 16, 0);
    };
    // the 16 block scales of the gate row and of the up row (bf16)
    uint4 sg[2], su[2];
    sg[0] = bload16(sres, gsoff, 0);
    sg[1] = bload16(sres, gsoff + 16, 0);
    su[0] = bload16(sres, usoff, 0);
    su[1] = bload16(sres, usoff + 16, 0);

    // issue order per block: codes(b+2) (4 loads) then A(b+2) (4 loads); the
    // vmcnt waits below count on it: waiting for A(b+1) also covers codes(b+1)
    __builtin_amdgcn_sched_barrier(0);
    fetch(0, 0);
    issue_a(0, 0);
    fetch(1, 1);
    issue_a(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt_lds<8>();   // codes(0), A(0) and the row_p stores done (codes(1), A(1) may be in flight)
    block_barrier();

    f32x16_t accg[2], accu[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) accg[h][i] = accu[h][i] = 0.0f;

#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
        const uint8_t *buf = slot_ptr(b % kGuRing);
        const int cs = b % 3;
        __builtin_amdgcn_sched_barrier(0);
        if (b + 2 < kBlocks) {
            fetch((b + 2) % 3, b + 2);
            issue_a((b + 2) % kGuRing, b + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x16_t dg[2], du[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) dg[h][i] = du[h][i] = 0.0f;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 bg = codes_to_f16(word(cb[cs][q], j));
                const uint4 bu = codes_to_f16(word(cb[cs][2 + q], j));
                const int grp = 8 * g + 4 * q + j;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint4 a =
                        *reinterpret_cast<const uint4 *>(buf + (32 * h + n) * 256 + ((grp ^ (n & 15)) * 16));
                    dg[h] = mfma32(a, bg, dg[h]);
                    du[h] = mfma32(a, bu, du[h]);
                }
            }
        }
        mfma_drain();
        const uint32_t swg = word(sg[b >> 3], (b >> 1) & 3), swu = word(su[b >> 3], (b >> 1) & 3);
        const float s_g = (b & 1) ? bf16hi(swg) : bf16lo(swg);
        const float s_u = (b & 1) ? bf16hi(swu) : bf16lo(swu);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                accg[h][i] = fmaf(s_g, dg[h][i], accg[h][i]);
                accu[h][i] = fmaf(s_u, du[h][i], accu[h][i]);
            }
        // codes(b+1) and A(b+1) must have landed for every wave before the
        // next block; after them only codes(b+2) and A(b+2) were issued
        __builtin_amdgcn_sched_barrier(0);
        if (b + 2 < kBlocks)
            wait_vmcnt<8>();
        else if (b + 1 < kBlocks)
            wait_vmcnt<0>();
        block_barrier();
    }
    __syncthreads();

    // a = silu(g) * u for this workgroup's 128 columns, into LDS (fp32):
    // rows 0..31 in ring0, rows 32..63 in ring1, 128 floats per row
    auto act_row = [&](int m) -> float * {
        return reinterpret_cast<float *>(m < 32 ? ring0 : ring1) + (m & 31) * kG;
    };
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = 32 * h + 8 * (i >> 2) + 4 * g + (i & 3);
            const float p = row_p[m];
            const float gv = accg[h][i] * p, uv = accu[h][i] * p;
            act_row(m)[32 * wave + n] = gv / (1.0f + expf(-gv)) * uv;
        }
    __syncthreads();

    // fwht128 of each row: 16 lanes per row, 8 values per lane, 4 rows per pass
    const int rl = lane & 15;
    for (int r0 = 4 * wave; r0 < kChunkRows; r0 += 16) {
        const int m = r0 + (lane >> 4);
        const float4 *sp = reinterpret_cast<const float4 *>(act_row(m) + 8 * rl);
        const float4 a0 = sp[0], a1 = sp[1];
        float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((i & hs) == 0) {
                    const float x0 = v[i], x1 = v[i + hs];
                    v[i] = x0 + x1;
                    v[i + hs] = x0 - x1;
                }
#pragma unroll
        for (int msk = 1; msk <= 8; msk <<= 1) {   // strides 8..64 across the row's 16 lanes
            const bool upper = (lane & msk) != 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float q = shfl_xor_f(v[i], msk);
                v[i] = upper ? (q - v[i]) : (v[i] + q);
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[i] *= 0.08838834764831845f;   // 1/sqrt(128)
            amax = fmaxf(amax, fabsf(v[i]));
        }
#pragma unroll
        for (int msk = 1; msk <= 8; msk <<= 1) amax = fmaxf(amax, shfl_xor_f(amax, msk));
        int sh = 0;
        if (amax > 0.0f && isfinite(amax)) {
            int ex;
            frexpf(amax, &ex);
            sh = ex - 14;   // largest magnitude in [2^13, 2^14)
        }
        if (m < rows) {
            uint4 w;
            w.x = pack_half2(ldexpf(v[0], -sh), ldexpf(v[4], -sh));
            w.y = pack_half2(ldexpf(v[1], -sh - 4), ldexpf(v[5], -sh - 4));
            w.z = pack_half2(ldexpf(v[2], -sh), ldexpf(v[6], -sh));
            w.w = pack_half2(ldexpf(v[3], -sh - 4), ldexpf(v[7], -sh - 4));
            const size_t p = (size_t)(row0 + m);
            reinterpret_cast<uint4 *>(at + p * (kI / 2) + nt * (kG / 2))[rl] = w;
            if (rl == 0) at_scale[p * (kI / kG) + nt] = ldexpf(1.0f, sh);
        }
    }
}

// =========================================================================
// down: a workgroup owns a chunk and loops over output features in tiles of
// 128 (32 per wave), so the chunk's A (64 rows x 512 fp16) is staged in LDS
// once; the codes of the next two tiles are in flight during each tile.
// =========================================================================
constexpr int kDnPitch = 1040;    // bytes per LDS row (1024 + 16)
constexpr int kDnSplit = 2;       // workgroups per chunk (each takes half of the 2048 features)
constexpr int kDnTiles = kH / 128 / kDnSplit;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_down_mfma(
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ scales, const uint32_t *__restrict__ at,
    const float *__restrict__ at_scale, const int4 *__restrict__ chunks, const int *__restrict__ n_chunks,
    float *__restrict__ o) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kChunkRows * kDnPitch];
    __shared__ __attribute__((aligned(16))) float row_p[kI / kG][kChunkRows];   // [block][row]
    int chunk, half;
    chunk_tile(kDnSplit, chunk, half);
    if (chunk >= *n_chunks) return;
    const int4 ch = chunks[chunk];
    const int e = uniform(ch.x), row0 = uniform(ch.y), rows = uniform(ch.z);
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int n = lane & 31, g = lane >> 5;

    const __amdgpu_buffer_rsrc_t cres =
        make_buf(codes + (size_t)e * kCodeBytesPerExpert + kCodeBytesGu, (uint32_t)(kH * kI / 2));
    const __amdgpu_buffer_rsrc_t sres =
        make_buf(scales + (size_t)e * kScalesPerExpert + kScalesGu, (uint32_t)(kH * (kI / kG) * 2));
    const int f0 = half * (kH / kDnSplit) + 32 * wave + n;   // this lane's feature in tile 0
    uint4 cb[3][8];
    uint2 sb[3];
    auto fetch = [&](int slot, int tile) {
        const uint32_t row = (uint32_t)(f0 + 128 * tile);
        const uint32_t off = row * (kI / 2) + 32 * g;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            cb[slot][2 * b] = bload16_nt(cres, off + 64 * b, 0);
            cb[slot][2 * b + 1] = bload16_nt(cres, off + 64 * b + 16, 0);
        }
        const u32x2_t sv = __builtin_amdgcn_raw_buffer_load_b64(sres, row * 8, 0, 0);
        sb[slot] = make_uint2(sv.x, sv.y);
    };
    // stage the chunk's activations: thread -> (row, quarter of 1 KB)
    {
        const int srow = tid >> 2, part = tid & 3;
        const int p = row0 + min(srow, rows - 1);
        const uint4 *src = reinterpret_cast<const uint4 *>(at + (size_t)p * (kI / 2)) + part;
        uint4 v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = src[4 * i];
        fetch(0, 0);   // after the activations: their wait below does not wait for the codes
        fetch(1, 1);
#pragma unroll
        for (int i = 0; i < 16; ++i) *reinterpret_cast<uint4 *>(lds + srow * kDnPitch + part * 16 + 64 * i) = v[i];
        if (tid < kChunkRows) {
            const float4 q = *reinterpret_cast<const float4 *>(at_scale + (size_t)(row0 + min(tid, rows - 1)) * (kI / kG));
            row_p[0][tid] = q.x;
            row_p[1][tid] = q.y;
            row_p[2][tid] = q.z;
            row_p[3][tid] = q.w;
        }
    }
    __syncthreads();
    // o rows of the chunk through a buffer descriptor: stores of rows past the
    // chunk's end fall outside it and are dropped by the hardware bounds check
    const __amdgpu_buffer_rsrc_t ores = make_buf(o + (size_t)row0 * kH, (uint32_t)rows * kH * 4);

#pragma unroll
    for (int t = 0; t < kDnTiles; ++t) {
        const int cs = t % 3;
        __builtin_amdgcn_sched_barrier(0);
        if (t + 2 < kDnTiles) fetch((t + 2) % 3, t + 2);
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t zero = opaque(0);
        const uint8_t *abase = lds + zero;
        const float *pbase = &row_p[0][0] + zero + 4 * g;
        f32x16_t acc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[h][i] = 0.0f;
#pragma unroll
        for (int b = 0; b < kI / kG; ++b) {
            f32x16_t d[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 16; ++i) d[h][i] = 0.0f;
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint4 bw = codes_to_f16(word(cb[cs][2 * b + q], j));
                    const int grp = 16 * b + 8 * g + 4 * q + j;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint4 a = *reinterpret_cast<const uint4 *>(abase + (32 * h + n) * kDnPitch + grp * 16);
                        d[h] = mfma32(a, bw, d[h]);
                    }
                    // one k-slice at a time: keeps the converted codes and A
                    // operands of a whole block from being live at once
                    __builtin_amdgcn_sched_barrier(0);
                }
            mfma_drain();
            const uint32_t sw = (b < 2) ? sb[cs].x : sb[cs].y;
            const float s = (b & 1) ? bf16hi(sw) : bf16lo(sw);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    // rows 32h + 8*i4 + 4g + 0..3 of block b's prescales
                    const float4 p4 = *reinterpret_cast<const float4 *>(pbase + b * kChunkRows + 32 * h + 8 * i4);
                    acc[h][4 * i4 + 0] = fmaf(s * p4.x, d[h][4 * i4 + 0], acc[h][4 * i4 + 0]);
                    acc[h][4 * i4 + 1] = fmaf(s * p4.y, d[h][4 * i4 + 1], acc[h][4 * i4 + 1]);
                    acc[h][4 * i4 + 2] = fmaf(s * p4.z, d[h][4 * i4 + 2], acc[h][4 * i4 + 2]);
                    acc[h][4 * i4 + 3] = fmaf(s * p4.w, d[h][4 * i4 + 3], acc[h][4 * i4 + 3]);
                }
        }
        const uint32_t ob = (uint32_t)(f0 + 128 * t + 4 * g * kH) * 4;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t r = 32 * h + 8 * (i >> 2) + (i & 3);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[h][i]), ores, ob + r * kH * 4, 0, 0);
            }
    }
}

int max_chunks(int T) { return min(kE, kTopK * T) + (kTopK * T + kChunkRows - 1) / kChunkRows; }

static int grid_for(int T, int tiles) {
    const int c = (max_chunks(T) + kXcds - 1) / kXcds * kXcds;
    return c * tiles;
}

void launch_gateup_mfma(const uint8_t *codes, const uint16_t *scales, const uint32_t *xt, const float *xt_scale,
                        const int *perm, const int *chunks, const int *n_chunks, int T, uint32_t *at,
                        float *at_scale, hipStream_t s) {
    hipLaunchKernelGGL(k_gateup_mfma, dim3(grid_for(T, kI / kG)), dim3(256), 0, s, codes, scales, xt, xt_scale,
                       perm, reinterpret_cast<const int4 *>(chunks), n_chunks, at, at_scale);
}

void launch_down_mfma(const uint8_t *codes, const uint16_t *scales, const uint32_t *at, const float *at_scale,
                      const int *chunks, const int *n_chunks, int T, float *o, hipStream_t s) {
    hipLaunchKernelGGL(k_down_mfma, dim3(grid_for(T, kDnSplit)), dim3(256), 0, s, codes, scales, at, at_scale,
                       reinterpret_cast<const int4 *>(chunks), n_chunks, o);
}

}  // namespace moe_w4
