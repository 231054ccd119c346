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
// are exact and the MFMA sums them in fp32; each 128-block's bf16 scale
// multiplies its codes exactly (see codes_to_f16_scaled) or its partial sum.
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
//
// The same two kernels serve the NVFP4 experts (template argument NV; Flint
// NVFP4 repack, kekzle/Flint-NVFP4, rows "Layout per Linear" and
// "Declaration": E2M1 codes two per byte in the int4 layout's rows, one E4M3
// scale per 16 of K, one fp32 tensor scale per Linear, W4A16, original
// basis).  Eight codes become four exact fp16 pairs by the gfx950 FP4 convert
// instruction (natural order), times their block's E4M3 scale in fp16 (exact:
// at most 6 significant bits, never below the fp16 normal range); the
// activations are natural-order fp16 (no Hadamard); the tensor scale is
// applied to the fp32 sums; gate/up writes a without a rotation and down
// writes fp32 expert rows.
#include "common.h"
#include "launch.h"

namespace moe_w4 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

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

// The same times a scale s' (fp16, both halves): c * s' and 16c * s' are
// exact in fp16 when s' has at most 8 significant bits and the products stay
// inside the fp16 range (|c| <= 8 adds at most 3 bits: 11 significant bits).
__device__ __forceinline__ uint4 codes_to_f16_scaled(uint32_t w, half2_t s) {
    const uint4 c = codes_to_f16(w);
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, c.x) * s);
    r.y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, c.y) * s);
    r.z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, c.z) * s);
    r.w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, c.w) * s);
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

// compile-time tile count for the main loops (one straight-line copy per
// count instead of a branch around every MFMA)
template <int N>
struct Tiles {
    static constexpr int value = N;
};
template <int MaxTiles, class F>
__device__ __forceinline__ void with_tiles(int n_mt, F &&f) {
    static_assert(MaxTiles == 2 || MaxTiles == 3, "two or three 32-row tiles at most");
    if constexpr (MaxTiles == 3) {
        if (n_mt >= 3) {
            f(Tiles<3>{});
            return;
        }
    }
    if (n_mt >= 2)
        f(Tiles<2>{});
    else
        f(Tiles<1>{});
}

// chunk index and tile index of this workgroup (XCD-aware deal, see above)
__device__ __forceinline__ void chunk_tile(int tiles, int &chunk, int &tile) {
    const int b = blockIdx.x, xcd = b % kXcds, k = b / kXcds;
    chunk = (k / tiles) * kXcds + xcd;
    tile = k % tiles;
}

// Power-of-two exponent k making the largest of a row's bf16 scales land in
// [2^7, 2^8) after multiplication by 2^k (0 if all scales are zero): the
// largest B operand, 16c * s' with |16c| <= 128, then stays below 2^15.
__device__ __forceinline__ int scale_shift(const uint4 &a, const uint4 &b) {
    uint32_t e = 0;
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        e = max(e, (w[i] >> 7) & 0xffu);
        e = max(e, (w[i] >> 23) & 0xffu);
    }
    return e ? 134 - (int)e : 0;
}
// The same over the 4 bf16 scales of one down row (two words).
__device__ __forceinline__ int scale_shift4(uint32_t a, uint32_t b) {
    const uint32_t e = max(max((a >> 7) & 0xffu, (a >> 23) & 0xffu), max((b >> 7) & 0xffu, (b >> 23) & 0xffu));
    return e ? 134 - (int)e : 0;
}
// bf16 scale s (low or high half of a word) -> fp16 s * 2^k in both halves
__device__ __forceinline__ half2_t scaled_half2(uint32_t word2, int hi, int k) {
    const float f = ldexpf(hi ? bf16hi(word2) : bf16lo(word2), k);
    const _Float16 h = (_Float16)f;
    return half2_t{h, h};
}

// =========================================================================
// gate/up + SwiGLU + rotation of a
//
// The chunk's A block (up to 64 rows) lives in LDS as [row][16 groups of 16 B]
// with group position grp ^ (row & 15): unpadded rows (one wave's direct
// global->LDS load fills 4 whole rows) whose MFMA reads still hit 16
// different 4-bank slots for 16 consecutive rows.  A three-slot ring keeps
// two blocks in flight; the codes run three blocks ahead in registers.
// Scales are folded into the B operand (codes_to_f16_scaled with the row's
// scales normalised by one power of two), so the MFMA accumulates over the
// whole of K and the normalisation is undone once at the end.
// =========================================================================
// (a fourth A slot, three blocks in flight, measured no faster)
constexpr int kGuRing = 3;                     // A blocks in LDS (kGuRing - 1 in flight)
constexpr int kGuCodeDist = 3;                 // codes requested this many blocks ahead
constexpr int kGuCodeRing = kGuCodeDist + 1;
constexpr int kGuADist = kGuRing - 1;          // A requested this many blocks ahead
constexpr int kGuBlocks = kH / kG;
constexpr bool kGuCodesFirst = kGuCodeDist <= kGuADist;   // order of the two requests of a block

// Issue order of the main loop's loads: codes(0 .. Dc-1) and A(0 .. Da-1) in
// the prologue, then per block b codes(b + Dc) and A(b + Da) (those below the
// block count; codes first if kGuCodesFirst).  The waits count on it: the
// number of loads requested after A(b + 1) up to the end of block b (F loads
// per codes block, NI per A block) may stay in flight when block b + 1 starts.
__host__ __device__ constexpr int gu_loads_after_a(int b, int ni, int f) {
    int n = 0;
    bool seen = false;
    for (int k = 0; k < kGuADist; ++k) {
        if (seen) n += ni;
        if (k == b + 1) seen = true;
    }
    for (int k = 0; k <= b; ++k) {
        const bool c = k + kGuCodeDist < kGuBlocks, a = k + kGuADist < kGuBlocks;
        if (kGuCodesFirst && c && seen) n += f;
        if (a) {
            if (seen) n += ni;
            if (k + kGuADist == b + 1) seen = true;
        }
        if (!kGuCodesFirst && c && seen) n += f;
    }
    return n;
}
// ... which covers codes(b + 1) only if it was requested before A(b + 1)
__host__ __device__ constexpr bool gu_codes_before_a() {
    for (int b = 0; b + 1 < kGuBlocks; ++b) {
        int pos = 0, pc = -1, pa = -1;
        for (int k = 0; k < kGuCodeDist; ++k, ++pos)
            if (k == b + 1) pc = pos;
        for (int k = 0; k < kGuADist; ++k, ++pos)
            if (k == b + 1) pa = pos;
        for (int k = 0; k < kGuBlocks; ++k) {
            const int ci = k + kGuCodeDist, ai = k + kGuADist;
            if (kGuCodesFirst) {
                if (ci == b + 1) pc = pos;
                ++pos;
                if (ai == b + 1) pa = pos;
                ++pos;
            } else {
                if (ai == b + 1) pa = pos;
                ++pos;
                if (ci == b + 1) pc = pos;
                ++pos;
            }
        }
        if (pc > pa) return false;
    }
    return true;
}
static_assert(gu_codes_before_a(), "codes(b+1) must be requested before A(b+1)");
// The main loop's waits are written out as constant counts (a count chosen
// at run time through a switch cost the kernel 80 bytes of spills per lane);
// they must agree with gu_loads_after_a for every block
__host__ __device__ constexpr int gu_wait_written(int b, int ni, int f) {
    return b + 3 < kGuBlocks ? (b >= 1 ? 2 * f + ni : f + ni) : b + 2 < kGuBlocks ? f + ni : 0;
}
__host__ __device__ constexpr bool gu_waits_agree() {
    for (int ni = 2; ni <= 6; ni += 2)
        for (int f = 4; f <= 6; f += 2)
            for (int b = 0; b + 1 < kGuBlocks; ++b)
                if (gu_wait_written(b, ni, f) != gu_loads_after_a(b, ni, f)) return false;
    return true;
}
static_assert(kGuRing == 3 && kGuCodeDist == 3 && gu_waits_agree(), "the written-out waits follow the issue order");

// NVFP4 block scales of an expert: gate [512][128], up [512][128], down [2048][32] bytes
constexpr uint32_t kNvScGate = (uint32_t)kI * kH / 16;
constexpr uint32_t kNvScGu = 2 * kNvScGate;
constexpr uint32_t kNvScPerExpert = kNvScGu + (uint32_t)kH * kI / 16;

// Eight E2M1 codes (element 2b in the low nibble of byte b) times one fp16
// scale (both halves): the B operand (c0 s, c1 s, ..., c7 s), exact.
__device__ __forceinline__ uint4 nv_codes_to_f16(uint32_t w, half2_t s) {
    uint4 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s);
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s);
    r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s);
    r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s);
    return r;
}
// Byte i of four E4M3 scales -> fp16 pair (exact).
__device__ __forceinline__ half2_t e4m3_half2(uint32_t w, int i) {
    const _Float16 h = (_Float16)e4m3_to_f32((w >> (8 * i)) & 0xffu);
    return half2_t{h, h};
}

// MaxMT: 32-row tiles of the longest chunk (2: chunks of <= 64 rows; 3: up to 96)
template <bool NV, int MaxMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_gateup_mfma(
    const uint8_t *__restrict__ codes, const void *__restrict__ scales_, const float *__restrict__ tscales,
    const uint32_t *__restrict__ xt, const float *__restrict__ xt_scale, const int *__restrict__ perm,
    const int4 *__restrict__ chunks, const int *__restrict__ n_chunks, int chunk_cap, uint32_t *__restrict__ at,
    float *__restrict__ at_scale) {
    // separate arrays rather than one: the compiler then knows that a block's
    // reads do not alias the direct loads in flight into the other slots and
    // does not wait for those loads before every LDS read
    constexpr int kRows = 32 * MaxMT;          // rows of the longest chunk
    constexpr int kGuBuf = kRows * 256;        // one A block: kRows rows x 128 fp16
    __shared__ __attribute__((aligned(16))) uint8_t ring0[kGuBuf], ring1[kGuBuf], ring2[kGuBuf],
        ring3[kGuRing > 3 ? kGuBuf : 16];
    __shared__ float row_p[kRows];
    auto slot_ptr = [&](int slot) -> uint8_t * {
        return slot == 0 ? ring0 : slot == 1 ? ring1 : slot == 2 ? ring2 : ring3;
    };
    int chunk, nt;
    chunk_tile(kI / kG, chunk, nt);
    // the chunk record is read beside the chunk count (one dependent load
    // less before the codes can be requested); chunk_cap records exist
    const int nch = *n_chunks;
    const int4 ch = chunks[min(chunk, chunk_cap - 1)];
    if (chunk >= nch) return;
    const int e = uniform(ch.x), row0 = uniform(ch.y), rows = uniform(ch.z);
    const int n_mt = uniform((rows + 31) >> 5);   // 32-row MFMA tiles in use
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int n = lane & 31, g = lane >> 5;
    constexpr int kBlocks = kGuBlocks;

    // this lane's gate and up rows
    const int gr = kG * nt + 32 * wave + n;
    const __amdgpu_buffer_rsrc_t cres = make_buf(codes + (size_t)e * kCodeBytesPerExpert, (uint32_t)kCodeBytesGu);
    const uint16_t *scales = static_cast<const uint16_t *>(scales_);
    const uint8_t *nv_scales = static_cast<const uint8_t *>(scales_);
    const __amdgpu_buffer_rsrc_t sres =
        NV ? make_buf(nv_scales + (size_t)e * kNvScPerExpert, kNvScGu)
           : make_buf(scales + (size_t)e * kScalesPerExpert, (uint32_t)kScalesGu * 2);
    const uint32_t goff = (uint32_t)gr * (kH / 2) + 32 * g, uoff = goff + (uint32_t)kPlaneGateBytes;
    const uint32_t gsoff = (uint32_t)gr * 32, usoff = gsoff + (uint32_t)kScalesGate * 2;
    // NVFP4: the lane's four E4M3 scales of a block (16-blocks 8 blk + 4 g ..)
    const uint32_t nsg = (uint32_t)gr * (kH / 16) + 4 * g, nsu = nsg + kNvScGate;
    uint4 cb[kGuCodeRing][4];
    uint32_t csg[kGuCodeRing], csu[kGuCodeRing];
    constexpr int kFetchLoads = NV ? 6 : 4;   // loads of one fetch
    auto fetch = [&](int slot, int blk) {
        const uint32_t o = (uint32_t)blk * 64;
        cb[slot][0] = bload16(cres, goff + o, 0);
        cb[slot][1] = bload16(cres, goff + o + 16, 0);
        cb[slot][2] = bload16(cres, uoff + o, 0);
        cb[slot][3] = bload16(cres, uoff + o + 16, 0);
        if constexpr (NV) {
            csg[slot] = bload4(sres, nsg + 8 * blk, 0);
            csu[slot] = bload4(sres, nsu + 8 * blk, 0);
        }
    };
    // the codes and scales depend only on the expert: requested before the
    // chunk's tokens are looked up, then (below) A(0 .. Da-1); the main loop
    // keeps the order of gu_loads_after_a, whose count of loads after A(b+1)
    // is what the wait at the end of block b lets stay in flight.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < kGuCodeDist; ++d) fetch(d, d);
    // the 16 block scales of the gate row and of the up row (bf16)
    uint4 sg[2], su[2];
    if constexpr (!NV) {
        sg[0] = bload16(sres, gsoff, 0);
        sg[1] = bload16(sres, gsoff + 16, 0);
        su[0] = bload16(sres, usoff, 0);
        su[1] = bload16(sres, usoff + 16, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (tid < kRows) row_p[tid] = xt_scale[perm[row0 + min(tid, rows - 1)] / kTopK];

    // a = silu(g) * u for this workgroup's 128 columns goes into LDS (fp32)
    // after the main loop: rows 0..31 in ring0, rows 32..63 in ring1
    constexpr int kActRowsPerSlot = kGuBuf / (kG * 4);
    static_assert(2 * kActRowsPerSlot >= kRows, "the fp32 rows of a fit two ring slots");
    auto act_row = [&](int m) -> float * {
        return reinterpret_cast<float *>(m < kActRowsPerSlot ? ring0 : ring1) +
               (m < kActRowsPerSlot ? m : m - kActRowsPerSlot) * kG;
    };
    with_tiles<MaxMT>(n_mt, [&](auto tiles) {
    constexpr int MT = decltype(tiles)::value;
    // A loads of the 32*MT rows in use: NI instructions per wave, 4 rows (1 KB)
    // each; lane l writes position l & 15 of row 4*(NI*w + i) + (l >> 4)
    constexpr int NI = 2 * MT;
    const uint8_t *asrc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = 4 * (NI * wave + i) + (lane >> 4);
        const int tok = perm[row0 + min(r, rows - 1)] / kTopK;
        asrc[i] = reinterpret_cast<const uint8_t *>(xt + (size_t)tok * (kH / 2)) + ((lane & 15) ^ (r & 15)) * 16;
    }
    auto issue_a = [&](int slot, int blk) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
            __builtin_amdgcn_global_load_lds(asrc[i] + blk * 256,
                                             (lds_void_t *)(slot_ptr(slot) + 4 * (NI * wave + i) * 256), 16, 0, 0);
    };
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < kGuADist; ++d) issue_a(d, d);
    __builtin_amdgcn_sched_barrier(0);
    const int kg = NV ? 0 : scale_shift(sg[0], sg[1]), ku = NV ? 0 : scale_shift(su[0], su[1]);
    wait_vmcnt_lds<(kGuADist - 1) * NI>();   // A(0) and the row_p stores done (later A blocks may be in flight)
    block_barrier();

    f32x16_t accg[MT], accu[MT];
#pragma unroll
    for (int h = 0; h < MT; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) accg[h][i] = accu[h][i] = 0.0f;

#pragma unroll
    for (int b = 0; b < kBlocks; ++b) {
        const uint8_t *buf = slot_ptr(b % kGuRing);
        const int cs = b % kGuCodeRing;
        __builtin_amdgcn_sched_barrier(0);
        if (kGuCodesFirst && b + kGuCodeDist < kBlocks) fetch((b + kGuCodeDist) % kGuCodeRing, b + kGuCodeDist);
        if (b + kGuADist < kBlocks) issue_a((b + kGuADist) % kGuRing, b + kGuADist);
        if (!kGuCodesFirst && b + kGuCodeDist < kBlocks) fetch((b + kGuCodeDist) % kGuCodeRing, b + kGuCodeDist);
        __builtin_amdgcn_sched_barrier(0);
        half2_t s_g, s_u, ng[4], nu[4];
        if constexpr (NV) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ng[i] = e4m3_half2(csg[cs], i);
                nu[i] = e4m3_half2(csu[cs], i);
            }
        } else {
            s_g = scaled_half2(word(sg[b >> 3], (b >> 1) & 3), b & 1, kg);
            s_u = scaled_half2(word(su[b >> 3], (b >> 1) & 3), b & 1, ku);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // 8-group 8g + 4q + j of the block: NVFP4 16-block 4g + 2q + j/2
                const uint4 bg = NV ? nv_codes_to_f16(word(cb[cs][q], j), ng[2 * q + (j >> 1)])
                                    : codes_to_f16_scaled(word(cb[cs][q], j), s_g);
                const uint4 bu = NV ? nv_codes_to_f16(word(cb[cs][2 + q], j), nu[2 * q + (j >> 1)])
                                    : codes_to_f16_scaled(word(cb[cs][2 + q], j), s_u);
                const int grp = 8 * g + 4 * q + j;
#pragma unroll
                for (int h = 0; h < MT; ++h) {
                    const uint4 a =
                        *reinterpret_cast<const uint4 *>(buf + (32 * h + n) * 256 + ((grp ^ (n & 15)) * 16));
                    accg[h] = mfma32(a, bg, accg[h]);
                    accu[h] = mfma32(a, bu, accu[h]);
                }
            }
        }
        // codes(b+1) and A(b+1) must have landed for every wave before the
        // next block; what was requested after A(b+1) may stay in flight
        __builtin_amdgcn_sched_barrier(0);
        if (b + 3 < kBlocks) {
            if (b >= 1)
                wait_vmcnt<2 * kFetchLoads + NI>();
            else
                wait_vmcnt<kFetchLoads + NI>();
        } else if (b + 2 < kBlocks) {
            wait_vmcnt<kFetchLoads + NI>();
        } else if (b + 1 < kBlocks) {
            wait_vmcnt<0>();
        }
        block_barrier();
    }
    mfma_drain();
    __syncthreads();
    const float gscale = NV ? tscales[3 * e] : ldexpf(1.0f, -kg);
    const float uscale = NV ? tscales[3 * e + 1] : ldexpf(1.0f, -ku);
#pragma unroll
    for (int h = 0; h < MT; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = 32 * h + 8 * (i >> 2) + 4 * g + (i & 3);
            const float p = row_p[m];
            const float gv = accg[h][i] * gscale * p, uv = accu[h][i] * uscale * p;
            // silu with the hardware exp and reciprocal (relative error ~1e-7)
            act_row(m)[32 * wave + n] = gv * __builtin_amdgcn_rcpf(1.0f + __expf(-gv)) * uv;
        }
    });
    __syncthreads();

    // fwht128 of each row (int4 experts; NVFP4 ones keep a in the original
    // basis): 16 lanes per row, 8 values per lane, 4 rows per pass
    const int rl = lane & 15;
    for (int r0 = 4 * wave; r0 < 32 * n_mt; r0 += 16) {
        const int m = r0 + (lane >> 4);
        const float4 *sp = reinterpret_cast<const float4 *>(act_row(m) + 8 * rl);
        const float4 a0 = sp[0], a1 = sp[1];
        float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
        for (int hs = 1; hs < (NV ? 1 : 8); hs <<= 1)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if ((i & hs) == 0) {
                    const float x0 = v[i], x1 = v[i + hs];
                    v[i] = x0 + x1;
                    v[i + hs] = x0 - x1;
                }
#pragma unroll
        for (int msk = 1; msk <= (NV ? 0 : 8); msk <<= 1) {   // strides 8..64 across the row's 16 lanes
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
            if (!NV) v[i] *= 0.08838834764831845f;   // 1/sqrt(128)
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
            if (NV) {   // natural order, the order of the E2M1 conversion
                w.x = pack_half2(ldexpf(v[0], -sh), ldexpf(v[1], -sh));
                w.y = pack_half2(ldexpf(v[2], -sh), ldexpf(v[3], -sh));
                w.z = pack_half2(ldexpf(v[4], -sh), ldexpf(v[5], -sh));
                w.w = pack_half2(ldexpf(v[6], -sh), ldexpf(v[7], -sh));
            } else {    // the operand order of int4x8_to_q
                w.x = pack_half2(ldexpf(v[0], -sh), ldexpf(v[4], -sh));
                w.y = pack_half2(ldexpf(v[1], -sh - 4), ldexpf(v[5], -sh - 4));
                w.z = pack_half2(ldexpf(v[2], -sh), ldexpf(v[6], -sh));
                w.w = pack_half2(ldexpf(v[3], -sh - 4), ldexpf(v[7], -sh - 4));
            }
            const size_t p = (size_t)(row0 + m);
            reinterpret_cast<uint4 *>(at + p * (kI / 2) + nt * (kG / 2))[rl] = w;
            if (rl == 0) at_scale[p * (kI / kG) + nt] = ldexpf(1.0f, sh);
        }
    }
}

// =========================================================================
// down: four workgroups own a chunk, each a quarter of the 2048 output
// features in four tiles of 128 (32 per wave), with up to 64 rows of the
// chunk's A (x 512 fp16) staged in LDS at a time: a chunk of 65-96 rows (an
// expert with that many) takes two passes, the second re-reading the
// workgroup's codes from L2.  At ~73 KB of LDS two workgroups share a CU, so
// one stages its rows while the other multiplies (96 staged rows, one
// workgroup per CU, left every staging exposed).  The codes of the next tile
// are in flight during each tile.  The MFMA runs transposed (codes as the row operand, tokens as the
// column operand), so a lane ends with 4 consecutive features of one token
// per group.  o is stored in fp16 with one power-of-two multiplier per row
// (o_scale), which halves the traffic of the fp32 rows at a relative rounding
// of 2^-11 (a bf16 o, 2^-9, added enough error on outputs six standard
// deviations out to cross the 2e-2 x rms bar).  The MFMA sums are bounded
// independently of the data (fp16 operands below 2^14 and codes times
// normalised scales below 2^11, 512 terms: |acc| < 2^34), so acc * 2^-20
// times each feature's normalisation relative to the expert's largest
// never overflows fp16; the row's prescale and that largest normalisation
// go to o_scale.
//
// Scales: A arrives with a power-of-two prescale per (token, 128-block); at
// staging each block is brought to the token's largest prescale (an exact
// power-of-two multiply in fp16), and each feature's 4 bf16 scales are
// normalised by one power of two and folded exactly into its fp16 codes
// (codes_to_f16_scaled), so the MFMA accumulates over all of K and the two
// normalisations are undone once per output.
// =========================================================================
constexpr int kDnPitch = 1040;   // bytes per LDS row (1024 + 16)
constexpr int kDnParts = 4;              // workgroups per chunk, each over a quarter of the features
constexpr int kDnFeat = kH / kDnParts;   // features of one workgroup
constexpr int kDnTiles = kDnFeat / 128;  // 128-feature tiles of a workgroup (32 features per wave)
constexpr int kDnRows = kChunkRows;    // rows of A staged at once (one pass)
constexpr int kDnCodeRing = 2;
static_assert(kDnTiles % kDnCodeRing == 0, "every pass starts on ring slot 0");
static_assert(2 * kDnRows >= kChunkMaxRows, "two passes cover a chunk");

// NVFP4 (NV): no scale normalisation; each lane's four E4M3 scales of a
// block come with its codes, and o is written as fp32 rows (o_scale unused).
// PASSES: chunks may have more than kDnRows rows (then up to two passes)
template <bool NV, bool PASSES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_down_mfma(
    const uint8_t *__restrict__ codes, const void *__restrict__ scales_, const float *__restrict__ tscales,
    const uint32_t *__restrict__ at, const float *__restrict__ at_scale, const int4 *__restrict__ chunks,
    const int *__restrict__ n_chunks, int chunk_cap, void *__restrict__ o_, float *__restrict__ o_scale) {
    const uint16_t *scales = static_cast<const uint16_t *>(scales_);
    uint16_t *o = static_cast<uint16_t *>(o_);
    __shared__ __attribute__((aligned(16))) uint8_t lds[kDnRows * kDnPitch];
    __shared__ float fk_wave[4];                                              // largest 2^-k per wave
    __shared__ float row_p[kDnRows];                                          // per token
    __shared__ __attribute__((aligned(16))) uint16_t sc[kI / kG][kDnFeat];    // [block][feature] bf16
    __shared__ __attribute__((aligned(16))) float fk[kDnFeat];                // 2^-k per feature
    // four workgroups per chunk (one per quarter of the features, on one XCD
    // so that they share the chunk's activations and codes in L2): one
    // workgroup per chunk left the grid at ~1.1 rounds of the CUs at T = 2048
    int chunk, quarter;
    chunk_tile(kDnParts, chunk, quarter);
    const int nch = *n_chunks;
    const int4 ch = chunks[min(chunk, chunk_cap - 1)];   // beside the count, as in gate/up
    if (chunk >= nch) return;
    const int e = uniform(ch.x), row0 = uniform(ch.y), rows = uniform(ch.z);
    const int n_pass = PASSES ? uniform((rows + kDnRows - 1) / kDnRows) : 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int n = lane & 31, g = lane >> 5;

    const __amdgpu_buffer_rsrc_t cres =
        make_buf(codes + (size_t)e * kCodeBytesPerExpert + kCodeBytesGu, (uint32_t)(kH * kI / 2));
    // the feature whose codes this lane loads, in tile 0
    const int fh = quarter * kDnFeat;
    const int f0 = fh + 32 * wave + n;
    const __amdgpu_buffer_rsrc_t nsres =
        make_buf(static_cast<const uint8_t *>(scales_) + (size_t)e * kNvScPerExpert + kNvScGu, kH * kI / 16);
    uint4 cb[kDnCodeRing][8];
    uint32_t cs4[kDnCodeRing][4];   // NVFP4: the lane's four E4M3 scales of each block
    auto fetch = [&](int slot, int tile) {
        const uint32_t off = (uint32_t)(f0 + 128 * tile) * (kI / 2) + 32 * g;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            cb[slot][2 * b] = bload16(cres, off + 64 * b, 0);
            cb[slot][2 * b + 1] = bload16(cres, off + 64 * b + 16, 0);
        }
        if constexpr (NV) {
            const uint32_t so = (uint32_t)(f0 + 128 * tile) * (kI / 16) + 4 * g;
#pragma unroll
            for (int b = 0; b < 4; ++b) cs4[slot][b] = bload4(nsres, so + 8 * b, 0);
        }
    };
    // the activations of a pass are needed first: thread -> (row, part), load
    // i takes the row's 16-byte group 4i + part (block i / 4); the codes of
    // the first tile are requested right behind those of pass 0
    static_assert(4 * kDnRows == 256, "one thread per quarter row");
    const int srow = tid >> 2, part = tid & 3;
    uint4 v[16];
    float4 ps;
    auto stage_load = [&](int pass) {
        const int p = row0 + min(kDnRows * pass + srow, rows - 1);
        const uint4 *src = reinterpret_cast<const uint4 *>(at + (size_t)p * (kI / 2)) + part;
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = src[4 * i];
        ps = *reinterpret_cast<const float4 *>(at_scale + (size_t)p * (kI / kG));
    };
    __builtin_amdgcn_sched_barrier(0);
    stage_load(0);
    // each block brought to the row's largest prescale, into LDS
    auto stage_store = [&]() {
        const float pm = fmaxf(fmaxf(ps.x, ps.y), fmaxf(ps.z, ps.w));
        const float pb[4] = {ps.x / pm, ps.y / pm, ps.z / pm, ps.w / pm};   // exact powers of two <= 1
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const _Float16 r = (_Float16)pb[bb];
            const half2_t r2 = {r, r};
#pragma unroll
            for (int i = 4 * bb; i < 4 * bb + 4; ++i) {
                v[i].x = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v[i].x) * r2);
                v[i].y = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v[i].y) * r2);
                v[i].z = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v[i].z) * r2);
                v[i].w = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, v[i].w) * r2);
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) *reinterpret_cast<uint4 *>(lds + srow * kDnPitch + part * 16 + 64 * i) = v[i];
        if (part == 0) row_p[srow] = pm;
    };
    // the expert's down scales: thread t < 256 takes features 8t..8t+7
    uint4 s4[4];
    if (!NV) {
        const uint4 *src = reinterpret_cast<const uint4 *>(scales + (size_t)e * kScalesPerExpert + kScalesGu) + 4 * tid;
#pragma unroll
        for (int i = 0; i < 4; ++i) s4[i] = src[i];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < kDnCodeRing - 1; ++d) fetch(d, d);
    __builtin_amdgcn_sched_barrier(0);

    // the down scales transposed to [block][feature], and each feature's
    // normalisation
    if (!NV) {
        const uint32_t w[16] = {s4[0].x, s4[0].y, s4[0].z, s4[0].w, s4[1].x, s4[1].y, s4[1].z, s4[1].w,
                                s4[2].x, s4[2].y, s4[2].z, s4[2].w, s4[3].x, s4[3].y, s4[3].z, s4[3].w};
        // feature f = 8t + k holds blocks 0,1 in w[2k] and 2,3 in w[2k+1];
        // the workgroup keeps its own features' scales (all of them give the
        // expert's largest normalisation)
        const int f_lo = quarter * kDnFeat;
        const bool own = 8 * tid >= f_lo && 8 * tid < f_lo + kDnFeat;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            uint32_t t4[4];
#pragma unroll
            for (int k2 = 0; k2 < 4; ++k2) {
                const uint32_t lo = w[2 * (2 * k2) + (bb >> 1)], hi = w[2 * (2 * k2 + 1) + (bb >> 1)];
                const uint32_t a0 = (bb & 1) ? (lo >> 16) : (lo & 0xffffu);
                const uint32_t a1 = (bb & 1) ? (hi >> 16) : (hi & 0xffffu);
                t4[k2] = a0 | (a1 << 16);
            }
            if (own) *reinterpret_cast<uint4 *>(&sc[bb][8 * tid - f_lo]) = make_uint4(t4[0], t4[1], t4[2], t4[3]);
        }
        // the expert's largest normalisation, over the features with a
        // nonzero scale (an all-zero feature's outputs are 0 whatever it is)
        float fmax = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float f = ldexpf(1.0f, -scale_shift4(w[2 * k], w[2 * k + 1]));
            if (own) fk[8 * tid - f_lo + k] = f;
            if ((w[2 * k] | w[2 * k + 1]) & 0x7f807f80u) fmax = fmaxf(fmax, f);
        }
        fmax = wave_max(fmax);
        if (lane == 0) fk_wave[wave] = fmax;
    }
    stage_store();
    __syncthreads();
    float fkmax = NV ? 1.0f : fmaxf(fmaxf(fk_wave[0], fk_wave[1]), fmaxf(fk_wave[2], fk_wave[3]));
    if (fkmax == 0.0f) fkmax = 1.0f;   // every scale of the expert is zero: o is 0
    const float to_half = 0x1p-20f / fkmax;   // a power of two
    const float tsd = NV ? tscales[3 * e + 2] : 1.0f;

    for (int pass = 0; pass < n_pass; ++pass) {
    if (PASSES && pass > 0) {
        // every wave is done with the previous rows before they are replaced
        __syncthreads();
        stage_load(pass);
        stage_store();
        __syncthreads();
    }
    const int prow0 = row0 + kDnRows * pass, prows = min(kDnRows, rows - kDnRows * pass);
    // o rows of the pass through a buffer descriptor: stores of rows past its
    // end fall outside it and are dropped by the hardware bounds check
    const __amdgpu_buffer_rsrc_t ores =
        NV ? make_buf(static_cast<float *>(o_) + (size_t)prow0 * kH, (uint32_t)prows * kH * 4)
           : make_buf(o + (size_t)prow0 * kH, (uint32_t)prows * kH * 2);
    if (!NV && quarter == 0 && tid < prows) o_scale[prow0 + tid] = row_p[tid] * fkmax * 0x1p20f;

    // fully unrolled, so ring slots are compile-time; the next tile's codes
    // (or the next pass's first tile's) are requested before this tile's
    // products
    with_tiles<kDnRows / 32>((prows + 31) >> 5, [&](auto tiles) {
    constexpr int MT = decltype(tiles)::value;
#pragma unroll
    for (int t = 0; t < kDnTiles; ++t) {
        const int cs = t % kDnCodeRing;
        __builtin_amdgcn_sched_barrier(0);
        if (t + kDnCodeRing - 1 < kDnTiles)
            fetch((t + kDnCodeRing - 1) % kDnCodeRing, t + kDnCodeRing - 1);
        else if (PASSES && pass + 1 < n_pass)
            fetch((t + kDnCodeRing - 1) % kDnCodeRing, t + kDnCodeRing - 1 - kDnTiles);
        __builtin_amdgcn_sched_barrier(0);
        const uint32_t zero = opaque(0);
        const uint8_t *abase = lds + zero;
        // this lane's codes feature and its normalised scales, as fp16 pairs
        // (NVFP4: the four E4M3 scales of each block, exact in fp16)
        const int fl = f0 + 128 * t;
        half2_t s2[4], ns[4][4];
        if constexpr (NV) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) ns[b][i] = e4m3_half2(cs4[cs][b], i);
        } else {
            const int kf = -ilogbf(fk[fl - quarter * kDnFeat + zero]);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const _Float16 h = (_Float16)ldexpf(bf16_to_f32(sc[b][fl - quarter * kDnFeat + zero]), kf);
                s2[b] = half2_t{h, h};
            }
        }
        f32x16_t acc[MT];
#pragma unroll
        for (int h = 0; h < MT; ++h)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[h][i] = 0.0f;
        // 32 k-slices of 16; the A operands and converted codes of slice
        // ks + 1 are read and built while the MFMAs of slice ks run (one wave
        // per SIMD here, so nothing else hides the LDS latency)
        auto slice_a = [&](int ks, uint4 (&dst)[MT]) {
            const int b = ks >> 3, q = (ks >> 2) & 1, j = ks & 3;
            const int grp = 16 * b + 8 * g + 4 * q + j;
#pragma unroll
            for (int h = 0; h < MT; ++h)
                dst[h] = *reinterpret_cast<const uint4 *>(abase + (32 * h + n) * kDnPitch + grp * 16);
        };
        auto slice_b = [&](int ks) -> uint4 {
            const int b = ks >> 3, q = (ks >> 2) & 1, j = ks & 3;
            // NVFP4: 8-group 16b + 8g + 4q + j, 16-block 8b + 4g + 2q + j/2
            return NV ? nv_codes_to_f16(word(cb[cs][2 * b + q], j), ns[b][2 * q + (j >> 1)])
                      : codes_to_f16_scaled(word(cb[cs][2 * b + q], j), s2[b]);
        };
        uint4 a_cur[MT], a_nxt[MT];
        slice_a(0, a_cur);
        uint4 b_cur = slice_b(0);
#pragma unroll
        for (int ks = 0; ks < 32; ++ks) {
            uint4 b_nxt = b_cur;
            if (ks + 1 < 32) {
                slice_a(ks + 1, a_nxt);
                b_nxt = slice_b(ks + 1);
            }
#pragma unroll
            for (int h = 0; h < MT; ++h) acc[h] = mfma32(b_cur, a_cur[h], acc[h]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int h = 0; h < MT; ++h) a_cur[h] = a_nxt[h];
            b_cur = b_nxt;
        }
        mfma_drain();
        // lane: token 32h + n, features 128t + 32w + 8q + 4g + 0..3 in acc[h][4q..4q+3]
        const int fb = fh + 128 * t + 32 * wave + 4 * g;
        if constexpr (NV) {
            // fp32 rows: acc times the tensor scale and the row's prescale
#pragma unroll
            for (int h = 0; h < MT; ++h) {
                const float mlt = tsd * row_p[min(32 * h + n, kDnRows - 1)];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const u32x4_t v = {__float_as_uint(acc[h][4 * q] * mlt), __float_as_uint(acc[h][4 * q + 1] * mlt),
                                       __float_as_uint(acc[h][4 * q + 2] * mlt),
                                       __float_as_uint(acc[h][4 * q + 3] * mlt)};
                    __builtin_amdgcn_raw_buffer_store_b128(v, ores, (uint32_t)((32 * h + n) * kH + fb + 8 * q) * 4, 0,
                                                           0);
                }
            }
            continue;
        }
        float4 kq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) kq[q] = *reinterpret_cast<const float4 *>(&fk[fb - quarter * kDnFeat + 8 * q + zero]);
        const uint32_t ob = (uint32_t)(n * kH + fb) * 2;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            kq[q].x *= to_half; kq[q].y *= to_half; kq[q].z *= to_half; kq[q].w *= to_half;
        }
#pragma unroll
        for (int h = 0; h < MT; ++h) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2_t v = {pack_half2(acc[h][4 * q] * kq[q].x, acc[h][4 * q + 1] * kq[q].y),
                                   pack_half2(acc[h][4 * q + 2] * kq[q].z, acc[h][4 * q + 3] * kq[q].w)};
                __builtin_amdgcn_raw_buffer_store_b64(v, ores, ob + (uint32_t)(32 * h * kH + 8 * q) * 2, 0, 0);
            }
        }
    }
    });
    }   // passes
}

int max_chunks(int T) { return min(kE, kTopK * T) + (kTopK * T + kChunkRows - 1) / kChunkRows; }

static int grid_for(int T, int tiles) {
    const int c = (max_chunks(T) + kXcds - 1) / kXcds * kXcds;
    return c * tiles;
}

void launch_gateup_mfma(const uint8_t *codes, const uint16_t *scales, const uint32_t *xt, const float *xt_scale,
                        const int *perm, const int *chunks, const int *n_chunks, int T, uint32_t *at,
                        float *at_scale, hipStream_t s) {
    auto k = chunk_long(T) ? k_gateup_mfma<false, 3> : k_gateup_mfma<false, 2>;
    hipLaunchKernelGGL(k, dim3(grid_for(T, kI / kG)), dim3(256), 0, s, codes,
                       static_cast<const void *>(scales), nullptr, xt, xt_scale, perm,
                       reinterpret_cast<const int4 *>(chunks), n_chunks, max_chunks(T), at, at_scale);
}

void launch_down_mfma(const uint8_t *codes, const uint16_t *scales, const uint32_t *at, const float *at_scale,
                      const int *chunks, const int *n_chunks, int T, uint16_t *o, float *o_scale, hipStream_t s) {
    auto k = chunk_long(T) ? k_down_mfma<false, true> : k_down_mfma<false, false>;
    hipLaunchKernelGGL(k, dim3(grid_for(T, kDnParts)), dim3(256), 0, s, codes,
                       static_cast<const void *>(scales), nullptr, at, at_scale,
                       reinterpret_cast<const int4 *>(chunks), n_chunks, max_chunks(T), static_cast<void *>(o), o_scale);
}

void launch_gateup_mfma_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscales, const uint32_t *xn,
                              const float *xn_scale, const int *perm, const int *chunks, const int *n_chunks, int T,
                              uint32_t *an, float *an_scale, hipStream_t s) {
    auto k = chunk_long(T) ? k_gateup_mfma<true, 3> : k_gateup_mfma<true, 2>;
    hipLaunchKernelGGL(k, dim3(grid_for(T, kI / kG)), dim3(256), 0, s, codes,
                       static_cast<const void *>(scales), tscales, xn, xn_scale, perm,
                       reinterpret_cast<const int4 *>(chunks), n_chunks, max_chunks(T), an, an_scale);
}

void launch_down_mfma_nvfp4(const uint8_t *codes, const uint8_t *scales, const float *tscales, const uint32_t *an,
                            const float *an_scale, const int *chunks, const int *n_chunks, int T, float *o,
                            hipStream_t s) {
    auto k = chunk_long(T) ? k_down_mfma<true, true> : k_down_mfma<true, false>;
    hipLaunchKernelGGL(k, dim3(grid_for(T, kDnParts)), dim3(256), 0, s, codes,
                       static_cast<const void *>(scales), tscales, an, an_scale,
                       reinterpret_cast<const int4 *>(chunks), n_chunks, max_chunks(T), static_cast<void *>(o), nullptr);
}

}  // namespace moe_w4
