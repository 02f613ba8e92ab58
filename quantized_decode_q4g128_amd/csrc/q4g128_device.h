// Device-side building blocks shared by the product kernel and the dequant
// export kernel, so both unpack codes the same way.
//
// Weight format (Token Rush README, weight format paragraph): 4-bit codes q in
// groups of 128 along K, one bf16 scale s and one bf16 minimum m per group,
// w = q*s + m.  Packing: word j of column n holds codes k = 8j..8j+7, code
// 8j+i in bits 4i..4i+3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4g128 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// bf16 128.0 (sign 0, exponent 134, fraction 0) in both 16-bit halves.  The
// fraction of a bf16 at 128 counts whole units, so OR-ing a 4-bit code into
// the low fraction bits gives exactly 128 + q.
constexpr uint32_t kBiasPair = 0x43004300u;
constexpr float kBias = 128.0f;
// bf16 1.0 in both halves.
constexpr uint32_t kOnePair = 0x3F803F80u;

// The two constants of the unpack held in registers (the mask in a scalar
// register, the bias pair in a vector register), so that each pair costs one
// v_and_or_b32: a gfx9 VOP3 instruction takes no literal operand.
struct UnpackConsts {
    uint32_t mask;   // 0x000F000F: nibble 0 of each 16-bit half
    uint32_t bias;   // kBiasPair
};

__device__ __forceinline__ UnpackConsts unpack_consts()
{
    UnpackConsts c;
    asm volatile("s_mov_b32 %0, 0xf000f" : "=s"(c.mask));
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(c.bias));
    return c;
}

// One packed word -> four bf16 pairs holding 128 + code.  Pair p carries code p
// (k = 8j + p) in its low half and code p + 4 (k = 8j + p + 4) in its high half:
// the mask keeps nibble p of each 16-bit half after the shift.
__device__ __forceinline__ u32x4 unpack_biased(uint32_t w, UnpackConsts c)
{
    u32x4 r;
    r.x = (w & c.mask) | c.bias;
    r.y = ((w >> 4) & c.mask) | c.bias;
    r.z = ((w >> 8) & c.mask) | c.bias;
    r.w = ((w >> 12) & c.mask) | c.bias;
    return r;
}

// Raw buffer descriptor over [base, base + bytes) for gfx9 buffer loads.
// Reads at or past `bytes` return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Each lane takes the four words that lane src_lane holds in v (one LDS
// crossbar permute per word; no LDS memory is used).
__device__ __forceinline__ u32x4 lane_gather(const u32x4 &v, int src_lane)
{
    const int a = src_lane * 4;
    u32x4 r;
    r.x = (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.x);
    r.y = (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.y);
    r.z = (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.z);
    r.w = (uint32_t)__builtin_amdgcn_ds_bpermute(a, (int)v.w);
    return r;
}

// Per lane: a where take_a, else b.
__device__ __forceinline__ u32x4 pick(bool take_a, const u32x4 &a, const u32x4 &b)
{
    u32x4 r;
    r.x = take_a ? a.x : b.x;
    r.y = take_a ? a.y : b.y;
    r.z = take_a ? a.z : b.z;
    r.w = take_a ? a.w : b.w;
    return r;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// bf16 held in the low / high half of a 32-bit register -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Eight consecutive bf16 x values x0..x7 (four 32-bit words, low half first)
// reordered into the pair order unpack_biased produces: (x0,x4) (x1,x5)
// (x2,x6) (x3,x7).  Applying the same order to both operands of a dot
// product leaves its set of products unchanged.
__device__ __forceinline__ u32x4 pair_order(u32x4 v)
{
    u32x4 r;
    r.x = (v.x & 0xFFFFu) | (v.z << 16);
    r.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    r.z = (v.y & 0xFFFFu) | (v.w << 16);
    r.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    return r;
}

// D += A * B on a 16x16 fp32 tile, 32-deep bf16 contraction (gfx950 MFMA).
// Lane l supplies row l%16 of A and column l%16 of B, k-slots 8*(l/16)..+7,
// and holds D rows 4*(l/16)..+3 of column l%16.
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 d)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), d, 0, 0, 0);
}

}  // namespace q4g128
