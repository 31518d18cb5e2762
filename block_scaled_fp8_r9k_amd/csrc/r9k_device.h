// Device helpers shared by the gfx950 kernels of libr9k.
//
// Number formats: bf16 inputs are bit patterns (the top half of a binary32),
// fp8 codes are OCP e4m3fn (largest finite 448), scales are fp32.  The group
// quantisation rule (activation groups of 128 along K, weight blocks of
// 128x128) is s = max(amax, 1e-10f) / 448, code = e4m3(fp32(a / s)) with
// round-to-nearest-even and saturation at +-448: the per-token-group-128 quant
// of the r9700-stack release v0.3.1 notes ("What changed for someone running
// it"), with the workload's stated constants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace r9k {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal hint (data read once: streamed weights).
__device__ __forceinline__ uint4 load_nt16(const void *p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16-byte buffer load at byte offset `off` of the descriptor's range, with the
// non-temporal hint (cache-policy operand 2); offsets past the range read 0.
__device__ __forceinline__ uint4 load_buf_nt16(__amdgpu_buffer_rsrc_t d, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(d, (int)off, 0, 2);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// ---- bf16 ------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint2 bf16x4_rne(float a, float b, float c, float d) {
    return make_uint2(bf16_rne(a) | (bf16_rne(b) << 16), bf16_rne(c) | (bf16_rne(d) << 16));
}

// Largest |value| among the 8 bf16 in v, as a bf16 bit pattern (sign cleared).
// For non-negative finite bf16 the integer order of the bit patterns is the
// numeric order, so the maximum is taken on 16-bit integers.
__device__ __forceinline__ uint32_t absmax8_bits(uint4 v) {
    us2 a = __builtin_bit_cast(us2, v.x & 0x7FFF7FFFu);
    us2 b = __builtin_bit_cast(us2, v.y & 0x7FFF7FFFu);
    us2 c = __builtin_bit_cast(us2, v.z & 0x7FFF7FFFu);
    us2 d = __builtin_bit_cast(us2, v.w & 0x7FFF7FFFu);
    us2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    return m.x > m.y ? (uint32_t)m.x : (uint32_t)m.y;
}

// Maximum over the 16 lanes of a DPP row (lanes 16r .. 16r+15).  Every lane of
// the row must be active.  quad_perm [1,0,3,2], [2,3,0,1], then row_ror 4, 8.
__device__ __forceinline__ uint32_t max16_dpp(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));
    return v;
}

// ---- group scale and the quotient -----------------------------------------

// s = max(amax, 1e-10f) / 448, the correctly rounded fp32 quotient, as a
// multiply by RN(1/448) and one fma correction (the same refinement as the
// element division below); for amax a bf16 value, as it always is here, this
// equals the division exactly (checked over every bf16 amax on the CPU).
__device__ __forceinline__ float group_scale(float amax) {
    const float c = 1.0f / 448.0f;
    const float x = fmaxf(amax, 1e-10f);
    const float q0 = x * c;
    const float e = __builtin_fmaf(-q0, 448.0f, x);
    return __builtin_fmaf(e, c, q0);
}

// RN32(a / s) from r = RN32(1 / s) with one correction step:
// q0 = RN(a r), d = q0 s - a (exact by fma), q = RN(q0 - d r).  This is
// Markstein's division refinement (Muller et al., Handbook of Floating-Point
// Arithmetic, division chapter); over every pair of bf16 a and bf16 amax with
// |a| <= amax it yields the same e4m3 code as the correctly rounded quotient
// (checked exhaustively on the CPU and against the oracle on the GPU).  The
// residual is formed as q0 s - a rather than a - q0 s so that a = -0 gives
// q = -0 (-0 - 0 r = -0), keeping the sign of zero that the codes carry.
__device__ __forceinline__ float div_by_scale(float a, float s, float r) {
    const float q0 = a * r;
    const float d = __builtin_fmaf(q0, s, -a);
    return __builtin_fmaf(-d, r, q0);
}

// ---- e4m3 encode -------------------------------------------------------------

__device__ __forceinline__ float clamp448(float x) { return __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f); }

// Four fp32 -> four e4m3 codes in one word (byte i = value i), round to
// nearest even by the hardware converter, after clamping to +-448.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    uint32_t r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(a), clamp448(b), 0, false);
    r = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clamp448(c), clamp448(d), (int)r, true);
    return r;
}

// Quantise 8 bf16 (one uint4) with scale s and reciprocal r -> 8 codes.
__device__ __forceinline__ uint2 quant8(uint4 v, float s, float r) {
    uint2 o;
    o.x = e4m3x4(div_by_scale(bf16_lo(v.x), s, r), div_by_scale(bf16_hi(v.x), s, r),
                 div_by_scale(bf16_lo(v.y), s, r), div_by_scale(bf16_hi(v.y), s, r));
    o.y = e4m3x4(div_by_scale(bf16_lo(v.z), s, r), div_by_scale(bf16_hi(v.z), s, r),
                 div_by_scale(bf16_lo(v.w), s, r), div_by_scale(bf16_hi(v.w), s, r));
    return o;
}

// One 128-value group spread over the 16 lanes of a DPP row, 8 values (16
// bytes of bf16) per lane: returns this lane's 8 codes and the group scale.
__device__ __forceinline__ uint2 quant_group16(uint4 v, float &scale) {
    uint32_t m = max16_dpp(absmax8_bits(v));
    float s = group_scale(__uint_as_float(m << 16));
    float r = 1.0f / s;
    scale = s;
    return quant8(v, s, r);
}

// One 128-value group spread over the 4 lanes of a DPP quad, 32 values (four
// uint4 of bf16) per lane: this lane's 32 codes (two uint4) and the scale.
__device__ __forceinline__ void quant_group4(const uint4 (&v)[4], uint4 (&codes)[2], float &scale) {
    uint32_t m = max(max(absmax8_bits(v[0]), absmax8_bits(v[1])), max(absmax8_bits(v[2]), absmax8_bits(v[3])));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
    const float s = group_scale(__uint_as_float(m << 16));
    const float r = 1.0f / s;
    const uint2 a = quant8(v[0], s, r), b = quant8(v[1], s, r), c = quant8(v[2], s, r), d = quant8(v[3], s, r);
    codes[0] = make_uint4(a.x, a.y, b.x, b.y);
    codes[1] = make_uint4(c.x, c.y, d.x, d.y);
    scale = s;
}

// ---- MFMA --------------------------------------------------------------------

// D = A(16x128 e4m3) * B(128x16 e4m3) + C, fp32.  Lane l supplies row (l % 16)
// of A and column (l % 16) of B, 32 K-bytes each (the same K positions for A
// and B); D lane l holds rows 4*(l/16) .. +3 of column l % 16.  The E8M0 block
// scales of the instruction are set to 1 (127).
__device__ __forceinline__ v4f mfma_e4m3_16x16x128(v8i a, v8i b, v4f c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Pin a value computed from MFMA results where it stands.  An MFMA mixes its
// operands across the wave's lanes, so it must run with every lane enabled; a
// value used only under a lane-dependent branch (a store of rows below M) lets
// the compiler sink the MFMAs that feed it into that branch, where lanes are
// disabled and their operands drop out of the other lanes' results.  An empty
// asm that reads and writes the value makes it be computed first.
__device__ __forceinline__ void pin_acc(v4f &x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ v8i make_frag(uint4 lo, uint4 hi) {
    v8i f;
    f[0] = (int)lo.x; f[1] = (int)lo.y; f[2] = (int)lo.z; f[3] = (int)lo.w;
    f[4] = (int)hi.x; f[5] = (int)hi.y; f[6] = (int)hi.z; f[7] = (int)hi.w;
    return f;
}

}  // namespace r9k
