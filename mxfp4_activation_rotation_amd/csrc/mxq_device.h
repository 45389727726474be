// Device-side building blocks for gfx950 (CDNA4): MXFP4 group encoding and
// the bf16 term split feeding the matrix cores.
//
// Encoding follows the OCP Microscaling Formats v1.0 FP32-to-MX conversion:
// shared exponent e = floor(log2 amax) - 2 clamped to [-127, 127] (E8M0 byte
// e + 127), elements rounded to the nearest E2M1 value of y / 2^e with
// ties-to-even and saturation.  The DuQuant++ page (sec. 2.1) describes the
// same two steps: group amax -> shared scale, then round each normalized
// element to the nearest 4-bit float.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// Largest |v| of a group whose 32 values sit 8 per lane in lanes j, j+16,
// j+32, j+48: in-lane max, then v_permlane32_swap and v_permlane16_swap with
// both operands equal, each leaving x[l] and x[l ^ 32] (resp. l ^ 16) in the
// two results.
__device__ __forceinline__ float group_amax8(const float* v) {
    float m0 = fmaxf(fabsf(v[0]), fabsf(v[1]));
    float m1 = fmaxf(fabsf(v[2]), fabsf(v[3]));
    m0 = fmaxf(m0, fmaxf(fabsf(v[4]), fabsf(v[5])));
    m1 = fmaxf(m1, fmaxf(fabsf(v[6]), fabsf(v[7])));
    uint32_t m = as_u32(fmaxf(m0, m1));
    const auto s32 = __builtin_amdgcn_permlane32_swap(m, m, false, false);
    m = as_u32(fmaxf(as_f32(s32[0]), as_f32(s32[1])));
    const auto s16 = __builtin_amdgcn_permlane16_swap(m, m, false, false);
    return fmaxf(as_f32(s16[0]), as_f32(s16[1]));
}

// E8M0 scale of a group maximum m (finite, m >= 0), returned as S << 23, with
// S = clamp(floor(log2 m) - 2, -127, 127) + 127.  As an fp32 pattern that is
// 2^(S-127) for S >= 1 and +0.0 for S = 0; the FP4 converter reads only the
// exponent field, so both mean 2^(S-127) to it.  For a normal fp32 m,
// floor(log2 m) is its biased exponent field minus 127, so S = field - 2;
// subnormal or zero m (field 0) and fields 1 and 2 clamp to S = 0.  One
// saturating subtract on the exponent bits does both.  A finite fp32 never
// gives S above 252.
__device__ __forceinline__ uint32_t e8m0_scale_bits(float m) {
    return __builtin_elementwise_sub_sat(as_u32(m) & 0x7f800000u, 2u << 23);
}

// A code nibble whose magnitude bits are 0 is made +0 (0x0): the gfx950
// converter keeps the sign of a negative value that rounds to zero (0x8).
// Per nibble, (mag + 7) has bit 3 set exactly when mag != 0, and the sum
// never carries into the next nibble.
__device__ __forceinline__ uint32_t drop_negative_zero(uint32_t d) {
    const uint32_t mag = d & 0x77777777u;
    const uint32_t nonzero = (mag + 0x77777777u) & 0x88888888u;
    return mag | (d & nonzero);
}

// Eight fp32 values -> one dword of E2M1 codes, element i in nibble i.
// v_cvt_scalef32_pk_fp4_f32 divides by 2^(field - 127) of `scale`'s biased
// exponent field (field 0 meaning 2^-127), rounds to nearest even, saturates
// at +-6, and writes its first operand to the low nibble of the selected byte.
__device__ __forceinline__ uint32_t encode8(const float* v, float scale) {
    uint32_t d = 0;
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[0], v[1], scale, 0);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[2], v[3], scale, 1);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[4], v[5], scale, 2);
    d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, v[6], v[7], scale, 3);
    return drop_negative_zero(d);
}

// Upper 16 bits of a and b as one bf16 pair {a_hi in the low half, b_hi in
// the high half}: the bf16 truncation of two fp32 values in one v_perm_b32.
__device__ __forceinline__ uint32_t bf16_pair_hi(float a, float b) {
    return __builtin_amdgcn_perm(as_u32(b), as_u32(a), 0x07060302u);
}

// fp32 value minus its bf16 truncation (exact in fp32).
__device__ __forceinline__ float bf16_residual(float a) {
    return a - as_f32(as_u32(a) & 0xffff0000u);
}

// ---- groups of tiny magnitude ----------------------------------------------
// The exact bf16 terms of x' stop being exact below bf16's smallest subnormal
// (2^-133), and products on the matrix cores below fp32's normal range lose
// bits, so a group whose rotated values are all tiny would carry errors that
// are large against its own norm.  A group whose rotated maximum is below
// 2^-64 (scale byte below 61) is therefore recomputed from x' * 2^k: the
// scale follows from the shifted maximum minus k (clamped at -127 like any
// other), and the converter divides the shifted values by 2^(e + k), which
// gives the codes of the unshifted group.  Above 2^-64 every lost bit is
// below 2^-57 of the group's norm.
constexpr uint32_t kTinyScaleBits = 61u << 23;  // S << 23 of a group maximum 2^-64

// Shift k in [0, 64] for a group whose largest |x'| is ax: x' * 2^k stays
// below 2^64, so the shifted products cannot overflow whatever the block is
// (for an orthogonal block a tiny group has ax < 2^-60, so k = 64).
__device__ __forceinline__ int tiny_shift(float ax) {
    const int k = 64 - __builtin_amdgcn_frexp_expf(ax);  // ax < 2^frexp_exp; 0 for ax = 0
    return k < 0 ? 0 : (k > 64 ? 64 : k);
}

// Scale bits (S << 23) and converter scale bits of a group computed 2^k
// times its size, from the shifted group maximum.
__device__ __forceinline__ void shifted_scale_bits(float amax_shifted, int k, uint32_t& s_bits,
                                                   uint32_t& conv_bits) {
    s_bits = __builtin_elementwise_sub_sat(as_u32(amax_shifted) & 0x7f800000u, static_cast<uint32_t>(2 + k) << 23);
    conv_bits = s_bits + (static_cast<uint32_t>(k) << 23);
}

// 2^-k as fp32, k in [0, 64].
__device__ __forceinline__ float pow2_neg(int k) { return as_f32(static_cast<uint32_t>(127 - k) << 23); }

// Does the condition hold in any lane of the wave?  (A scalar branch on the
// result keeps the rare path out of the common one.)
__device__ __forceinline__ bool any_lane(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0; }

// Widen 8 packed 16-bit elements (one 16-byte load) to fp32, element order kept.
template <bool IS_FP16>
__device__ __forceinline__ void widen8(u32x4_t q, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if constexpr (IS_FP16) {
            f[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(q[i] & 0xffffu)));
            f[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(q[i] >> 16)));
        } else {
            f[2 * i] = as_f32(q[i] << 16);
            f[2 * i + 1] = as_f32(q[i] & 0xffff0000u);
        }
    }
}

__device__ __forceinline__ void widen4_f32(u32x4_t q, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = as_f32(q[i]);
}

// Buffer resource for `bytes` bytes at `base` (raw buffer, stride 0): loads
// beyond `bytes` return zero and stores beyond it are dropped, which is how
// lanes of groups past the end of a row are handled without branches.
// base and bytes must be the same in every lane of the wave (a resource
// lives in scalar registers); they are read from the first active lane.
// Without that the compiler, which cannot always prove a row address
// uniform through 64-bit index arithmetic, wraps every buffer access in a
// loop over the distinct values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(p & 0xffffffffu)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(p >> 32)));
    void* u = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, 0, __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), 0x00020000);
}

constexpr int kAuxNT = 2;  // cache policy bits of buffer ops: non-temporal

// 4x4 transpose of one register per sub-tile across the lanes j, j+16, j+32,
// j+48: the word in lane 16 k + j, register s moves to lane 16 s + j,
// register k.  Stage one exchanges lane bit 5 with register bit 1
// (v_permlane32_swap swaps the upper 32 lanes of its first operand with the
// lower 32 lanes of its second); stage two exchanges lane bit 4 with register
// bit 0 (v_permlane16_swap swaps the odd 16-lane rows of its first operand
// with the even rows of its second).
__device__ __forceinline__ void transpose_words(uint32_t (&w)[4]) {
#pragma unroll
    for (int s0 = 0; s0 < 2; ++s0) {
        const auto r = __builtin_amdgcn_permlane32_swap(w[s0], w[2 + s0], false, false);
        w[s0] = r[0];
        w[2 + s0] = r[1];
    }
#pragma unroll
    for (int s1 = 0; s1 < 2; ++s1) {
        const auto r = __builtin_amdgcn_permlane16_swap(w[2 * s1], w[2 * s1 + 1], false, false);
        w[2 * s1] = r[0];
        w[2 * s1 + 1] = r[1];
    }
}

}  // namespace mxq
