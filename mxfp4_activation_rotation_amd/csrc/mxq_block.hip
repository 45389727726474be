// Rotation by a B x B block for B = 16, 32, 64, 128, then MXFP4 of every
// 32-element group: the block sizes of the DuQuant++ page's ablation
// (sec. 4.3), which keeps MXFP4 groups 32 wide and varies the rotation
// block.  B = 32 is the main path: the entry point sends it to the fused
// kernel of mxq_rotate_quant (the same MFMA products, so the same bits);
// this kernel serves the error study's other sizes.
//
// Layout.  A block of B = 32 KB channels is one column of the MFMA and its KB
// input groups are KB k-steps: for the 16 blocks of a sub-tile, lane l
// supplies column l % 16 and, in k-step kappa, channels 32 kappa + 8 (l / 16)
// .. + 7 of its block (one 16-byte load each).  Output group gamma of the
// block (channels 32 gamma .. + 31) comes from two MFMA tiles h = 0, 1 whose
// rows are permuted as in the main kernel (row i -> channel
// 32 gamma + 8 (i / 4) + 4 h + i % 4), accumulated over the KB k-steps, so a
// lane again ends with 8 contiguous values of one output group.  B = 16 is
// the 32-wide case with the A operand holding two copies of the 16 x 16
// block on its diagonal.  A super-tile of 64 groups is 4 / KB sub-tiles of
// 16 blocks; its 4 code words per lane (index s KB + gamma) go through the
// same 4 x 4 lane/register transpose as the main kernel, after which lane
// L holds group KB (16 (s' / KB) + L % 16) + s' % KB, s' = L / 16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "mxq.h"
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {
namespace blk {

constexpr int kWave = 64;
constexpr int kGroup = 32;
constexpr int kTileGroups = 64;
constexpr int kBlockWaves = 4;
constexpr int kBlockThreads = kWave * kBlockWaves;

struct BlockArgs {
    const void* x;
    int64_t stride;
    const float* lambda;
    const uint16_t* r;  // B x B bf16, row-major
    uint8_t* codes;
    uint8_t* scales;
    float* y;
    int32_t tokens;
    int32_t gpr;
    int32_t tcols;     // super-tile columns
    int32_t row_step;  // waves per super-tile column
};

// Waves per SIMD each instance reaches without the tiny-block pass; stated
// to the compiler so that the pass (rare) spills rather than lowering the
// occupancy of the main loop.
// B = 64 and 128: the KB x 2 x KB A operands (32 and 128 VGPRs per lane in
// registers) live in LDS, 8 or 32 KB shared by the block's waves, each read
// by one conflict-free ds_read_b128 (64 lanes x 16 bytes in lane order) next
// to its MFMAs.  At B = 128 this frees half the register file: 3 waves per
// SIMD instead of 2 (1 with smoothing, which now also keeps the next row in
// flight).  Side by side, bit-identical: bf16 8192 x 14336 B = 128 60.0 ->
// 56.7-57.1 us, fp16 32768 x 8192 with lambda 280 -> 160 us; B = 64 54.0 ->
// 53.0 us and 133.9 -> 130.9 us.
template <int KB>
constexpr bool kLdsOperands = KB >= 2;

// (fp16 without smoothing at B = 128 keeps 2: its two exact terms of all
// four k-steps do not fit the main loop in 168 registers)
template <int XT, bool LAM, int KB>
constexpr int kWavesPerSimd = LAM ? (KB == 1 ? 4 : 3)
                                  : (KB == 1 ? 7 : KB == 2 ? 4 : (XT == MXQ_FP16 ? 2 : 3));

// fp16 activations without smoothing never need the tiny-block pass (a
// nonzero fp16 value is at least 2^-24).
template <int XT, bool LAM>
constexpr bool kGuardTiny = !(XT == MXQ_FP16 && !LAM);

// Whole-block loads for B = 64 without smoothing.  With one MFMA column per
// block, a 16-byte-per-lane load of one k-step reads 64 bytes of each of 16
// blocks: half of 16 different 128-byte lines.  Instead load i (i = 0, 1)
// of a sub-tile reads 1 KB of whole blocks: lane (q, j) takes block
// 8 i + j % 8, k-step j / 8, 8-channel chunk q.  K-step k's operand is then
// load k with its other half-row (lanes 8..15 for k = 0, lanes 0..7 for
// k = 1) taken from load 1 - k rotated by 8 lanes (DPP row_ror:8 with a
// per-bank write mask), which puts block j, k-step k, chunk q in lane
// (q, j) as the MFMA expects.  The smoothed instances do more VALU work per
// element and gain nothing from it, and for B = 128 the 4-way merge costs
// what the loads save, so they keep the per-k-step loads.
template <int KB, bool LAM>
constexpr bool kWholeBlockLoads = KB == 2 && !LAM;

__device__ __forceinline__ void merge_half_rows(const u32x4_t& l0, const u32x4_t& l1, u32x4_t& k0, u32x4_t& k1) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int a0 = static_cast<int>(l0[d]), a1 = static_cast<int>(l1[d]);
        k0[d] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(a0, a1, 0x128, 0xf, 0xc, false));
        k1[d] = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(a1, a0, 0x128, 0xf, 0x3, false));
    }
}

// The rotated-value output (YOUT) is a template parameter: a runtime branch
// around its stores would cut each row's unrolled sub-tiles into separate
// basic blocks that the scheduler cannot interleave.
template <int XT, bool LAM, int KB, bool HALF, bool YOUT>
__global__ __attribute__((amdgpu_flat_work_group_size(1, kBlockThreads),
                          amdgpu_waves_per_eu(kWavesPerSimd<XT, LAM, KB>))) void block_quant_kernel(BlockArgs a) {
    constexpr bool kFp16 = XT == MXQ_FP16;
    constexpr int kSubs = 4 / KB;  // sub-tiles per super-tile
    constexpr int kB = HALF ? 16 : 32 * KB;
    constexpr int kTerms = (XT == MXQ_BF16 && !LAM) ? 1 : ((XT == MXQ_FP16 && !LAM) ? 2 : 3);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int w = static_cast<int>(blockIdx.x) * kBlockWaves + wave;

    // A operand (g, h, k) of lane ln: element t is
    // R[32 k + 8 (ln / 16) + t][32 g + 8 (ln % 16 / 4) + 4 h + ln % 4]
    auto operand = [&](int g, int h, int k, int ln) {
        bf16x8_t op;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int row = 32 * k + 8 * (ln >> 4) + t;
            const int col = 32 * g + 8 * ((ln & 15) >> 2) + 4 * h + (ln & 3);
            uint16_t bits;
            if constexpr (HALF)
                bits = (row >> 4) == (col >> 4) ? a.r[(row & 15) * 16 + (col & 15)] : uint16_t(0);
            else
                bits = a.r[row * kB + col];
            op[t] = __builtin_bit_cast(__bf16, bits);
        }
        return op;
    };
    constexpr bool kLds = kLdsOperands<KB>;
    __shared__ __attribute__((aligned(16))) bf16x8_t a_lds[kLds ? KB * 2 * KB * kWave : 1];
    if constexpr (kLds) {
        // every wave of the block fills its share and meets the barrier
        // before any wave without work leaves
        for (int e = static_cast<int>(threadIdx.x); e < KB * 2 * KB * kWave; e += kBlockThreads) {
            const int op = e / kWave;
            a_lds[e] = operand(op / (2 * KB), (op / KB) & 1, op % KB, e % kWave);
        }
        __syncthreads();
    }
    if (w >= a.tcols * a.row_step) return;
    const int tc = w % a.tcols;
    const int r0 = w / a.tcols;
    const int j = lane & 15;
    const int q = lane >> 4;
    const uint32_t gpr = static_cast<uint32_t>(a.gpr);
    const int p0 = tc * kTileGroups;

    // A operands in registers (B <= 32), or read from LDS where they are used
    bf16x8_t A[kLds ? 1 : KB][2][kLds ? 1 : KB];
    if constexpr (!kLds) {
#pragma unroll
        for (int g = 0; g < KB; ++g)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int k = 0; k < KB; ++k) A[g][h][k] = operand(g, h, k, lane);
    }
    auto opA = [&](int g, int h, int k) -> bf16x8_t {
        if constexpr (kLds)
            return a_lds[((g * 2 + h) * KB + k) * kWave + lane];
        else
            return A[g][h][k];
    };

    // 1 / lambda for the lane's 8 channels of every (sub-tile, k-step)
    float il[kSubs][KB][8];
    if constexpr (LAM) {
        const auto lrsrc = row_rsrc(a.lambda, gpr * kGroup * 4);
#pragma unroll
        for (int s = 0; s < kSubs; ++s)
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int grp = p0 + KB * (16 * s + j) + k;
                const uint32_t off = (static_cast<uint32_t>(grp) * kGroup + 8 * q) * 4;
                const u32x4_t l0 = __builtin_amdgcn_raw_buffer_load_b128(lrsrc, off, 0, 0);
                const u32x4_t l1 = __builtin_amdgcn_raw_buffer_load_b128(lrsrc, off + 16, 0, 0);
                const bool valid = grp < a.gpr;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    il[s][k][t] = valid ? __builtin_amdgcn_rcpf(as_f32(l0[t])) : 0.0f;
                    il[s][k][4 + t] = valid ? __builtin_amdgcn_rcpf(as_f32(l1[t])) : 0.0f;
                }
            }
    }

    const uint32_t row_bytes = gpr * kGroup * 2;
    const char* xb = static_cast<const char*>(a.x);

    // x' of the lane's 8 channels of k-step k of sub-tile s, in fp32.
    auto smoothed = [&](const u32x4_t& xq, int s, int k, float* f) {
        widen8<kFp16>(xq, f);
        if constexpr (LAM) {
#pragma unroll
            for (int t = 0; t < 8; ++t) f[t] *= il[s][k][t];
        }
    };
    // The rotated values of sub-tile s: d0[g], d1[g] hold output group g's
    // two halves.  SHIFT: x' is formed 2^ksh times larger (rounded to fp32
    // once from the exact product in fp64), for the tiny-block pass.
    auto product = [&](const u32x4_t (&xin)[kSubs][KB], int s, int ksh, f32x4_t (&d0)[KB], f32x4_t (&d1)[KB],
                       auto shift_tag) {
        constexpr bool SHIFT = decltype(shift_tag)::value;
#pragma unroll
        for (int g = 0; g < KB; ++g) d0[g] = d1[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (kTerms == 1 && !SHIFT) {
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xin[s][k]);
#pragma unroll
                for (int g = 0; g < KB; ++g) {
                    d0[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opA(g, 0, k), b, d0[g], 0, 0, 0);
                    d1[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opA(g, 1, k), b, d1[g], 0, 0, 0);
                }
            }
        } else {
            float f[KB][8];
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                if constexpr (SHIFT) {
                    widen8<kFp16>(xin[s][k], f[k]);
                    if constexpr (LAM) {
                        const double p = __builtin_bit_cast(double, static_cast<uint64_t>(1023 + ksh) << 52);
#pragma unroll
                        for (int t = 0; t < 8; ++t)
                            f[k][t] = static_cast<float>(static_cast<double>(f[k][t]) *
                                                         (static_cast<double>(il[s][k][t]) * p));
                    } else {
                        // 16-bit x times 2^ksh is exact (the block's |x| 2^ksh < 2^64)
                        const float p = as_f32(static_cast<uint32_t>(127 + ksh) << 23);
#pragma unroll
                        for (int t = 0; t < 8; ++t) f[k][t] *= p;
                    }
                } else {
                    smoothed(xin[s][k], s, k, f[k]);
                }
            }
            if constexpr (LAM && !SHIFT) {
                // x' as two bf16 terms rounded to nearest, as in the main
                // kernel (|x' - hi - lo| <= 2^-18 |x'|), so B = 32 gives its bits
                typedef __attribute__((ext_vector_type(2))) float f32x2_t;
                typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
#pragma unroll
                for (int k = 0; k < KB; ++k) {
                    u32x4_t hi, lo;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const f32x2_t p2 = f32x2_t{f[k][2 * i], f[k][2 * i + 1]};
                        const bf16x2_t h = __builtin_convertvector(p2, bf16x2_t);
                        hi[i] = __builtin_bit_cast(uint32_t, h);
                        lo[i] = __builtin_bit_cast(uint32_t,
                                                   __builtin_convertvector(p2 - __builtin_convertvector(h, f32x2_t), bf16x2_t));
                    }
#pragma unroll
                    for (int g = 0; g < KB; ++g) {
                        d0[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opA(g, 0, k), __builtin_bit_cast(bf16x8_t, hi), d0[g], 0, 0, 0);
                        d1[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opA(g, 1, k), __builtin_bit_cast(bf16x8_t, hi), d1[g], 0, 0, 0);
                        d0[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opA(g, 0, k), __builtin_bit_cast(bf16x8_t, lo), d0[g], 0, 0, 0);
                        d1[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opA(g, 1, k), __builtin_bit_cast(bf16x8_t, lo), d1[g], 0, 0, 0);
                    }
                }
                return;
            }
            constexpr int kT = SHIFT && kTerms == 1 ? 1 : kTerms;
#pragma unroll
            for (int term = 0; term < kT; ++term) {
#pragma unroll
                for (int k = 0; k < KB; ++k) {
                    u32x4_t bt;
#pragma unroll
                    for (int i = 0; i < 4; ++i) bt[i] = bf16_pair_hi(f[k][2 * i], f[k][2 * i + 1]);
                    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bt);
#pragma unroll
                    for (int g = 0; g < KB; ++g) {
                        d0[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opA(g, 0, k), b, d0[g], 0, 0, 0);
                        d1[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(opA(g, 1, k), b, d1[g], 0, 0, 0);
                    }
                    if (term + 1 < kT) {
#pragma unroll
                        for (int t = 0; t < 8; ++t) f[k][t] = bf16_residual(f[k][t]);
                    }
                }
            }
        }
    };
    auto store_y = [&](int64_t r, int s, int g, const float (&v)[8], int ksh) {
        const float down = pow2_neg(ksh);
        const auto yrsrc = row_rsrc(a.y + r * a.gpr * kGroup, gpr * kGroup * 4);
        const uint32_t grp = static_cast<uint32_t>(p0 + KB * (16 * s + j) + g);
        const uint32_t off = (grp * kGroup + 8 * q) * 4;
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4_t{as_u32(v[0] * down), as_u32(v[1] * down), as_u32(v[2] * down), as_u32(v[3] * down)}, yrsrc, off,
            0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4_t{as_u32(v[4] * down), as_u32(v[5] * down), as_u32(v[6] * down), as_u32(v[7] * down)}, yrsrc,
            off + 16, 0, 0);
    };

    // One row.  FIX (the pass for rows with tiny groups, below): a block
    // column whose output groups all have a rotated maximum below 2^-64 is
    // recomputed from x' * 2^k, k from the block's largest |x'|; a block with
    // a larger output group keeps its values, whose errors scale with the
    // block's norm.  Returns whether some group of the row had S < 61.
    // The operands of row r, in the MFMA's layout.  Rows past the end read
    // through an empty range (zeros, no traffic), so the prefetch below needs
    // no branch: a conditional load would make the wait before the current
    // row's first use count the next row's loads too.
    auto load_row = [&](u32x4_t (&xin)[kSubs][KB], int64_t r, auto nt_tag) {
        constexpr int aux = decltype(nt_tag)::value ? kAuxNT : 0;
        const bool in = r < a.tokens;
        const auto rsrc = row_rsrc(xb + (in ? r : 0) * a.stride * 2, in ? row_bytes : 0u);
        if constexpr (kWholeBlockLoads<KB, LAM>) {
#pragma unroll
            for (int s = 0; s < kSubs; ++s) {
                const uint32_t base = static_cast<uint32_t>(p0) * kGroup * 2 + s * 2048 +
                                      static_cast<uint32_t>(j & 7) * 128 + static_cast<uint32_t>(j >> 3) * 64 + 16 * q;
                const u32x4_t l0 = __builtin_amdgcn_raw_buffer_load_b128(rsrc, base, 0, aux);
                const u32x4_t l1 = __builtin_amdgcn_raw_buffer_load_b128(rsrc, base + 1024, 0, aux);
                merge_half_rows(l0, l1, xin[s][0], xin[s][1]);
            }
        } else {
#pragma unroll
            for (int s = 0; s < kSubs; ++s)
#pragma unroll
                for (int k = 0; k < KB; ++k) {
                    const uint32_t grp = static_cast<uint32_t>(p0 + KB * (16 * s + j) + k);
                    xin[s][k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (grp * kGroup + 8 * q) * 2, 0, aux);
                }
        }
    };

    // One row.  FIX (the pass for rows with tiny groups, below): a block
    // column whose output groups all have a rotated maximum below 2^-64 is
    // recomputed from x' * 2^k, k from the block's largest |x'|; a block with
    // a larger output group keeps its values, whose errors scale with the
    // block's norm.  Returns whether some group of the row had S < 61.
    auto row_body = [&](int64_t r, const u32x4_t (&xin)[kSubs][KB], auto fix_tag) -> bool {
        constexpr bool FIX = decltype(fix_tag)::value;
        // (LDS operands are re-read for every row, not held in registers
        // across rows: the clobber keeps the compiler from hoisting them)
        if constexpr (kLds) asm volatile("" ::: "memory");
        uint32_t word[4], sc[4];
        bool redo = false;
#pragma unroll
        for (int s = 0; s < kSubs; ++s) {
            f32x4_t d0[KB], d1[KB];
            product(xin, s, 0, d0, d1, std::false_type{});
            uint32_t sb[KB], cb[KB];
            int ksh = 0;
            uint32_t colmax = 0;
#pragma unroll
            for (int g = 0; g < KB; ++g) {
                float v[8];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    v[t] = d0[g][t];
                    v[4 + t] = d1[g][t];
                }
                sb[g] = cb[g] = e8m0_scale_bits(group_amax8(v));
                colmax = sb[g] > colmax ? sb[g] : colmax;
            }
            if constexpr (FIX) {
                const bool tiny = colmax < kTinyScaleBits;
                if (any_lane(tiny)) {
                    redo = true;
                    float ax = 0.0f;
#pragma unroll
                    for (int k = 0; k < KB; ++k) {
                        float f[8];
                        smoothed(xin[s][k], s, k, f);
                        ax = fmaxf(ax, group_amax8(f));
                    }
                    ksh = tiny ? tiny_shift(ax) : 0;
                    f32x4_t e0[KB], e1[KB];
                    product(xin, s, ksh, e0, e1, std::true_type{});
#pragma unroll
                    for (int g = 0; g < KB; ++g) {
                        float w[8];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            w[t] = e0[g][t];
                            w[4 + t] = e1[g][t];
                        }
                        uint32_t s2, c2;
                        shifted_scale_bits(group_amax8(w), ksh, s2, c2);
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            d0[g][t] = tiny ? e0[g][t] : d0[g][t];
                            d1[g][t] = tiny ? e1[g][t] : d1[g][t];
                        }
                        sb[g] = tiny ? s2 : sb[g];
                        cb[g] = tiny ? c2 : cb[g];
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < KB; ++g) {
                float v[8];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    v[t] = d0[g][t];
                    v[4 + t] = d1[g][t];
                }
                sc[s * KB + g] = sb[g] >> 23;
                word[s * KB + g] = encode8(v, as_f32(cb[g]));
                if constexpr (YOUT) store_y(r, s, g, v, ksh);
            }
        }
        transpose_words(word);
        const uint32_t S = q == 0 ? sc[0] : q == 1 ? sc[1] : q == 2 ? sc[2] : sc[3];
        const uint32_t grp = static_cast<uint32_t>(p0 + KB * (16 * (q / KB) + j) + q % KB);
        if (!FIX || redo) {
            const auto crsrc = row_rsrc(a.codes + r * a.gpr * 16, gpr * 16);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{word[0], word[1], word[2], word[3]}, crsrc, grp * 16, 0,
                                                   kAuxNT);
            const auto srsrc = row_rsrc(a.scales + r * a.gpr, gpr);
            __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(S), srsrc, grp, 0, 0);
        }
        // (groups past the row end, zeros whose stores are dropped, do not count)
        bool tiny = S < (kTinyScaleBits >> 23) && grp < gpr;
        if constexpr (!FIX) {
            // A block of zero inputs (padding rows of a serving batch) has
            // x' = 0 exactly, so its codes and scales are exact already: only
            // blocks holding a nonzero input bit pattern count (bit j of
            // nzm[s]: block j of sub-tile s).  The ballots run only where some
            // group fell below the bound.
            if (any_lane(tiny)) {
                uint32_t nzm[kSubs];
#pragma unroll
                for (int s = 0; s < kSubs; ++s) {
                    uint32_t o = 0;
#pragma unroll
                    for (int k = 0; k < KB; ++k) o |= xin[s][k][0] | xin[s][k][1] | xin[s][k][2] | xin[s][k][3];
                    const uint64_t b = __builtin_amdgcn_ballot_w64((o & 0x7fff7fffu) != 0u);
                    const uint64_t f = b | (b >> 32);
                    nzm[s] = static_cast<uint32_t>(f | (f >> 16)) & 0xffffu;
                }
                uint32_t nz = nzm[0];
#pragma unroll
                for (int s = 1; s < kSubs; ++s) nz = q / KB == s ? nzm[s] : nz;
                tiny = tiny && ((nz >> j) & 1u);
            }
        }
        return tiny;
    };

    bool tiny_seen = false;
    if constexpr (KB == 2 || (KB == 4 && LAM)) {
        // Two row buffers alternate: the next row is in flight while the
        // current one computes.  Measured side by side it helps B = 64 and
        // smoothed B = 128 (170 -> 160 us on fp16 32768 x 8192): B <= 32 runs
        // more waves per SIMD (up to 7), which hide the latency already, and
        // unsmoothed B = 128 stays level (56.7 against 57.1 us).
        u32x4_t bufA[kSubs][KB], bufB[kSubs][KB];
        const int64_t rs = a.row_step;
        load_row(bufA, __builtin_amdgcn_readfirstlane(r0), std::true_type{});
        for (int r_loop = r0; r_loop < a.tokens; r_loop += 2 * a.row_step) {
            const int64_t r = __builtin_amdgcn_readfirstlane(r_loop);
            load_row(bufB, r + rs, std::true_type{});
            tiny_seen |= row_body(r, bufA, std::false_type{});
            if (r + rs >= a.tokens) break;
            load_row(bufA, r + 2 * rs, std::true_type{});
            tiny_seen |= row_body(r + rs, bufB, std::false_type{});
        }
    } else {
        for (int r_loop = r0; r_loop < a.tokens; r_loop += a.row_step) {
            const int64_t r = __builtin_amdgcn_readfirstlane(r_loop);
            u32x4_t xin[kSubs][KB];
            load_row(xin, r, std::true_type{});
            tiny_seen |= row_body(r, xin, std::false_type{});
        }
    }
    // Rows holding a group with S < 61 (rare) are redone; the wave first waits
    // for its own first stores of these rows, so the second ones land after.
    if (kGuardTiny<XT, LAM> && any_lane(tiny_seen)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        for (int r_loop = r0; r_loop < a.tokens; r_loop += a.row_step) {
            const int64_t r = __builtin_amdgcn_readfirstlane(r_loop);
            u32x4_t xin[kSubs][KB];
            load_row(xin, r, std::false_type{});
            row_body(r, xin, std::true_type{});
        }
    }
}

bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

template <int XT, bool LAM, int KB, bool HALF, bool YOUT>
int waves_per_cu() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, block_quant_kernel<XT, LAM, KB, HALF, YOUT>, kBlockThreads,
                                                     0) != hipSuccess ||
        blocks <= 0)
        blocks = 1;
    v = blocks * kBlockWaves;
    cached.store(v, std::memory_order_relaxed);
    return v;
}

template <int XT, bool LAM, int KB, bool HALF, bool YOUT>
mxq_status launch_y(BlockArgs a, hipStream_t st) {
    a.tcols = (a.gpr + kTileGroups - 1) / kTileGroups;
    // The plan fills at most 8 waves per CU (two per SIMD), each walking more
    // rows, whatever the occupancy allows: side by side (bf16 8192 x 14336)
    // B = 16 52.8 -> 48.9 us, B = 64 52.7 -> 48.4 us, B = 128 57.2 -> 55.0 us,
    // and fp16 32768 x 8192 with lambda B = 16 124.0 -> 116.3 us, B = 64
    // level; 6 or 12 waves per CU were slower.  Smoothed B = 128 keeps its
    // 12 (164.5 against 168.9 us with 8).
    constexpr int kCapWavesPerCu = (KB == 4 && LAM) ? 1 << 20 : 8;
    const int wpc = waves_per_cu<XT, LAM, KB, HALF, YOUT>();
    const int64_t slots = static_cast<int64_t>(device_cu_count()) * (wpc < kCapWavesPerCu ? wpc : kCapWavesPerCu);
    int64_t rs = slots / a.tcols;
    if (rs < 1) rs = 1;
    if (rs > a.tokens) rs = a.tokens;
    a.row_step = static_cast<int32_t>(rs);
    const int64_t waves = static_cast<int64_t>(a.tcols) * rs;
    const int blocks = static_cast<int>((waves + kBlockWaves - 1) / kBlockWaves);
    hipLaunchKernelGGL((block_quant_kernel<XT, LAM, KB, HALF, YOUT>), dim3(blocks), dim3(kBlockThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

template <int XT, bool LAM, int KB, bool HALF>
mxq_status launch(const BlockArgs& a, hipStream_t st) {
    return a.y ? launch_y<XT, LAM, KB, HALF, true>(a, st) : launch_y<XT, LAM, KB, HALF, false>(a, st);
}

template <int XT, bool LAM>
mxq_status dispatch_block(const BlockArgs& a, int block, hipStream_t st) {
    switch (block) {
        case 16: return launch<XT, LAM, 1, true>(a, st);
        case 64: return launch<XT, LAM, 2, false>(a, st);
        default: return launch<XT, LAM, 4, false>(a, st);
    }
}

}  // namespace blk
}  // namespace mxq

using namespace mxq::blk;

extern "C" mxq_status mxq_rotate_quant_block(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                             int64_t x_row_stride, const float* lambda, const uint16_t* r_block,
                                             int32_t block, uint8_t* codes, uint8_t* scales, float* y_rot,
                                             void* stream) {
    if (x_dtype != MXQ_BF16 && x_dtype != MXQ_FP16) return MXQ_ERR_DTYPE;
    if (block != 16 && block != 32 && block != 64 && block != 128) return MXQ_ERR_SHAPE;
    if (tokens < 0 || channels < 0 || channels % kGroup || channels % block || tokens >= (int64_t(1) << 31) ||
        channels > (int64_t(1) << 28))
        return MXQ_ERR_SHAPE;
    if (block == 32)
        return mxq::rotate_impl(x, x_dtype, tokens, channels, x_row_stride, lambda, r_block, codes, scales, y_rot,
                                stream, false);
    if (tokens == 0 || channels == 0) return MXQ_OK;
    if (!x || !r_block || !codes || !scales) return MXQ_ERR_NULL;
    if (x_row_stride < channels) return MXQ_ERR_STRIDE;
    if (!aligned_to(x, 16) || (x_row_stride * 2) % 16 || !aligned_to(codes, 16) || !aligned_to(r_block, 2) ||
        (lambda && !aligned_to(lambda, 16)) || (y_rot && !aligned_to(y_rot, 16)))
        return MXQ_ERR_ALIGN;
    BlockArgs a{x, x_row_stride, lambda, r_block, codes, scales, y_rot, static_cast<int32_t>(tokens),
                static_cast<int32_t>(channels / kGroup), 0, 0};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (x_dtype == MXQ_BF16)
        return lambda ? dispatch_block<MXQ_BF16, true>(a, block, st) : dispatch_block<MXQ_BF16, false>(a, block, st);
    return lambda ? dispatch_block<MXQ_FP16, true>(a, block, st) : dispatch_block<MXQ_FP16, false>(a, block, st);
}
