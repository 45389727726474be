// gfx950 kernels and the C ABI declared in include/mxq.h.
//
// The online path of the DuQuant++ page ("DuQuant++: block-aligned rotation
// quantization for MXFP4 activation outliers"): X * Lambda^-1 * R with R block
// diagonal (one shared 32x32 block, sec. 3.2-3.3), followed by MXFP4 encoding
// of every 32-element group (sec. 2.1), in a single pass over HBM (the fused
// operator of sec. 5.2 item 1 and sec. 5.4 item 3, extended with the
// quantization).
//
// Work decomposition.  A wave owns a super-tile: 64 consecutive groups (2048
// channels) of one token row, processed as four sub-tiles of 16 groups.  In a
// sub-tile, lane l handles quarter q = l / 16 (channels 8q..8q+7) of group
// j = l % 16, so each of the wave's four 16-byte loads per lane covers 1 KB
// contiguously.  The grid is persistent: each wave keeps one super-tile
// column (its lambda values stay in registers) and walks down the rows with a
// fixed row step, keeping the next batch of rows in flight (non-temporal
// loads: the activations are read exactly once).
//
// Rotation on the matrix cores (sec. 3.3 asks for the small dense product to
// run on matrix hardware, and the pitfalls list, item 4, for a batched GEMM
// over the [..., groups, 32] view rather than one big sparse product).  Per
// sub-tile and bf16 term we form Y^T = R^T X^T with two
// v_mfma_f32_16x16x32_bf16 (output channels split in two halves h = 0, 1):
//   B operand = the sub-tile's activations: lane l supplies column (group)
//               l % 16 and k-slots 8 (l / 16) + t -- the 8 channels it loaded;
//   A operand = R^T with permuted rows, register-resident for the kernel:
//               row i of MFMA h carries output channel 8 (i / 4) + 4 h + i % 4;
//   D         = lane l, register r holds row 4 (l / 16) + r of column l % 16,
//               i.e. output channel 8 q + 4 h + r of group j.
// So each lane ends with the 8 contiguous rotated values y[8q .. 8q+7] of its
// group: the group maximum is an in-lane max plus two cross-lane swaps
// (lanes l ^ 32, l ^ 16), and the lane packs them into one 4-byte code word.
// After the four sub-tiles, a 4x4 transpose of the code words across lanes
// j, j+16, j+32, j+48 (two v_permlane32_swap, two v_permlane16_swap) leaves
// lane l with all 16 code bytes of group l of the super-tile: the wave writes
// 1 KB of codes and 64 scale bytes, both contiguous and in lane order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "../../include/mxq.h"
#include "mxq_device.h"
#include "mxq_internal.h"

// Resident waves per CU and rows in flight per wave: one setting for the
// single-term kernels (bf16 rotate, plain quantization), one for the kernels
// that split activations into several bf16 terms (fp16 and/or lambda).
#ifndef MXQ_WAVES_PER_CU
#define MXQ_WAVES_PER_CU 8
#endif
#ifndef MXQ_BATCH
#define MXQ_BATCH 1
#endif
#ifndef MXQ_WAVES_PER_CU_SPLIT
#define MXQ_WAVES_PER_CU_SPLIT 16
#endif
#ifndef MXQ_BATCH_SPLIT
#define MXQ_BATCH_SPLIT 1
#endif
// ... and at most MXQ_SPLIT_LONG_WAVES per CU once the batch gives each wave
// at least MXQ_SPLIT_LONG_ROWS rows (unsmoothed fp16; see launch()).
#ifndef MXQ_SPLIT_LONG_WAVES
#define MXQ_SPLIT_LONG_WAVES 12
#endif
#ifndef MXQ_SPLIT_LONG_ROWS
#define MXQ_SPLIT_LONG_ROWS 4
#endif
// Smoothed instances (x * 1/lambda, x * lambda: two rounded bf16 terms)
// keep one row in flight per wave at 8 waves per CU (side by side against
// two rows at 12: fp16 32768 x 8192 118.6 -> 115.7 us, bf16 32768 x 4096
// 61.4 -> 60.4 us, 16384 x 8192 62.0 -> 60.6 us, 8192 x 14336 level).
#ifndef MXQ_WAVES_PER_CU_LAM
#define MXQ_WAVES_PER_CU_LAM 8
#endif
#ifndef MXQ_BATCH_LAM
#define MXQ_BATCH_LAM 1
#endif
// fp16 x times its factor in one v_fma_mix_f32; bf16 terms of a smoothed
// x' (2: each rounded to nearest, |x' - hi - lo| <= 2^-18 |x'|; 3: exact).
#ifndef MXQ_FMA_MIX
#define MXQ_FMA_MIX 1
#endif
// Short smoothed batches (each wave of the row-major plan would take at most
// eight batches of rows): the waves of a block work on one super-tile column
// and share its factors, loaded and inverted once per block and kept in LDS,
// and each wave keeps one row in flight at 16 waves per CU (the row-major
// instance fits one 8-wave block per CU).  In a launch of a round or a few
// the factor loads and each wave's serial work sit on the critical path; in
// long launches the factors are paid once per wave and the row-major wave
// order streams better.
#ifndef MXQ_SHARE_LAM
#define MXQ_SHARE_LAM 1
#endif
#ifndef MXQ_WAVES_PER_CU_SHARE
#define MXQ_WAVES_PER_CU_SHARE 16
#endif
#ifndef MXQ_BATCH_SHARE
#define MXQ_BATCH_SHARE 1
#endif
#ifndef MXQ_LAM_TERMS
#define MXQ_LAM_TERMS 2
#endif
#ifndef MXQ_NT_LOAD
#define MXQ_NT_LOAD 1
#endif
#ifndef MXQ_NT_STORE
#define MXQ_NT_STORE 1
#endif
#ifndef MXQ_NT_SCALE
#define MXQ_NT_SCALE 0
#endif
// Waves per block of the quantize kernels: the plan's waves (7 per CU on the
// headline shape) then land as one block per CU rather than as one or two
// 4-wave blocks.
#ifndef MXQ_WAVES_PER_BLOCK
#define MXQ_WAVES_PER_BLOCK 8
#endif
#ifndef MXQ_DEQUANT_WAVES_PER_CU
#define MXQ_DEQUANT_WAVES_PER_CU 16
#endif
#ifndef MXQ_DEQUANT_WAVES_PER_BLOCK
#define MXQ_DEQUANT_WAVES_PER_BLOCK 4
#endif
#ifndef MXQ_DEQUANT_UNROLL
#define MXQ_DEQUANT_UNROLL 16
#endif
// Smallest acceptable fraction of busy wave-rows in the last round; among
// row steps meeting it, the plan takes the one with the most waves.
#ifndef MXQ_PLAN_MIN_EFF
#define MXQ_PLAN_MIN_EFF 1.0
#endif

namespace mxq {

constexpr int kGroup = 32;
constexpr int kSub = 4;          // sub-tiles of 16 groups per super-tile
constexpr int kTileGroups = 64;  // groups per wave super-tile
constexpr int kWave = 64;
constexpr int kWavesPerBlock = MXQ_WAVES_PER_BLOCK;
constexpr int kBlockThreads = kWave * kWavesPerBlock;

// Does this kernel instance split the activations into several bf16 terms?
// Per-channel factor applied before the block product: none, x / lambda
// (online smoothing of activations) or x * lambda (offline absorption of the
// smoothing factors into weight rows).
enum : int { kLamNone = 0, kLamDiv = 1, kLamMul = 2 };

template <int XT, int MODE, int LAM>
constexpr bool kSplit = MODE == 1 && (XT != MXQ_BF16 || LAM != kLamNone);
template <int XT, int MODE, int LAM>
constexpr int kBatchOf = (MODE == 1 && LAM != kLamNone) ? MXQ_BATCH_LAM
                         : kSplit<XT, MODE, LAM>         ? MXQ_BATCH_SPLIT
                                                         : MXQ_BATCH;  // rows in flight per wave
// Block-shared factors: smoothed row-layout instances launched for short
// batches.
template <int LAM, bool TILED, bool SHARE>
constexpr bool kShareLamOf = SHARE && MXQ_SHARE_LAM && LAM != kLamNone && !TILED;

template <int XT, int MODE, int LAM>
constexpr int kWavesPerCuOf = (MODE == 1 && LAM != kLamNone) ? MXQ_WAVES_PER_CU_LAM
                              : kSplit<XT, MODE, LAM>         ? MXQ_WAVES_PER_CU_SPLIT
                                                              : MXQ_WAVES_PER_CU;
template <int XT, int MODE, int LAM, bool TILED, bool SHARE>
constexpr int kBatchFor = TILED ? 1 : kShareLamOf<LAM, TILED, SHARE> ? MXQ_BATCH_SHARE : kBatchOf<XT, MODE, LAM>;
template <int XT, int MODE, int LAM, bool TILED, bool SHARE>
constexpr int kWavesPerCuFor = kShareLamOf<LAM, TILED, SHARE> ? MXQ_WAVES_PER_CU_SHARE : kWavesPerCuOf<XT, MODE, LAM>;

enum : int { kBF16 = MXQ_BF16, kFP16 = MXQ_FP16, kFP32 = MXQ_FP32 };
enum : int { kQuant = 0, kRotate = 1 };

struct Args {
    const void* x;
    int64_t stride;  // elements
    const float* lambda;
    const uint16_t* r_hat;
    uint8_t* codes;
    uint8_t* scales;
    float* y;
    int32_t tokens;
    int32_t gpr;      // groups per row = channels / 32
    int32_t tcols;    // super-tile columns = ceil(gpr / 64)
    int32_t row_step; // waves per super-tile column
    int32_t waves;    // tcols * row_step
    int32_t unit;     // rows a wave takes back to back (1, or 16 for tiled output)
};

// Does a rotate instance need the tiny-group path?  fp16 activations without
// smoothing never do: a nonzero fp16 value is at least 2^-24, and the group's
// rotated maximum is then far above 2^-64.
template <int XT, int LAM>
constexpr bool kGuardTiny = !(XT == kFP16 && LAM == kLamNone);

// x' of a lane's 8 channels in fp32: x * (1/lambda), x * lambda, or x.
template <int XT, int LAM>
__device__ __forceinline__ void smoothed8(u32x4_t xq, const float* il, float* f) {
    if constexpr (XT == kFP16 && LAM != kLamNone && MXQ_FMA_MIX) {
        // fp16 x times an fp32 factor in one v_fma_mix_f32 (fp16 source
        // widened inside the instruction): the exact product rounded once
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const _Float16 h0 = __builtin_bit_cast(_Float16, static_cast<uint16_t>(xq[i] & 0xffffu));
            const _Float16 h1 = __builtin_bit_cast(_Float16, static_cast<uint16_t>(xq[i] >> 16));
            f[2 * i] = __builtin_fmaf(static_cast<float>(h0), il[2 * i], 0.0f);
            f[2 * i + 1] = __builtin_fmaf(static_cast<float>(h1), il[2 * i + 1], 0.0f);
        }
    } else {
        widen8<XT == kFP16>(xq, f);
        if constexpr (LAM != kLamNone) {
#pragma unroll
            for (int t = 0; t < 8; ++t) f[t] *= il[t];
        }
    }
}

// The rotated values y = x' R of a lane's 8 channels of one sub-tile: lane l
// ends with y[8 q .. 8 q + 7] of group j (the layout described at the top).
// xq holds the channels as loaded and il their smoothing factors.  The
// activations enter the matrix cores as exact bf16 terms of the fp32 x': 1
// for bf16 x, 2 for fp16 x, 3 for x * (1/lambda) or x * lambda.
// SHIFT: x' is formed 2^k times larger (k in [0, 64], per lane), rounded to
// fp32 once from the exact product x * factor * 2^k (exact in fp64), for the
// tiny-group path.
template <int XT, int LAM, bool SHIFT>
__device__ __forceinline__ void rotate8(u32x4_t xq, const float* il, bf16x8_t A0, bf16x8_t A1, int k, float* v) {
    f32x4_t d0 = {}, d1 = {};
    if constexpr (XT == kBF16 && LAM == kLamNone && !SHIFT) {
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xq);
        d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, b, d0, 0, 0, 0);
        d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, b, d1, 0, 0, 0);
    } else {
        float f[8];
        if constexpr (SHIFT && LAM != kLamNone) {
            widen8<XT == kFP16>(xq, f);
            const double p = __builtin_bit_cast(double, static_cast<uint64_t>(1023 + k) << 52);
#pragma unroll
            for (int t = 0; t < 8; ++t)
                f[t] = static_cast<float>(static_cast<double>(f[t]) * (static_cast<double>(il[t]) * p));
        } else if constexpr (SHIFT) {
            // bf16 x: x * 2^k is exact (the group's |x| * 2^k stays below 2^64)
            widen8<XT == kFP16>(xq, f);
            const float p = as_f32(static_cast<uint32_t>(127 + k) << 23);
#pragma unroll
            for (int t = 0; t < 8; ++t) f[t] *= p;
        } else {
            smoothed8<XT, LAM>(xq, il, f);
        }
        if constexpr (LAM != kLamNone && MXQ_LAM_TERMS == 2 && !SHIFT) {
            // two bf16 terms, each rounded to nearest: hi = bf16(x'),
            // lo = bf16(x' - hi); |x' - hi - lo| <= 2^-18 |x'|
            typedef __attribute__((ext_vector_type(2))) float f32x2_t;
            typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
            u32x4_t hi, lo;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x2_t h = __builtin_convertvector(f32x2_t{f[2 * i], f[2 * i + 1]}, bf16x2_t);
                hi[i] = __builtin_bit_cast(uint32_t, h);
                const f32x2_t r = f32x2_t{f[2 * i], f[2 * i + 1]} - __builtin_convertvector(h, f32x2_t);
                lo[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
            }
            d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, __builtin_bit_cast(bf16x8_t, hi), d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, __builtin_bit_cast(bf16x8_t, hi), d1, 0, 0, 0);
            d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, __builtin_bit_cast(bf16x8_t, lo), d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, __builtin_bit_cast(bf16x8_t, lo), d1, 0, 0, 0);
        } else {
        constexpr int kTerms = LAM != kLamNone ? 3 : (XT == kFP16 ? 2 : 1);
#pragma unroll
        for (int term = 0; term < kTerms; ++term) {
            u32x4_t bt;
#pragma unroll
            for (int i = 0; i < 4; ++i) bt[i] = bf16_pair_hi(f[2 * i], f[2 * i + 1]);
            const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bt);
            d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, b, d0, 0, 0, 0);
            d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, b, d1, 0, 0, 0);
            if (term + 1 < kTerms) {
#pragma unroll
                for (int t = 0; t < 8; ++t) f[t] = bf16_residual(f[t]);
            }
        }
        }
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        v[t] = d0[t];
        v[4 + t] = d1[t];
    }
}

// The occupancy the plan aims at is stated to the compiler, so that the
// rarely taken tiny-group pass after the main loop does not raise the
// register count above it (that pass may spill instead; the main loop does
// not).  The test-only y output instances, and the tiled ones (whose LDS
// stage allows one 8-wave block per CU), aim at 2 waves per SIMD.
// TU: rows per unit of the tiled output (1, 8 or 16; 0 for the row layout),
// a template parameter so that each unit's loop gets its own registers.
template <int XT, int MODE, int LAM, bool YOUT, bool TILED = false, bool SHARE = false, int TU = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(1, kBlockThreads),
                          amdgpu_waves_per_eu((YOUT || TILED) ? 2 : kWavesPerCuFor<XT, MODE, LAM, TILED, SHARE> / 4))) void quant_kernel(Args a) {
    constexpr int kN = (XT == kFP32) ? 2 : 1;  // 16-byte loads per lane per sub-tile
    constexpr uint32_t esz = (XT == kFP32) ? 4 : 2;
    constexpr int kBatch = kBatchFor<XT, MODE, LAM, TILED, SHARE>;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    constexpr bool kShareLam = kShareLamOf<LAM, TILED, SHARE>;
    // Wave -> (super-tile column, first row).  With shared factors a block
    // holds 4 consecutive row offsets of one column (the plan's row step is a
    // multiple of 4 and every wave of the grid exists); otherwise consecutive
    // waves take consecutive columns.
    const int w = static_cast<int>(blockIdx.x) * kWavesPerBlock + wave;
    if (!kShareLam && w >= a.waves) return;
    const int tc = kShareLam ? static_cast<int>(blockIdx.x) % a.tcols : w % a.tcols;
    const int64_t r0 = kShareLam ? static_cast<int64_t>(static_cast<int>(blockIdx.x) / a.tcols) * kWavesPerBlock + wave
                                 : static_cast<int64_t>(w / a.tcols) * (TILED ? TU : 1);
    const int64_t rs = a.row_step;
    const int64_t T = a.tokens;
    const int j = lane & 15;
    const int q = lane >> 4;
    const int p0 = tc * kTileGroups;  // first group of the super-tile
    const uint32_t gpr = static_cast<uint32_t>(a.gpr);

    // Byte offsets inside a row: the 8 channels (8q..8q+7) of group p0+16s+j
    // that this lane loads in sub-tile s, and the group p0+lane whose codes
    // and scale it stores.  Groups past the row end fall outside the row's
    // buffer range: their loads read zero and their stores are dropped.
    uint32_t xoff[kSub];
#pragma unroll
    for (int s = 0; s < kSub; ++s) xoff[s] = (static_cast<uint32_t>(p0 + 16 * s + j) * kGroup + 8 * q) * esz;
    const uint32_t row_bytes = gpr * kGroup * esz;
    const uint32_t code_off = static_cast<uint32_t>(p0 + lane) * 16;
    const uint32_t scale_off = static_cast<uint32_t>(p0 + lane);
    const char* xb = static_cast<const char*>(a.x);

    typedef u32x4_t Rows[kBatch][kSub][kN];
    // With shared factors, rows past the end load through an empty buffer
    // range (zeros, no traffic) instead of behind a branch: with a
    // conditional load the compiler's wait for the factors, issued before
    // the rows, must assume the row loads may be the later ones and waits for
    // them as well, which puts the whole first-row latency in front of the
    // block's factor setup.  (The row-major instances keep the branch: their
    // setup is per wave, and without the branch the long batches ran 2 %
    // slower, 49.0 against 48.1 us on bf16 8192 x 14336.)
    auto load_rows = [&](Rows& buf, int64_t r) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t rr = r + u * rs;
            const bool in = rr < T;
            if (kShareLam || in) {
                const auto rsrc = row_rsrc(xb + (in ? rr : 0) * a.stride * esz, in ? row_bytes : 0u);
#pragma unroll
                for (int s = 0; s < kSub; ++s)
#pragma unroll
                    for (int k = 0; k < kN; ++k)
                        buf[u][s][k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, xoff[s] + 16 * k, 0,
                                                                             MXQ_NT_LOAD ? kAuxNT : 0);
            }
        }
    };

    // Block and smoothing factors are set up while the first rows load.
    // Their loads are issued first: vector-memory loads complete in issue
    // order for the wait counter, so a wait for a factor issued after the
    // rows would also wait for the rows, and the setup (with its block
    // barrier) would not overlap them.  In a launch of one round of waves
    // that setup is on the critical path.
    constexpr int kLamSlots = kShareLam ? kTileGroups * kGroup / kBlockThreads / 4 : 1;
    u32x4_t lam_raw[kLamSlots];
    if constexpr (kShareLam) {
        const auto lrsrc = row_rsrc(a.lambda, gpr * kGroup * 4);
#pragma unroll
        for (int h = 0; h < kLamSlots; ++h) {
            const uint32_t e = kLamSlots * threadIdx.x + h;  // 16-byte slot in the column
            lam_raw[h] = __builtin_amdgcn_raw_buffer_load_b128(lrsrc, (static_cast<uint32_t>(p0) * kGroup + 4 * e) * 4,
                                                               0, 0);
        }
    }
    // Rotation block as the A operands of the two output halves, bf16 bits:
    // A_h[t] = R[8q + t][8 (j / 4) + 4 h + j % 4].
    uint16_t r_raw[2][8];
    if constexpr (MODE == kRotate) {
        const int n0 = 8 * (j >> 2) + (j & 3);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            r_raw[0][t] = a.r_hat[(8 * q + t) * kGroup + n0];
            r_raw[1][t] = a.r_hat[(8 * q + t) * kGroup + n0 + 4];
        }
    }

    Rows bufA, bufB;
    load_rows(bufA, r0);

    bf16x8_t A0, A1;
    if constexpr (MODE == kRotate) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            A0[t] = __builtin_bit_cast(__bf16, r_raw[0][t]);
            A1[t] = __builtin_bit_cast(__bf16, r_raw[1][t]);
        }
    }
    // 1 / lambda (v_rcp_f32, within 1 ulp), or lambda itself, for the 8
    // channels this lane feeds in each sub-tile.  Lanes of groups past the
    // row end get 0.
    float il[kSub][8];
    if constexpr (kShareLam) {
        // Each thread of the block inverts kPer consecutive channels of the
        // column into LDS; each lane then reads its 8 channels per sub-tile.
        // A group's 8 slots of 16 bytes are padded to 9, so the 16 groups a
        // read instruction touches start on distinct bank quads.
        constexpr int kPer = kTileGroups * kGroup / kBlockThreads;
        static_assert(kPer % 4 == 0 && kPer * kBlockThreads == kTileGroups * kGroup, "whole 16-byte loads");
        __shared__ u32x4_t lam_s[kTileGroups * 9];
#pragma unroll
        for (int h = 0; h < kPer / 4; ++h) {
            const uint32_t e = kPer / 4 * threadIdx.x + h;  // 16-byte slot in the column
            const u32x4_t l = lam_raw[h];
            // (slots of groups past the row end, which loaded zeros, hold 0)
            const bool valid = p0 + static_cast<int>(e >> 3) < a.gpr;
            u32x4_t inv;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                inv[t] = !valid ? 0u : LAM == kLamMul ? l[t] : as_u32(__builtin_amdgcn_rcpf(as_f32(l[t])));
            lam_s[e + (e >> 3)] = inv;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kSub; ++s) {
            const int idx = (16 * s + j) * 9 + 2 * q;
            const u32x4_t v0 = lam_s[idx], v1 = lam_s[idx + 1];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                il[s][t] = as_f32(v0[t]);
                il[s][4 + t] = as_f32(v1[t]);
            }
        }
    } else if constexpr (LAM != kLamNone) {
        const auto lrsrc = row_rsrc(a.lambda, gpr * kGroup * 4);
#pragma unroll
        for (int s = 0; s < kSub; ++s) {
            const uint32_t off = (static_cast<uint32_t>(p0 + 16 * s + j) * kGroup + 8 * q) * 4;
            const u32x4_t l0 = __builtin_amdgcn_raw_buffer_load_b128(lrsrc, off, 0, 0);
            const u32x4_t l1 = __builtin_amdgcn_raw_buffer_load_b128(lrsrc, off + 16, 0, 0);
            const bool valid = p0 + 16 * s + j < a.gpr;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float f0 = LAM == kLamMul ? as_f32(l0[t]) : __builtin_amdgcn_rcpf(as_f32(l0[t]));
                const float f1 = LAM == kLamMul ? as_f32(l1[t]) : __builtin_amdgcn_rcpf(as_f32(l1[t]));
                il[s][t] = valid ? f0 : 0.0f;
                il[s][4 + t] = valid ? f1 : 0.0f;
            }
        }
    }

    // y output of a sub-tile (test use): v holds y * 2^ksh.
    auto store_y = [&](int64_t rr, int s, const float (&v)[8], int ksh) {
        const float down = pow2_neg(ksh);
        const auto yrsrc = row_rsrc(a.y + rr * a.gpr * kGroup, gpr * kGroup * 4);
        const uint32_t off = (static_cast<uint32_t>(p0 + 16 * s + j) * kGroup + 8 * q) * 4;
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4_t{as_u32(v[0] * down), as_u32(v[1] * down), as_u32(v[2] * down), as_u32(v[3] * down)}, yrsrc, off,
            0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(
            u32x4_t{as_u32(v[4] * down), as_u32(v[5] * down), as_u32(v[6] * down), as_u32(v[7] * down)}, yrsrc,
            off + 16, 0, 0);
    };
    // Codes and scales of row rr (held in buf[u]): after the transpose lane l
    // holds the 16 code bytes of group p0 + l, and S is that group's scale.
    // A group whose rotated maximum is below 2^-64 (S < 61) only sets
    // tiny_seen here; such rows are redone after the main loop (below), so
    // the common path carries one compare per row and no extra registers.
    bool tiny_seen = false;
    constexpr bool kFlagTiny = MODE == kRotate && kGuardTiny<XT, LAM>;
    auto encode_row = [&](const Rows& buf, int u, int64_t rr, uint32_t (&word)[kSub], uint32_t& S) {
            uint32_t sc[kSub];
#pragma unroll
            for (int s = 0; s < kSub; ++s) {
                float v[8];
                if constexpr (MODE == kRotate) {
                    rotate8<XT, LAM, false>(buf[u][s][0], il[s], A0, A1, 0, v);
                } else if constexpr (XT == kFP32) {
                    widen4_f32(buf[u][s][0], v);
                    widen4_f32(buf[u][s][1], v + 4);
                } else {
                    widen8<XT == kFP16>(buf[u][s][0], v);
                }
                const uint32_t scale_bits = e8m0_scale_bits(group_amax8(v));
                sc[s] = scale_bits >> 23;
                word[s] = encode8(v, as_f32(scale_bits));
                if constexpr (YOUT) store_y(rr, s, v, 0);
            }
            transpose_words(word);
            // the scale of group 16 q + j is the one computed in sub-tile q
            S = q == 0 ? sc[0] : q == 1 ? sc[1] : q == 2 ? sc[2] : sc[3];
            // Groups past the row end (zeros whose stores are dropped) do not
            // count, nor do groups of zeros: their rotated maximum is 0 like
            // that of a tiny group, but their codes and scale are exact
            // already.  Telling zeros from tiny values takes the input, so it
            // is looked at only in a row where some group fell below the bound.
            if constexpr (kFlagTiny) {
                bool t = S < (kTinyScaleBits >> 23) && static_cast<uint32_t>(p0 + lane) < gpr;
                if (any_lane(t)) {
                    // bit j of nzm[s]: group 16 s + j holds a nonzero input bit pattern
                    uint32_t nzm[kSub];
#pragma unroll
                    for (int s = 0; s < kSub; ++s) {
                        const u32x4_t& w = buf[u][s][0];
                        const uint64_t b = __builtin_amdgcn_ballot_w64((w[0] | w[1] | w[2] | w[3]) != 0u);
                        const uint64_t f = b | (b >> 32);
                        nzm[s] = static_cast<uint32_t>(f | (f >> 16)) & 0xffffu;
                    }
                    const uint32_t nz = q == 0 ? nzm[0] : q == 1 ? nzm[1] : q == 2 ? nzm[2] : nzm[3];
                    tiny_seen |= t && ((nz >> j) & 1u);
                }
            }
    };
    auto store_row = [&](int64_t rr, const uint32_t (&word)[kSub], uint32_t S) {
            if constexpr (TILED) {
                // Fragment-tiled output: group g of row rr is slot
                // 16 (g % 4) + rr % 16 of record (rr / 16, g / 4); a record
                // row holds gpr / 4 records (1 KB of codes, 64 scale bytes
                // each).  Groups past the row end land past the record row's
                // range and are dropped.
                const uint32_t nrec = gpr / 4;
                const int64_t rrow = rr >> 4;
                const uint32_t grp = static_cast<uint32_t>(p0 + lane);
                const uint32_t slot = (grp >> 2) * 64 + (grp & 3) * 16 + static_cast<uint32_t>(rr & 15);
                const auto crsrc = row_rsrc(a.codes + rrow * nrec * 1024, nrec * 1024);
                __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{word[0], word[1], word[2], word[3]}, crsrc,
                                                       slot * 16, 0, 0);
                const auto srsrc = row_rsrc(a.scales + rrow * nrec * 64, nrec * 64);
                __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(S), srsrc, slot, 0, 0);
            } else {
                const auto crsrc = row_rsrc(a.codes + rr * a.gpr * 16, gpr * 16);
                __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{word[0], word[1], word[2], word[3]}, crsrc,
                                                       code_off, 0, MXQ_NT_STORE ? kAuxNT : 0);
                const auto srsrc = row_rsrc(a.scales + rr * a.gpr, gpr);
                __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(S), srsrc, scale_off, 0,
                                                     MXQ_NT_SCALE ? kAuxNT : 0);
            }
    };
    auto process_rows = [&](const Rows& buf, int64_t r) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t rr = r + u * rs;
            if (rr >= T) break;
            uint32_t word[kSub];
            uint32_t S;
            encode_row(buf, u, rr, word, S);
            store_row(rr, word, S);
        }
    };

    // Two row buffers alternate: the next batch is in flight while the
    // current one is computed.
    if constexpr (TILED) {
        static_assert(kBatch == 1, "one row per step");
        // Units of U consecutive rows (U = 16: one record row; U = 8: half of
        // one), units r0 / U + k * rs.  The unit's codes go to a per-wave LDS
        // tile ([row][group], padded) and leave it record by record.  U = 16:
        // lane l carries slot l (row l % 16, group 4 rec + l / 16), so each
        // store instruction writes one whole 1 KB record.  U = 8: lane l
        // carries row l % 8 of group (l / 8) % 4 of record 2 m + l / 32, so
        // every 8 lanes write one 128-byte line (rows 8 h .. + 7 of a 256-byte
        // group chunk).  Scattered 16-byte stores (one line per lane) cost
        // half the bandwidth; records written as two 8-row halves at
        // different times cost 5 % when 16-row units fill the grid, but give
        // twice the units when they do not.  The U scale bytes of a lane's
        // group are contiguous in its record and go out as one store per
        // unit.  Both stores are non-temporal (written once, read by the
        // next kernel).  The tile's row pitch is 65 slots of 16 bytes: the 16
        // lanes of a ds_read_b128 pass read 16 rows of one group (U = 16),
        // which an odd pitch spreads over all 16 bank quads.
        __shared__ u32x4_t stg[kWavesPerBlock][16][kTileGroups + 1];
        const uint32_t nrec = gpr / 4;
        const uint32_t rec0 = static_cast<uint32_t>(p0) / 4;
        const uint32_t grp = static_cast<uint32_t>(p0 + lane);
        const uint32_t soff = (grp >> 2) * 64 + (grp & 3) * 16;
        auto run_units = [&](auto u_tag) {
            constexpr int U = decltype(u_tag)::value;
            for (int64_t unit = r0; unit < T; unit += U * rs) {
                uint32_t spk[4] = {0u, 0u, 0u, 0u};
                const auto crsrc = row_rsrc(a.codes + (unit >> 4) * nrec * 1024, nrec * 1024);
#pragma unroll
                for (int k = 0; k < U; ++k) {
                    const int64_t r = unit + k;
                    if (r < T) {
                        const int64_t rn = k < U - 1 ? r + 1 : unit + U * rs;
                        Rows& cur = (k & 1) ? bufB : bufA;
                        Rows& nxt = (k & 1) ? bufA : bufB;
                        if (rn < T) load_rows(nxt, rn);
                        uint32_t word[kSub];
                        uint32_t S;
                        encode_row(cur, 0, r, word, S);
                        stg[wave][k][lane] = u32x4_t{word[0], word[1], word[2], word[3]};
                        spk[k / 4] |= S << (8 * (k % 4));
                    }
                }
                const auto srsrc = row_rsrc(a.scales + (unit >> 4) * nrec * 64, nrec * 64);
                if constexpr (U == 16) {
                    // rows past the end (the last unit's padding) are not written
                    const int st_row = lane & 15;
                    const int st_grp = lane >> 4;
                    const bool row_ok = unit + st_row < T;
#pragma unroll
                    for (int rec = 0; rec < 16; ++rec) {
                        const u32x4_t v = stg[wave][st_row][4 * rec + st_grp];
                        if (row_ok)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                v, crsrc, (rec0 + static_cast<uint32_t>(rec)) * 1024 + 16 * static_cast<uint32_t>(lane),
                                0, kAuxNT);
                    }
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{spk[0], spk[1], spk[2], spk[3]}, srsrc, soff, 0,
                                                           kAuxNT);
                } else {
                    const uint32_t h = static_cast<uint32_t>(unit >> 3) & 1;  // which half of the record row
                    const int st_row = lane & 7;
                    const int st_grp = (lane >> 3) & 3;
                    const int st_rec = lane >> 5;
                    const bool row_ok = unit + st_row < T;
#pragma unroll
                    for (int m = 0; m < 8; ++m) {
                        const int rec = 2 * m + st_rec;
                        const u32x4_t v = stg[wave][st_row][4 * rec + st_grp];
                        if (row_ok)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                v, crsrc,
                                (rec0 + static_cast<uint32_t>(rec)) * 1024 + static_cast<uint32_t>(st_grp) * 256 +
                                    (8 * h + static_cast<uint32_t>(st_row)) * 16,
                                0, kAuxNT);
                    }
                    __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{spk[0], spk[1]}, srsrc, soff + 8 * h, 0, kAuxNT);
                }
            }
        };
        static_assert(!TILED || TU == 1 || TU == 8 || TU == 16, "tiled units of 1, 8 or 16 rows");
        if constexpr (TU == 16) {
            run_units(std::integral_constant<int, 16>{});
        } else if constexpr (TU == 8) {
            run_units(std::integral_constant<int, 8>{});
        } else {
            for (int64_t r = r0; r < T; r += 2 * rs) {
                if (r + rs < T) load_rows(bufB, r + rs);
                process_rows(bufA, r);
                if (r + rs >= T) break;
                if (r + 2 * rs < T) load_rows(bufA, r + 2 * rs);
                process_rows(bufB, r + rs);
            }
        }
    } else {
        const int64_t step = kBatch * rs;
        for (int64_t r = r0; r < T; r += 2 * step) {
            if (r + step < T) load_rows(bufB, r + step);
            process_rows(bufA, r);
            if (r + step >= T) break;
            if (r + 2 * step < T) load_rows(bufA, r + 2 * step);
            process_rows(bufB, r + step);
        }
    }

    // ---- rows holding a tiny group (rare): redone from x' * 2^k ----------
    // Every row of this wave is reloaded and re-encoded; in a row with a
    // group whose rotated maximum is below 2^-64, the sub-tiles holding such
    // groups are recomputed with x' shifted by 2^k (k per group, from its
    // largest |x'|), and the row's codes and scales are written again (the
    // other groups' bytes are rewritten unchanged).  The wave first waits for
    // its own first stores of these rows, so the second ones land after them
    // (the rows are the wave's own; an agent-scope release fence would also
    // write back the L2).
    if constexpr (MODE == kRotate && kGuardTiny<XT, LAM>) {
        if (any_lane(tiny_seen)) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            auto fix_row = [&](int64_t rr) {
                const auto rsrc = row_rsrc(xb + rr * a.stride * esz, row_bytes);
                uint32_t word[kSub], sc[kSub];
                bool redo = false;
                // one sub-tile at a time (scheduling barriers between them):
                // this path must not need more registers than the main loop
#pragma unroll
                for (int s = 0; s < kSub; ++s) {
                    __builtin_amdgcn_sched_barrier(0);
                    u32x4_t xr_s = __builtin_amdgcn_raw_buffer_load_b128(rsrc, xoff[s], 0, 0);
                    // an opaque copy of the factors: their fp64 forms are not
                    // hoisted out of this loop into registers of the main one
                    float ilc[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        ilc[t] = il[s][t];
                        if constexpr (LAM != kLamNone) asm volatile("" : "+v"(ilc[t]));
                    }
                    float v[8];
                    rotate8<XT, LAM, false>(xr_s, ilc, A0, A1, 0, v);
                    uint32_t sb = e8m0_scale_bits(group_amax8(v)), cb = sb;
                    const bool tiny = sb < kTinyScaleBits;
                    if (any_lane(tiny)) {
                        redo = true;
                        float xp[8];
                        smoothed8<XT, LAM>(xr_s, ilc, xp);
                        const int k = tiny ? tiny_shift(group_amax8(xp)) : 0;
                        float w[8];
                        rotate8<XT, LAM, true>(xr_s, ilc, A0, A1, k, w);
                        uint32_t sb2, cb2;
                        shifted_scale_bits(group_amax8(w), k, sb2, cb2);
#pragma unroll
                        for (int t = 0; t < 8; ++t) v[t] = tiny ? w[t] : v[t];
                        sb = tiny ? sb2 : sb;
                        cb = tiny ? cb2 : cb;
                        if constexpr (YOUT) store_y(rr, s, v, tiny ? k : 0);
                    }
                    sc[s] = sb >> 23;
                    word[s] = encode8(v, as_f32(cb));
                }
                if (redo) {
                    transpose_words(word);
                    const uint32_t S = q == 0 ? sc[0] : q == 1 ? sc[1] : q == 2 ? sc[2] : sc[3];
                    store_row(rr, word, S);
                }
            };
            if constexpr (TILED && TU > 1) {
                for (int64_t unit = r0; unit < T; unit += TU * rs)
                    for (int64_t rr = unit; rr < unit + TU && rr < T; ++rr) fix_row(rr);
            } else {
                for (int64_t rr = r0; rr < T; rr += rs) fix_row(rr);
            }
        }
    }
}

// Decode.  A lane turns 8 (bf16 output) or 4 (fp32 output) consecutive codes
// into one 16-byte store, so each wave store instruction writes 1 KB
// contiguously.  v_cvt_scalef32_pk_bf16_fp4 decodes the two codes of one
// byte and multiplies by 2^(S-127) taken from the exponent field of its scale
// operand; on every code byte and every scale byte it gives exactly the
// E2M1 value times 2^(S-127) (subnormal results kept, +-inf beyond the
// range, NaN for S = 0xFF, -0 for code 0x8).  Every finite result is exact
// in bf16, so fp32 output is the bf16 result widened.  (The fp32-output form
// of the converter is not used: this compiler folds its second result into
// the first.)
constexpr int kDequantWaves = MXQ_DEQUANT_WAVES_PER_BLOCK;

template <bool OUT_BF16>
__global__ __launch_bounds__(kWave * kDequantWaves) void dequant_kernel(const uint8_t* codes, const uint8_t* scales,
                                                                       void* y, int64_t elems) {
    constexpr int kPerLane = OUT_BF16 ? 8 : 4;
    constexpr int64_t kChunk = kWave * kPerLane;              // elements per wave store
    constexpr int kUnroll = MXQ_DEQUANT_UNROLL;               // chunks per wave iteration
    constexpr uint32_t osz = OUT_BF16 ? 2 : 4;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = static_cast<int64_t>(blockIdx.x) * kDequantWaves +
                         __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int64_t waves = static_cast<int64_t>(gridDim.x) * kDequantWaves;
    const uint32_t first = static_cast<uint32_t>(lane * kPerLane);  // lane's first element in a chunk
    for (int64_t base = wave * kUnroll * kChunk; base < elems; base += waves * kUnroll * kChunk) {
        const int64_t rem = elems - base;
        // n elements (a multiple of 32) from here on belong to this iteration
        const uint32_t n = static_cast<uint32_t>(rem < kUnroll * kChunk ? rem : kUnroll * kChunk);
        const auto crsrc = row_rsrc(codes + base / 2, n / 2);
        const auto srsrc = row_rsrc(scales + base / kGroup, n / kGroup);
        const auto yrsrc = row_rsrc(static_cast<char*>(y) + base * osz, n * osz);
        uint32_t c[kUnroll], S[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t e = static_cast<uint32_t>(u * kChunk) + first;
            S[u] = __builtin_amdgcn_raw_buffer_load_b8(srsrc, e / kGroup, 0, 0);
            if constexpr (OUT_BF16)
                c[u] = __builtin_amdgcn_raw_buffer_load_b32(crsrc, e / 2, 0, kAuxNT);
            else
                c[u] = __builtin_amdgcn_raw_buffer_load_b16(crsrc, e / 2, 0, kAuxNT);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const float scale = as_f32(S[u] << 23);
            u32x4_t out;
            if constexpr (OUT_BF16) {
                out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[u], scale, 0));
                out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[u], scale, 1));
                out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[u], scale, 2));
                out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[u], scale, 3));
            } else {
                const uint32_t p0 =
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[u], scale, 0));
                const uint32_t p1 =
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[u], scale, 1));
                out = u32x4_t{p0 << 16, p0 & 0xffff0000u, p1 << 16, p1 & 0xffff0000u};
            }
            __builtin_amdgcn_raw_buffer_store_b128(out, yrsrc, (static_cast<uint32_t>(u * kChunk) + first) * osz, 0,
                                                   kAuxNT);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.

struct Plan {
    int32_t blocks, waves, tcols, row_step;
};

constexpr int64_t kMaxI32 = 2147483647;
// Row byte counts (up to 4 bytes per channel) must fit a buffer resource's
// 32-bit record count.
constexpr int64_t kMaxChannels = int64_t(1) << 28;

// Grid for tokens x channels on cu_count CUs with at most waves_per_cu
// resident waves per CU (the kernel's occupancy bound, so the persistent grid
// runs in a single round).  Waves share a super-tile column in groups of
// row_step; among row steps between half and all of the target, pick the one
// whose last round of rows leaves the fewest waves idle.
static bool make_plan(int64_t tokens, int64_t channels, int cu_count, int waves_per_cu, Plan* out) {
    if (tokens <= 0 || channels <= 0 || channels % kGroup) return false;
    if (tokens > kMaxI32 || channels > kMaxChannels) return false;
    const int64_t gpr = channels / kGroup;
    const int64_t tcols = (gpr + kTileGroups - 1) / kTileGroups;
    if (tokens * tcols > kMaxI32) return false;
    const int64_t target = static_cast<int64_t>(cu_count > 0 ? cu_count : 1) * (waves_per_cu > 0 ? waves_per_cu : 1);
    int64_t rs_max = target / tcols;
    if (rs_max < 1) rs_max = 1;
    if (rs_max > tokens) rs_max = tokens;
    const int64_t q_min = (tokens + rs_max - 1) / rs_max;  // rounds of rows per wave
    int64_t best_rs = rs_max;
    double best_eff = -1.0;
    for (int64_t q = q_min; q <= 2 * q_min; ++q) {
        const int64_t rs = (tokens + q - 1) / q;
        if (rs < 1) break;
        const double eff = static_cast<double>(tokens) / static_cast<double>(q * rs);
        if (eff >= MXQ_PLAN_MIN_EFF - 1e-12) {  // first hit has the most waves
            best_rs = rs;
            break;
        }
        if (eff > best_eff + 1e-12) {
            best_eff = eff;
            best_rs = rs;
        }
    }
    const int64_t waves = tcols * best_rs;
    if (waves > kMaxI32 - kWavesPerBlock) return false;
    out->tcols = static_cast<int32_t>(tcols);
    out->row_step = static_cast<int32_t>(best_rs);
    out->waves = static_cast<int32_t>(waves);
    out->blocks = static_cast<int32_t>((waves + kWavesPerBlock - 1) / kWavesPerBlock);
    return true;
}

// Rows per unit of the tiled output (16, 8 or 1), from a cost model fitted
// to timings of each unit forced on smoothed bf16 batches of 256 to 12000
// rows x 4096, 8192 and 14336 channels: a wave's rows, ceil(units / (slots
// / columns)) rounds of U rows, times a per-row cost of 1.5 for single rows
// (each lane's 16-byte store lands in its own record), 1 for 8-row units and
// 0.95 for 16-row units.  On those 27 shapes the cheapest unit was the
// fastest or within 7 % of it.
static int tiled_unit(int64_t tokens, int64_t channels, int64_t slots) {
    const int64_t tcols = (channels / kGroup + kTileGroups - 1) / kTileGroups;
    int64_t per_col = slots / (tcols > 0 ? tcols : 1);
    if (per_col < 1) per_col = 1;
    static const int kUnits[3] = {16, 8, 1};
    static const int kCost20[3] = {19, 20, 30};  // per-row cost x 20
    int best = 1;
    int64_t best_cost = -1;
    for (int i = 0; i < 3; ++i) {
        const int64_t units = (tokens + kUnits[i] - 1) / kUnits[i];
        const int64_t rounds = (units + per_col - 1) / per_col;
        const int64_t cost = rounds * kUnits[i] * kCost20[i];
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = kUnits[i];
        }
    }
    return best;
}

// Shapes the launch plan accepts (no device query).
static bool shape_ok(int64_t tokens, int64_t channels) {
    Plan pl;
    return make_plan(tokens, channels, 1, 1, &pl);
}

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
    cache[dev].store(cu, std::memory_order_relaxed);
    return cu;
}

static bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

static size_t dtype_size(int32_t dt) { return dt == MXQ_FP32 ? 4 : 2; }

// Resident waves per CU the kernel instance allows (registers), queried once.
template <int XT, int MODE, int LAM, bool YOUT, bool TILED, bool SHARE = false>
static int occupancy_waves_per_cu() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int blocks = 0;
    // (the tiled instances share one LDS size and register target)
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, quant_kernel<XT, MODE, LAM, YOUT, TILED, SHARE, TILED ? 16 : 0>,
                                                     kBlockThreads, 0) != hipSuccess ||
        blocks <= 0)
        blocks = 1;
    v = blocks * kWavesPerBlock;
    cached.store(v, std::memory_order_relaxed);
    return v;
}

template <int XT, int MODE, int LAM, bool YOUT, bool TILED = false>
static mxq_status launch(Args a, int64_t tokens, int64_t channels, hipStream_t st) {
    const int occ = occupancy_waves_per_cu<XT, MODE, LAM, YOUT, TILED>();
    Plan pl;
    constexpr int want = kWavesPerCuOf<XT, MODE, LAM>;
    int per_cu = occ < want ? occ : want;
    const int cus = device_cu_count();
    // fp16 without smoothing (two exact bf16 terms): 16 waves per CU suit
    // batches of a round or two, but long batches stream better with fewer,
    // longer-lived waves (fp16 32768 x 8192: 123.5 -> 112.9 us at 12 waves
    // per CU; 8192 x 14336: 55.1 -> 52.6 us; 2048 x 4096 stays at 16: 6.2
    // against 6.7 us).
    if constexpr (kSplit<XT, MODE, LAM> && LAM == kLamNone && !TILED) {
        const int64_t units = tokens * ((channels / kGroup + kTileGroups - 1) / kTileGroups);
        if (per_cu > MXQ_SPLIT_LONG_WAVES &&
            units >= static_cast<int64_t>(cus) * MXQ_SPLIT_LONG_WAVES * MXQ_SPLIT_LONG_ROWS)
            per_cu = MXQ_SPLIT_LONG_WAVES;
    }
    a.unit = 1;
    if (TILED) a.unit = tiled_unit(tokens, channels, static_cast<int64_t>(cus) * per_cu);
    if (!make_plan((tokens + a.unit - 1) / a.unit, channels, cus, per_cu, &pl)) return MXQ_ERR_SHAPE;
    a.tcols = pl.tcols;
    if constexpr (kShareLamOf<LAM, TILED, true>) {
        // A short batch (at most 192 rows per CU and super-tile column:
        // 16 rows per wave at 12 waves per CU) takes the block-shared-factor
        // instance, planned at its own occupancy.  Whole blocks per column:
        // the row step rounds up to a multiple of the block's waves (waves
        // whose first row is past the end do nothing but share the block's
        // factor load).
        if ((tokens + pl.row_step - 1) / pl.row_step * per_cu <= 192) {
            const int occ_s = occupancy_waves_per_cu<XT, MODE, LAM, YOUT, TILED, true>();
            constexpr int want_s = kWavesPerCuFor<XT, MODE, LAM, TILED, true>;
            Plan ps;
            if (!make_plan(tokens, channels, cus, occ_s < want_s ? occ_s : want_s, &ps)) return MXQ_ERR_SHAPE;
            const int64_t rs =
                (static_cast<int64_t>(ps.row_step) + kWavesPerBlock - 1) / kWavesPerBlock * kWavesPerBlock;
            if (rs * ps.tcols > kMaxI32) return MXQ_ERR_SHAPE;
            a.row_step = static_cast<int32_t>(rs);
            a.waves = static_cast<int32_t>(rs * ps.tcols);
            hipLaunchKernelGGL((quant_kernel<XT, MODE, LAM, YOUT, TILED, true>), dim3(a.waves / kWavesPerBlock),
                               dim3(kBlockThreads), 0, st, a);
            return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
        }
    }
    a.row_step = pl.row_step;
    a.waves = pl.waves;
    if constexpr (TILED) {
        if (a.unit == 16)
            hipLaunchKernelGGL((quant_kernel<XT, MODE, LAM, YOUT, TILED, false, 16>), dim3(pl.blocks), dim3(kBlockThreads),
                               0, st, a);
        else if (a.unit == 8)
            hipLaunchKernelGGL((quant_kernel<XT, MODE, LAM, YOUT, TILED, false, 8>), dim3(pl.blocks), dim3(kBlockThreads),
                               0, st, a);
        else
            hipLaunchKernelGGL((quant_kernel<XT, MODE, LAM, YOUT, TILED, false, 1>), dim3(pl.blocks), dim3(kBlockThreads),
                               0, st, a);
    } else {
        hipLaunchKernelGGL((quant_kernel<XT, MODE, LAM, YOUT, TILED>), dim3(pl.blocks), dim3(kBlockThreads), 0, st, a);
    }
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

template <int XT>
static mxq_status dispatch_rotate(const Args& a, int64_t tokens, int64_t channels, hipStream_t st, bool tiled) {
    if (tiled) {
        return a.lambda ? launch<XT, kRotate, kLamDiv, false, true>(a, tokens, channels, st)
                        : launch<XT, kRotate, kLamNone, false, true>(a, tokens, channels, st);
    }
    if (a.lambda) {
        return a.y ? launch<XT, kRotate, kLamDiv, true>(a, tokens, channels, st)
                   : launch<XT, kRotate, kLamDiv, false>(a, tokens, channels, st);
    }
    return a.y ? launch<XT, kRotate, kLamNone, true>(a, tokens, channels, st)
               : launch<XT, kRotate, kLamNone, false>(a, tokens, channels, st);
}

static mxq_status check_common(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                               int64_t stride, bool allow_fp32) {
    if (x_dtype != MXQ_BF16 && x_dtype != MXQ_FP16 && !(allow_fp32 && x_dtype == MXQ_FP32)) return MXQ_ERR_DTYPE;
    if (tokens < 0 || channels < 0 || channels % kGroup) return MXQ_ERR_SHAPE;
    (void)x;
    (void)stride;
    return MXQ_OK;
}

mxq_status rotate_impl(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels, int64_t stride,
                       const float* lambda, const uint16_t* r_hat, uint8_t* codes, uint8_t* scales, float* y,
                       void* stream, bool tiled) {
    mxq_status s = check_common(x, x_dtype, tokens, channels, stride, false);
    if (s != MXQ_OK) return s;
    if (tiled && channels % 128) return MXQ_ERR_SHAPE;
    if (tiled && scales && (reinterpret_cast<uintptr_t>(scales) % 16)) return MXQ_ERR_ALIGN;
    if (tokens == 0 || channels == 0) return MXQ_OK;
    if (!x || !r_hat || !codes || !scales) return MXQ_ERR_NULL;
    if (stride < channels) return MXQ_ERR_STRIDE;
    if (!aligned(x, 16) || (stride * 2) % 16 || !aligned(codes, 16) || !aligned(r_hat, 2) ||
        (lambda && !aligned(lambda, 16)) || (y && !aligned(y, 16)))
        return MXQ_ERR_ALIGN;
    if (!shape_ok(tokens, channels)) return MXQ_ERR_SHAPE;
    Args a{x, stride, lambda, r_hat, codes, scales, y, static_cast<int32_t>(tokens),
           static_cast<int32_t>(channels / kGroup), 0, 0, 0};
    hipStream_t st = static_cast<hipStream_t>(stream);
    return x_dtype == MXQ_BF16 ? dispatch_rotate<kBF16>(a, tokens, channels, st, tiled)
                               : dispatch_rotate<kFP16>(a, tokens, channels, st, tiled);
}

static mxq_status absorb_impl(const void* w, int32_t w_dtype, int64_t rows, int64_t cols, int64_t stride,
                              const float* lambda, const uint16_t* r_hat, uint8_t* codes, uint8_t* scales,
                              void* stream) {
    mxq_status s = check_common(w, w_dtype, rows, cols, stride, false);
    if (s != MXQ_OK) return s;
    if (rows == 0 || cols == 0) return MXQ_OK;
    if (!w || !r_hat || !codes || !scales) return MXQ_ERR_NULL;
    if (stride < cols) return MXQ_ERR_STRIDE;
    if (!aligned(w, 16) || (stride * 2) % 16 || !aligned(codes, 16) || !aligned(r_hat, 2) ||
        (lambda && !aligned(lambda, 16)))
        return MXQ_ERR_ALIGN;
    if (!shape_ok(rows, cols)) return MXQ_ERR_SHAPE;
    Args a{w, stride, lambda, r_hat, codes, scales, nullptr, static_cast<int32_t>(rows),
           static_cast<int32_t>(cols / kGroup), 0, 0, 0};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (w_dtype == MXQ_BF16)
        return lambda ? launch<kBF16, kRotate, kLamMul, false>(a, rows, cols, st)
                      : launch<kBF16, kRotate, kLamNone, false>(a, rows, cols, st);
    return lambda ? launch<kFP16, kRotate, kLamMul, false>(a, rows, cols, st)
                  : launch<kFP16, kRotate, kLamNone, false>(a, rows, cols, st);
}

}  // namespace mxq

using namespace mxq;

extern "C" {

mxq_status mxq_rotate_quant(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                            int64_t x_row_stride, const float* lambda, const uint16_t* r_hat,
                            uint8_t* codes, uint8_t* scales, void* stream) {
    return rotate_impl(x, x_dtype, tokens, channels, x_row_stride, lambda, r_hat, codes, scales, nullptr,
                       stream, false);
}

mxq_status mxq_rotate_quant_tiled(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                  int64_t x_row_stride, const float* lambda, const uint16_t* r_hat,
                                  uint8_t* tiled_codes, uint8_t* tiled_scales, void* stream) {
    return rotate_impl(x, x_dtype, tokens, channels, x_row_stride, lambda, r_hat, tiled_codes, tiled_scales,
                       nullptr, stream, true);
}

mxq_status mxq_rotate_quant_ex(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                               int64_t x_row_stride, const float* lambda, const uint16_t* r_hat,
                               uint8_t* codes, uint8_t* scales, float* y_rot, void* stream) {
    return rotate_impl(x, x_dtype, tokens, channels, x_row_stride, lambda, r_hat, codes, scales, y_rot,
                       stream, false);
}

mxq_status mxq_absorb_quant(const void* w, int32_t w_dtype, int64_t rows, int64_t cols, int64_t w_row_stride,
                            const float* lambda, const uint16_t* r_hat, uint8_t* codes, uint8_t* scales,
                            void* stream) {
    return absorb_impl(w, w_dtype, rows, cols, w_row_stride, lambda, r_hat, codes, scales, stream);
}

mxq_status mxq_quant(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels, int64_t x_row_stride,
                     uint8_t* codes, uint8_t* scales, void* stream) {
    mxq_status s = check_common(x, x_dtype, tokens, channels, x_row_stride, true);
    if (s != MXQ_OK) return s;
    if (tokens == 0 || channels == 0) return MXQ_OK;
    if (!x || !codes || !scales) return MXQ_ERR_NULL;
    if (x_row_stride < channels) return MXQ_ERR_STRIDE;
    if (!aligned(x, 16) || (x_row_stride * static_cast<int64_t>(dtype_size(x_dtype))) % 16 || !aligned(codes, 16))
        return MXQ_ERR_ALIGN;
    if (!shape_ok(tokens, channels)) return MXQ_ERR_SHAPE;
    Args a{x, x_row_stride, nullptr, nullptr, codes, scales, nullptr, static_cast<int32_t>(tokens),
           static_cast<int32_t>(channels / kGroup), 0, 0, 0};
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (x_dtype) {
        case MXQ_BF16: return launch<kBF16, kQuant, kLamNone, false>(a, tokens, channels, st);
        case MXQ_FP16: return launch<kFP16, kQuant, kLamNone, false>(a, tokens, channels, st);
        default: return launch<kFP32, kQuant, kLamNone, false>(a, tokens, channels, st);
    }
}

mxq_status mxq_dequant(const uint8_t* codes, const uint8_t* scales, int64_t tokens, int64_t channels, void* y,
                       int32_t y_dtype, void* stream) {
    if (y_dtype != MXQ_BF16 && y_dtype != MXQ_FP32) return MXQ_ERR_DTYPE;
    if (tokens < 0 || channels < 0 || channels % kGroup) return MXQ_ERR_SHAPE;
    if (tokens == 0 || channels == 0) return MXQ_OK;
    if (tokens > kMaxI32 || channels > kMaxChannels) return MXQ_ERR_SHAPE;
    if (!codes || !scales || !y) return MXQ_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(y, 16)) return MXQ_ERR_ALIGN;
    const int64_t elems = tokens * channels;
    const int64_t per_wave = (y_dtype == MXQ_BF16 ? 8 : 4) * kWave * MXQ_DEQUANT_UNROLL;
    const int64_t chunks = (elems + per_wave - 1) / per_wave;
    int64_t blocks = (chunks + kDequantWaves - 1) / kDequantWaves;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * (MXQ_DEQUANT_WAVES_PER_CU / kDequantWaves);
    if (blocks > cap) blocks = cap;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (y_dtype == MXQ_BF16)
        hipLaunchKernelGGL((dequant_kernel<true>), dim3(static_cast<unsigned>(blocks)), dim3(kWave * kDequantWaves), 0,
                           st, codes, scales, y, elems);
    else
        hipLaunchKernelGGL((dequant_kernel<false>), dim3(static_cast<unsigned>(blocks)), dim3(kWave * kDequantWaves), 0,
                           st, codes, scales, y, elems);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

const char* mxq_status_str(int32_t status) {
    switch (status) {
        case MXQ_OK: return "MXQ_OK";
        case MXQ_ERR_NULL: return "MXQ_ERR_NULL: a required pointer is NULL";
        case MXQ_ERR_SHAPE: return "MXQ_ERR_SHAPE: bad or unsupported tokens/channels";
        case MXQ_ERR_DTYPE: return "MXQ_ERR_DTYPE: unsupported dtype for this entry point";
        case MXQ_ERR_ALIGN: return "MXQ_ERR_ALIGN: pointer or row pitch not 16-byte aligned";
        case MXQ_ERR_STRIDE: return "MXQ_ERR_STRIDE: row stride smaller than channels";
        case MXQ_ERR_HIP: return "MXQ_ERR_HIP: HIP launch error";
        default: return "unknown mxq status";
    }
}

mxq_status mxq_plan(int64_t tokens, int64_t channels, int32_t cu_count, int32_t* out) {
    if (!out) return MXQ_ERR_NULL;
    Plan pl;
    if (!make_plan(tokens, channels, cu_count, MXQ_WAVES_PER_CU, &pl)) return MXQ_ERR_SHAPE;
    out[0] = pl.blocks;
    out[1] = pl.waves;
    out[2] = pl.tcols;
    out[3] = pl.row_step;
    out[4] = kWavesPerBlock;
    return MXQ_OK;
}

int32_t mxq_version(void) { return 1; }

}  // extern "C"
