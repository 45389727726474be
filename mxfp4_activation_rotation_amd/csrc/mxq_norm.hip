// Norm + smooth + rotate + MXFP4 in one pass over HBM.
//
// The DuQuant++ page (sec. 5.2 item 1) notes that the per-channel 1/lambda
// of the online transform folds into the output of the LayerNorm in front of
// the linear layer, and asks for the online operations to run as one kernel.
// This kernel takes the norm's input h (the residual stream) and writes the
// MXFP4 codes and scales of
//     y = BlockDiag(R) applied to (norm(h) * gamma + beta) / lambda
// for RMSNorm, n = h / sqrt(mean(h^2) + eps), or LayerNorm,
// n = (h - mu) / sqrt(mean((h - mu)^2) + eps).  gamma / lambda and
// beta / lambda are formed once per block into LDS, so per element the
// smoothing costs one fused multiply-add.
//
// Work decomposition.  A norm needs the statistics of the whole row before
// any output, so a wave owns whole rows: it loads a row into registers (NT
// super-tiles of 64 groups, 16 bytes per lane per sub-tile of 16 groups, the
// layout of the plain rotate kernel), reduces the row's sums across the wave
// in fp64, and then runs every sub-tile through the same rotate + encode
// steps as the plain kernel.  Waves walk the rows with a stride of the grid's
// wave count; channels up to 2048 NT (NT = 1, 2, 4, 8).
//
// Row statistics.  Per super-tile (4 x 32 values of each of a lane's
// groups) a sum is formed in fp32 and the super-tiles are accumulated in
// fp64, then reduced across the wave in fp64, so the relative error of the
// mean square stays within ~128 ulp of fp32 at worst whatever the row
// length.  The RMS sum of squares and the LayerNorm sum run
// on the matrix cores, straight from the packed 16-bit elements: for the
// 16 x 16 x 32 MFMA the A and B operand layouts agree (lane l holds positions
// 8 (l / 16) .. + 7 of row, or column, l % 16), so the register that holds a
// sub-tile (lane l: channels 8 q .. + 7 of group j) times itself gives the
// Gram matrix of the sub-tile's 16 groups, whose diagonal holds the groups'
// sums of squares; with an all-ones A operand every row of the product holds
// the groups' sums.  The products are exact in fp32 (16-bit significands).
// LayerNorm takes a shift near the mean in a first sweep over the registers
// and the sums of x - shift and of its square on the VALU in a second, which
// gives the mean and variance with errors relative to the row's spread (a
// mean rounded to fp32 would be off by up to half an fp32 ulp of the mean,
// 3e-5 sd at mean / sd = 1000).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "mxq.h"
#include "mxq_device.h"
#include "mxq_internal.h"

// bf16 terms of x' = fma(n, gamma/lambda, beta/lambda): 2, each rounded to
// nearest (|x' - hi - lo| <= 2^-18 |x'|), or 3 (exact).
#ifndef MXQ_NORM_TERMS
#define MXQ_NORM_TERMS 2
#endif

namespace mxq {
namespace norm {

constexpr int kWave = 64;
constexpr int kGroup = 32;
constexpr int kSub = 4;            // sub-tiles of 16 groups per super-tile
constexpr int kTileGroups = 64;    // groups per super-tile
// Waves per block.  Every block builds the factor tables once, so long
// batches take blocks as large as the row buffers' registers allow (16
// waves leave 128 VGPRs per lane, 8 waves 256); short batches take 4-wave
// blocks, which spread their rows over more CUs.
template <int NT>
constexpr int kBigBlockWaves = NT <= 2 ? 16 : (NT == 4 ? 8 : 4);
constexpr int kSmallBlockWaves = 4;
constexpr int kMaxTiles = 8;       // channels <= 16384
enum : int { kRms = 0, kLayer = 1 };

struct NormArgs {
    const void* x;
    int64_t stride;  // elements
    const float* gamma;
    const float* beta;
    const float* lambda;
    const uint16_t* r_hat;
    uint8_t* codes;
    uint8_t* scales;
    float* y;
    float eps;
    int32_t tokens;
    int32_t channels;
    int32_t gpr;
    int32_t waves;  // waves in the grid (row stride)
};

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;

// c + the 16 x 16 x 32 product of two operands of packed 16-bit elements
// (the format of x), accumulated in fp32.
template <bool IS_FP16>
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t z) {
    if constexpr (IS_FP16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), z,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                       z, 0, 0, 0);
}

// v + the partner lane's v, the partner taken by a DPP move of both dwords
// (row_mirror 0x140: lane 15 - i of each 16-lane row; row_half_mirror 0x141:
// lane 7 - i of each 8; quad_perm 0xb1 and 0x4e: lane i ^ 1 and i ^ 2).
template <int CTRL>
__device__ __forceinline__ double add_dpp(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u)), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(u >> 32)), CTRL, 0xf, 0xf,
                                               false);
    return v + __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                              static_cast<uint32_t>(lo));
}

// v of lane l + v of lane l ^ 32 (l ^ 16 with SIXTEEN): a permlane swap of
// both dwords with both operands equal leaves the two values in its results.
template <bool SIXTEEN>
__device__ __forceinline__ double add_swap(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = static_cast<uint32_t>(u), hi = static_cast<uint32_t>(u >> 32);
    const auto sl = SIXTEEN ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                            : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto sh = SIXTEEN ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                            : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(sh[0]) << 32) | sl[0]) +
           __builtin_bit_cast(double, (static_cast<uint64_t>(sh[1]) << 32) | sl[1]);
}

// Sum over the wave's 64 lanes, the same bits in every lane.  Two permlane
// swaps fold lanes l ^ 32 and l ^ 16 together; within each 16-lane row, the
// mirror, half mirror and two quad exchanges each add two partial sums that
// together cover the row (lane i: {i, 15 - i}, then {i, 15 - i, 7 - i, 8 + i}
// within its half, then the quad).  Each step adds a, b in one lane and b, a
// in its partner, so all lanes agree.  No LDS round trip (a ds_bpermute per
// dword and step before).
__device__ __forceinline__ double wave_sum(double v) {
    v = add_swap<false>(v);
    v = add_swap<true>(v);
    v = add_dpp<0x140>(v);
    v = add_dpp<0x141>(v);
    v = add_dpp<0xb1>(v);
    return add_dpp<0x4e>(v);
}

// Waves per SIMD each instance reaches without the pass that redoes rare
// rows (after the main loop); stated to the compiler so that the pass spills
// rather than lowering the main loop's occupancy (16-wave blocks need 4).
template <int NORM, int NT, bool YOUT, int BW>
constexpr int kWavesPerSimd = BW == 16 ? 4
                              : NT == 1  ? 4
                              : NT == 2  ? ((YOUT || NORM == kLayer) ? 3 : 4)
                              : NT == 4  ? 2
                                         : 1;

template <int XT, int NORM, int NT, bool YOUT, bool TILED, int BW>
__global__ __attribute__((amdgpu_flat_work_group_size(1, kWave * BW),
                          amdgpu_waves_per_eu(kWavesPerSimd<NORM, NT, YOUT, BW>))) void norm_quant_kernel(NormArgs a) {
    constexpr int kBlockWaves = BW;
    constexpr int kBlockThreads = kWave * BW;
    constexpr bool kFp16 = XT == MXQ_FP16;
    constexpr int kUnits = NT * kSub * 2 * kWave;  // 16-byte factor units per table
    // Per-channel factors in the order the lanes consume them: unit
    // ((st * 4 + s) * 2 + h) * 64 + l holds the 4 factors of lane l's channels
    // 8 q + 4 h .. + 3 of group 64 st + 16 s + j (q = l / 16, j = l % 16), so a
    // wave reads 1 KB contiguously per ds_read_b128 (no bank conflicts).
    __shared__ __attribute__((aligned(16))) f32x4_t fm[kUnits];  // gamma / lambda
    __shared__ __attribute__((aligned(16))) f32x4_t fb[kUnits];  // beta / lambda

    // Fragment-tiled output of long batches (blocks of 8 or 16 waves): the
    // waves of a block hold BW consecutive rows (a record row, or half of
    // one), so their codes and scales meet in a block-shared LDS tile (two
    // of them, alternating) and the block stores whole records, 128-byte
    // lines at least, instead of one 16-byte piece per line from each row.
    // The stores are non-temporal (written once, read by the next kernel).
    // Row pitches in 16-byte slots: odd for 16 rows (a store lane l reads
    // row l % 16 of one group), 2 mod 16 for 8 rows (row l % 8 of group
    // (l / 8) % 4), so the 16 lanes of a ds_read_b128 pass hit distinct
    // bank quads.
    constexpr bool kStaged = TILED && BW >= 8;
    constexpr int kGroups = NT * kTileGroups;
    constexpr int kPitch = kGroups + (BW == 16 ? 1 : 2);
    __shared__ __attribute__((aligned(16))) u32x4_t stg[kStaged ? 2 : 1][kStaged ? BW : 1][kStaged ? kPitch : 1];
    __shared__ __attribute__((aligned(16))) uint8_t sstg[kStaged ? 2 : 1][kStaged ? kGroups * BW : 1];
    static_assert(!kStaged || BW == 8 || BW == 16, "a staged tile is a record row or half of one");

    const int C = a.channels;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int w = static_cast<int>(blockIdx.x) * kBlockWaves + wave;
    const int j = lane & 15;
    const int q = lane >> 4;
    const uint32_t gpr = static_cast<uint32_t>(a.gpr);

    const uint32_t row_bytes = gpr * kGroup * 2;
    const char* xb = static_cast<const char*>(a.x);
    // (row indices are uniform; readfirstlane tells the compiler so, or it
    // wraps every buffer access in a loop over distinct descriptors)
    auto load_tile = [&](u32x4_t (&tile)[kSub], int64_t r_any, int st) {
        const int64_t r = __builtin_amdgcn_readfirstlane(static_cast<int>(r_any));
        const auto rsrc = row_rsrc(xb + r * a.stride * 2, row_bytes);
#pragma unroll
        for (int s = 0; s < kSub; ++s) {
            const uint32_t off = (static_cast<uint32_t>(kTileGroups * st + 16 * s + j) * kGroup + 8 * q) * 2;
            tile[s] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, kAuxNT);
        }
    };
    auto load_row = [&](u32x4_t (&buf)[NT][kSub], int64_t r_any) {
#pragma unroll
        for (int st = 0; st < NT; ++st) load_tile(buf[st], r_any, st);
    };

    // The block's 2 KB (raw bf16 bits; the operands are formed after the setup).
    uint16_t r_raw[2][8];
    {
        const int n0 = 8 * (j >> 2) + (j & 3);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            r_raw[0][t] = a.r_hat[(8 * q + t) * kGroup + n0];
            r_raw[1][t] = a.r_hat[(8 * q + t) * kGroup + n0 + 4];
        }
    }

    // Factor setup: thread t takes the runs of 4 consecutive channels
    // 4 t, 4 (t + threads), ... with 16-byte loads of gamma, beta and lambda
    // (coalesced).  The 4 channels of a run fill one factor unit (one group,
    // one lane, one half), so a run is one 16-byte LDS store.  A batch of
    // runs issues all its loads before the first division waits on them: one
    // memory latency per batch, not one per channel.  Runs past the row end
    // (C is a multiple of 32, so a run is in or out whole) keep factor 0.
    // The wave's first row is loaded right after the first batch's factors:
    // vector loads complete in issue order for the wait counter, so the
    // setup waits for its own loads only and overlaps the row's latency; the
    // row load is unconditional (past the end through an empty buffer
    // range), or the compiler's wait for the factors would have to assume
    // the row loads may be the later ones and wait for them too.
    constexpr int kRuns = NT * kTileGroups * kGroup / 4;
    constexpr int kPerThread = (kRuns + kBlockThreads - 1) / kBlockThreads;
    constexpr int kBatch = kPerThread < 4 ? kPerThread : 4;
    static_assert(kPerThread % kBatch == 0, "whole batches");
    const uint32_t nbytes = static_cast<uint32_t>(C) * 4;
    const auto grs = row_rsrc(a.gamma, nbytes);
    const auto brs = row_rsrc(a.beta, a.beta ? nbytes : 0);
    const auto lrs = row_rsrc(a.lambda, a.lambda ? nbytes : 0);
    typedef u32x4_t Batch[kBatch];
    auto factor_loads = [&](int b0, Batch& gv, Batch& bv, Batch& lv) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const uint32_t off = (static_cast<uint32_t>(b0 + i) * kBlockThreads + threadIdx.x) * 16;
            gv[i] = __builtin_amdgcn_raw_buffer_load_b128(grs, off, 0, 0);
            bv[i] = __builtin_amdgcn_raw_buffer_load_b128(brs, off, 0, 0);
            lv[i] = __builtin_amdgcn_raw_buffer_load_b128(lrs, off, 0, 0);
        }
    };
    auto factor_math = [&](int b0, const Batch& gv, const Batch& bv, const Batch& lv) {
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int u = (b0 + i) * kBlockThreads + static_cast<int>(threadIdx.x);  // run: channels 4u .. 4u + 3
            if (kRuns % kBlockThreads != 0 && u >= kRuns) continue;
            f32x4_t mv = {0.0f, 0.0f, 0.0f, 0.0f}, bq = {0.0f, 0.0f, 0.0f, 0.0f};
            if (4 * u < C) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float lam = a.lambda ? as_f32(lv[i][t]) : 1.0f;
                    mv[t] = as_f32(gv[i][t]) / lam;
                    bq[t] = a.beta ? as_f32(bv[i][t]) / lam : 0.0f;
                }
            }
            const int p = u >> 3;  // group: 16 ss + j
            const int k = 4 * (u & 7);  // first channel of the run in its group: 8 q + 4 h
            const int lane_c = 16 * (k >> 3) + (p & 15);
            const int unit = ((p >> 4) * 2 + ((k >> 2) & 1)) * kWave + lane_c;
            fm[unit] = mv;
            fb[unit] = bq;
        }
    };
    u32x4_t bufA[NT][kSub], bufB[NT][kSub];
    {
        Batch gv, bv, lv;
        factor_loads(0, gv, bv, lv);
        // (keeps the compiler from hoisting the row loads above the factors')
        asm volatile("" ::: "memory");
        const bool in = w < a.tokens;
        const auto rsrc0 = row_rsrc(xb + (in ? static_cast<int64_t>(w) : 0) * a.stride * 2, in ? row_bytes : 0u);
#pragma unroll
        for (int st = 0; st < NT; ++st)
#pragma unroll
            for (int s = 0; s < kSub; ++s) {
                const uint32_t off = (static_cast<uint32_t>(kTileGroups * st + 16 * s + j) * kGroup + 8 * q) * 2;
                bufA[st][s] = __builtin_amdgcn_raw_buffer_load_b128(rsrc0, off, 0, kAuxNT);
            }
        factor_math(0, gv, bv, lv);
    }
#pragma unroll 1
    for (int b0 = kBatch; b0 < kPerThread; b0 += kBatch) {
        Batch gv, bv, lv;
        factor_loads(b0, gv, bv, lv);
        factor_math(b0, gv, bv, lv);
    }
    // A bare barrier: __syncthreads() would also wait for the row's loads.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // The block as the A operands of the two output halves (the layout of the
    // plain rotate kernel): A_h[t] = R[8q + t][8 (j / 4) + 4 h + j % 4].
    bf16x8_t A0, A1;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        A0[t] = __builtin_bit_cast(__bf16, r_raw[0][t]);
        A1[t] = __builtin_bit_cast(__bf16, r_raw[1][t]);
    }

    // Row statistics of a row held in registers (groups past the row end
    // loaded zeros).  LayerNorm: the first sweep gives a shift mu0 (an fp32
    // value near the mean); the second accumulates x - mu0 and its square, so
    // that mean = mu0 + E[x - mu0] and var = E[(x - mu0)^2] - E[x - mu0]^2
    // carry errors relative to the spread of the row, not to its mean.  The
    // mean is then applied as an fp32 pair mu + mu_lo.  s2 is the row's sum
    // of squares (of x - mu0 for LayerNorm).
    auto row_stats = [&](u32x4_t (&buf)[NT][kSub], double& s2, double& var, double& mean, float& mu,
                         float& mu_lo) {
        mu = 0.0f;
        mu_lo = 0.0f;
        mean = 0.0;
        if constexpr (NORM == kLayer) {
            // all-ones A operand (packed 1.0 pairs): row 0 of the product
            // (register 0 of lanes 0..15) holds the sums of groups j = lane
            constexpr uint32_t kOne2 = kFp16 ? 0x3c003c00u : 0x3f803f80u;
            const u32x4_t ones = {kOne2, kOne2, kOne2, kOne2};
            double part = 0.0;
#pragma unroll
            for (int st = 0; st < NT; ++st) {
                f32x4_t sums = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < kSub; ++s) sums = mfma16<kFp16>(ones, buf[st][s], sums);
                part += q == 0 ? static_cast<double>(sums[0]) : 0.0;
            }
            mu = static_cast<float>(wave_sum(part) / C);
#pragma unroll
            for (int st = 0; st < NT; ++st)
#pragma unroll
                for (int s = 0; s < kSub; ++s) asm volatile("" : "+v"(buf[st][s]));
        }
        double part = 0.0, part1 = 0.0;
#pragma unroll
        for (int st = 0; st < NT; ++st) {
            if constexpr (NORM == kLayer) {
#pragma unroll
                for (int s = 0; s < kSub; ++s) {
                    // lanes of groups past the row end loaded zeros, which
                    // are not zero once centred
                    const bool valid = kTileGroups * st + 16 * s + j < a.gpr;
                    float f[8];
                    widen8<kFp16>(buf[st][s], f);
                    float c8 = 0.0f, s8 = 0.0f;
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const float d = f[t] - mu;
                        s8 += d;
                        c8 += d * d;
                    }
                    part += valid ? static_cast<double>(c8) : 0.0;
                    part1 += valid ? static_cast<double>(s8) : 0.0;
                }
            } else {
                // diagonal entry (j, j) of the super-tile's Gram matrices:
                // lane 16 (j / 4) + j, register j % 4
                f32x4_t gram = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < kSub; ++s) gram = mfma16<kFp16>(buf[st][s], buf[st][s], gram);
                const int r = j & 3;
                const float dj = r == 0 ? gram[0] : r == 1 ? gram[1] : r == 2 ? gram[2] : gram[3];
                part += q == (j >> 2) ? static_cast<double>(dj) : 0.0;
            }
        }
        s2 = wave_sum(part);
        var = s2 / C;
        if constexpr (NORM == kLayer) {
            const double d1 = wave_sum(part1) / C;  // E[x - mu0]
            var -= d1 * d1;
            mean = static_cast<double>(mu) + d1;
            mu = static_cast<float>(mean);
            mu_lo = static_cast<float>(mean - static_cast<double>(mu));
        }
        // Keep only the packed row live across the statistics: an empty asm
        // that claims to change the registers stops the compiler from holding
        // the widened fp32 copies (twice the registers) until the second use.
#pragma unroll
        for (int st = 0; st < NT; ++st)
#pragma unroll
            for (int s = 0; s < kSub; ++s) asm volatile("" : "+v"(buf[st][s]));
    };

    // Rows of one super-tile (up to 2048 channels) alternate between two row
    // buffers: the next row is in flight while the current one computes.
    // Longer rows keep one buffer, and each super-tile of the next row loads
    // into its registers as soon as the current row's super-tile is encoded
    // (at 4096 channels this is 2-4 % faster than two buffers, bit-identical).
    constexpr bool kDouble = NT <= 1;
    // Rows the main loop cannot do exactly enough (rare) only set fix_seen
    // there and are redone after it: bf16 rows whose squares leave fp32's
    // range, and rows holding a group whose rotated maximum is below 2^-64.
    bool fix_seen = false;
    // Staged: the loop runs over the block's row groups, the same for every
    // wave of the block (it meets a barrier each time); a wave whose row is
    // past the end stages zeros, which become the padding rows.
    int sb = 0;  // staging tile of this step
    for (int64_t r_loop = kStaged ? w - wave : w; r_loop < a.tokens; r_loop += a.waves) {
        const int64_t r = __builtin_amdgcn_readfirstlane(static_cast<int>(kStaged ? r_loop + wave : r_loop));
        u32x4_t (&buf)[NT][kSub] = bufA;
        if (kStaged && r >= a.tokens) {
#pragma unroll
            for (int st = 0; st < NT; ++st) {
                stg[sb][kStaged ? wave : 0][kTileGroups * st + lane] = u32x4_t{0u, 0u, 0u, 0u};
                sstg[sb][(kTileGroups * st + lane) * BW + wave] = 0;
            }
        } else {
            if constexpr (kDouble) {
                if (r + a.waves < a.tokens) load_row(bufB, r + a.waves);
            }
            // ---- row statistics (groups past the row end loaded zeros)
            double s2, var, mean;
            float mu, mu_lo;
            row_stats(buf, s2, var, mean, mu, mu_lo);
            // bf16 rows whose sum of squares left fp32's safe range (squares
            // over 2^128 or below 2^-149) are redone after the main loop; a
            // row of zeros (padding in a serving batch) has exact statistics
            // and is not (the test of its bits runs only in such rows)
            if constexpr (!kFp16) {
                if (!(s2 >= 0x1p-80 && s2 <= 0x1p+1000)) {
                    uint32_t nz = 0;
#pragma unroll
                    for (int st = 0; st < NT; ++st)
#pragma unroll
                        for (int s = 0; s < kSub; ++s)
#pragma unroll
                            for (int i = 0; i < 4; ++i) nz |= buf[st][s][i] & 0x7fff7fffu;
                    fix_seen |= !(s2 == 0.0 && !any_lane(nz != 0u));
                }
            }
            const float inv = static_cast<float>(1.0 / sqrt(var + static_cast<double>(a.eps)));

            // ---- normalize, smooth, rotate, encode
            // Row layout: the row's codes and scales.  Fragment-tiled layout
            // (records of 16 rows x 4 groups): the row's record row; group g of
            // row r is slot 16 (g % 4) + r % 16 of record g / 4.
            const uint32_t nrec = gpr / 4;
            const auto crsrc = TILED ? row_rsrc(a.codes + (r >> 4) * nrec * 1024, nrec * 1024)
                                     : row_rsrc(a.codes + r * a.gpr * 16, gpr * 16);
            const auto srsrc = TILED ? row_rsrc(a.scales + (r >> 4) * nrec * 64, nrec * 64)
                                     : row_rsrc(a.scales + r * a.gpr, gpr);
            const uint32_t r16 = static_cast<uint32_t>(r & 15);
#pragma unroll
            for (int st = 0; st < NT; ++st) {
                uint32_t word[kSub];
                uint32_t sc[kSub];
#pragma unroll
                for (int s = 0; s < kSub; ++s) {
                    const int ss = st * kSub + s;
                    const f32x4_t m0 = fm[(ss * 2 + 0) * kWave + lane];
                    const f32x4_t m1 = fm[(ss * 2 + 1) * kWave + lane];
                    const f32x4_t b0 = fb[(ss * 2 + 0) * kWave + lane];
                    const f32x4_t b1 = fb[(ss * 2 + 1) * kWave + lane];
                    float f[8];
                    widen8<kFp16>(buf[st][s], f);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float d0 = NORM == kLayer ? ((f[t] - mu) - mu_lo) * inv : f[t] * inv;
                        const float d1 = NORM == kLayer ? ((f[4 + t] - mu) - mu_lo) * inv : f[4 + t] * inv;
                        f[t] = __builtin_fmaf(d0, m0[t], b0[t]);
                        f[4 + t] = __builtin_fmaf(d1, m1[t], b1[t]);
                    }
                    f32x4_t d0 = {}, d1 = {};
                    if constexpr (MXQ_NORM_TERMS == 2) {
                        // two bf16 terms, each rounded to nearest
                        typedef __attribute__((ext_vector_type(2))) float f32x2_t;
                        typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
                        u32x4_t hi, lo;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const bf16x2_t h = __builtin_convertvector(f32x2_t{f[2 * i], f[2 * i + 1]}, bf16x2_t);
                            hi[i] = __builtin_bit_cast(uint32_t, h);
                            const f32x2_t rr = f32x2_t{f[2 * i], f[2 * i + 1]} - __builtin_convertvector(h, f32x2_t);
                            lo[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(rr, bf16x2_t));
                        }
                        d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, __builtin_bit_cast(bf16x8_t, hi), d0, 0, 0, 0);
                        d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, __builtin_bit_cast(bf16x8_t, hi), d1, 0, 0, 0);
                        d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, __builtin_bit_cast(bf16x8_t, lo), d0, 0, 0, 0);
                        d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, __builtin_bit_cast(bf16x8_t, lo), d1, 0, 0, 0);
                    } else {
                    // exact bf16 terms of the fp32 values (3 terms cover 24 bits)
#pragma unroll
                    for (int term = 0; term < 3; ++term) {
                        u32x4_t bt;
#pragma unroll
                        for (int i = 0; i < 4; ++i) bt[i] = bf16_pair_hi(f[2 * i], f[2 * i + 1]);
                        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bt);
                        d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, b, d0, 0, 0, 0);
                        d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, b, d1, 0, 0, 0);
                        if (term < 2) {
#pragma unroll
                            for (int t = 0; t < 8; ++t) f[t] = bf16_residual(f[t]);
                        }
                    }
                    }
                    float v[8];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        v[t] = d0[t];
                        v[4 + t] = d1[t];
                    }
                    const uint32_t scale_bits = e8m0_scale_bits(group_amax8(v));
                    sc[s] = scale_bits >> 23;
                    word[s] = encode8(v, as_f32(scale_bits));
                    if constexpr (YOUT) {
                        const auto yrsrc = row_rsrc(a.y + r * a.gpr * kGroup, gpr * kGroup * 4);
                        const uint32_t off = (static_cast<uint32_t>(kTileGroups * st + 16 * s + j) * kGroup + 8 * q) * 4;
                        __builtin_amdgcn_raw_buffer_store_b128(
                            u32x4_t{as_u32(v[0]), as_u32(v[1]), as_u32(v[2]), as_u32(v[3])}, yrsrc, off, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b128(
                            u32x4_t{as_u32(v[4]), as_u32(v[5]), as_u32(v[6]), as_u32(v[7])}, yrsrc, off + 16, 0, 0);
                    }
                }
                transpose_words(word);
                const uint32_t S = q == 0 ? sc[0] : q == 1 ? sc[1] : q == 2 ? sc[2] : sc[3];
                const uint32_t g = static_cast<uint32_t>(kTileGroups * st + lane);
                // (groups past the row end, zeros whose stores are dropped, do not count)
                bool tiny = S < (kTinyScaleBits >> 23) && g < gpr;
                if constexpr (NORM == kRms) {
                    // With RMSNorm and no beta a group of zero inputs has
                    // x' = 0 exactly, so its codes and scale are exact
                    // already: only groups holding a nonzero input bit
                    // pattern (bit j of nzm[s]: group 16 s + j) count.  The
                    // ballots run only where some group fell below the bound.
                    if (!a.beta && any_lane(tiny)) {
                        uint32_t nzm[kSub];
#pragma unroll
                        for (int s = 0; s < kSub; ++s) {
                            const u32x4_t& w = buf[st][s];
                            const uint64_t b =
                                __builtin_amdgcn_ballot_w64(((w[0] | w[1] | w[2] | w[3]) & 0x7fff7fffu) != 0u);
                            const uint64_t f = b | (b >> 32);
                            nzm[s] = static_cast<uint32_t>(f | (f >> 16)) & 0xffffu;
                        }
                        const uint32_t nz = q == 0 ? nzm[0] : q == 1 ? nzm[1] : q == 2 ? nzm[2] : nzm[3];
                        tiny = tiny && ((nz >> j) & 1u);
                    }
                }
                fix_seen |= tiny;
                if constexpr (kStaged) {
                    stg[sb][wave][g] = u32x4_t{word[0], word[1], word[2], word[3]};
                    sstg[sb][g * BW + wave] = static_cast<uint8_t>(S);
                } else {
                    const uint32_t slot = TILED ? (g >> 2) * 64 + (g & 3) * 16 + r16 : g;
                    __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{word[0], word[1], word[2], word[3]}, crsrc, slot * 16,
                                                           0, TILED ? 0 : kAuxNT);
                    __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(S), srsrc, slot, 0, 0);
                }
                if constexpr (!kDouble) {
                    if (r + a.waves < a.tokens) load_tile(bufA[st], r + a.waves, st);
                }
            }
            if constexpr (kDouble) {
#pragma unroll
                for (int st = 0; st < NT; ++st)
#pragma unroll
                    for (int s = 0; s < kSub; ++s) bufA[st][s] = bufB[st][s];
            }
        }  // row of this wave
        if constexpr (kStaged) {
            // Every wave's LDS writes complete, then the block meets.  A bare
            // s_barrier: __syncthreads() would also wait for the next rows'
            // loads in flight.  The "memory" clobber keeps the compiler from
            // moving LDS accesses across it.
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            const int64_t base = r_loop;  // first row of the block's group
            const uint32_t nrec = gpr / 4;
            const auto crt = row_rsrc(a.codes + (base >> 4) * nrec * 1024, nrec * 1024);
            const auto srt = row_rsrc(a.scales + (base >> 4) * nrec * 64, nrec * 64);
            if constexpr (BW == 16) {
                // lane l: slot l of record s = row l % 16, group 4 s + l / 16
                for (uint32_t s = static_cast<uint32_t>(wave); s < nrec; s += BW)
                    __builtin_amdgcn_raw_buffer_store_b128(stg[sb][lane & 15][4 * s + (lane >> 4)], crt,
                                                           s * 1024 + 16 * static_cast<uint32_t>(lane), 0, kAuxNT);
                for (uint32_t g = static_cast<uint32_t>(wave * kWave + lane); g < gpr; g += BW * kWave)
                    __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t*>(&sstg[sb][g * BW]), srt,
                                                           (g >> 2) * 64 + (g & 3) * 16, 0, kAuxNT);
            } else {
                // half record rows: lane l carries row l % 8 of group (l / 8) % 4
                // of record 2 m + l / 32
                const uint32_t hb = static_cast<uint32_t>(base >> 3) & 1;
                const uint32_t lr = static_cast<uint32_t>(lane & 7);
                const uint32_t lg = static_cast<uint32_t>(lane >> 3) & 3;
                for (uint32_t m = static_cast<uint32_t>(wave); 2 * m < nrec; m += BW) {
                    const uint32_t s = 2 * m + static_cast<uint32_t>(lane >> 5);
                    if (s < nrec)
                        __builtin_amdgcn_raw_buffer_store_b128(stg[sb][lr][4 * s + lg], crt,
                                                               s * 1024 + lg * 256 + (8 * hb + lr) * 16, 0, kAuxNT);
                }
                for (uint32_t g = static_cast<uint32_t>(wave * kWave + lane); g < gpr; g += BW * kWave)
                    __builtin_amdgcn_raw_buffer_store_b64(*reinterpret_cast<const u32x2_t*>(&sstg[sb][g * BW]), srt,
                                                          (g >> 2) * 64 + (g & 3) * 16 + 8 * hb, 0, kAuxNT);
            }
            sb ^= 1;
        }
    }

    // ---- rows redone (rare) -------------------------------------------------
    // When any of this wave's rows set fix_seen, the wave recomputes all of
    // its rows and stores them again, row by row (the bytes of rows that
    // needed nothing come out the same).  Per row:
    //  - bf16 rows whose sum of squares left [2^-80, 2^1000] are scaled by
    //    2^kr (kr from the row's largest |h|, exact for the 16-bit values
    //    that matter) and the statistics retaken, with eps scaled by 2^(2 kr):
    //    the normalized row is unchanged;
    //  - a group whose rotated maximum is below 2^-64 is recomputed from
    //    x' * 2^k (k from its largest |x'|, at most 64), formed as
    //    fma(d 2^k, gamma / lambda, (beta / lambda) 2^k), with d 2^k taken
    //    from 1/sqrt in fp64 times 2^k, so no fp32 subnormal enters.
    // Staged blocks first let every wave's record stores complete (each wave
    // waits for its own, then the block meets), since a row's records were
    // stored by several waves of its block; the wait before the pass does
    // the same for the wave's own stores.  The waves of a block share one
    // L2, so the wait is enough: an agent-scope release fence here (an L2
    // write-back, buffer_wbl2, by every wave) took 8192 x 4096 from 22.6 to
    // 76 us.
    if constexpr (kStaged) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (any_lane(fix_seen)) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // x' of a sub-tile's 8 values -> the rotated values (3 exact bf16 terms)
        auto rotate3 = [&](const float (&xp)[8], float (&v)[8]) {
            float f[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) f[t] = xp[t];
            f32x4_t d0 = {}, d1 = {};
#pragma unroll
            for (int term = 0; term < 3; ++term) {
                u32x4_t bt;
#pragma unroll
                for (int i = 0; i < 4; ++i) bt[i] = bf16_pair_hi(f[2 * i], f[2 * i + 1]);
                const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bt);
                d0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, b, d0, 0, 0, 0);
                d1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, b, d1, 0, 0, 0);
                if (term < 2) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) f[t] = bf16_residual(f[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                v[t] = d0[t];
                v[4 + t] = d1[t];
            }
        };
        for (int64_t r_any = w; r_any < a.tokens; r_any += a.waves) {
            const int64_t r = __builtin_amdgcn_readfirstlane(static_cast<int>(r_any));
            u32x4_t rb[NT][kSub];
            load_row(rb, r);
            double s2, var, mean;
            float mu, mu_lo;
            row_stats(rb, s2, var, mean, mu, mu_lo);
            double eps_d = static_cast<double>(a.eps);
            if constexpr (!kFp16) {
                if (!(s2 >= 0x1p-80 && s2 <= 0x1p+1000)) {
                    uint32_t m = 0;  // largest |h| of the row, as bf16 bits
#pragma unroll
                    for (int st = 0; st < NT; ++st)
#pragma unroll
                        for (int s = 0; s < kSub; ++s)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const uint32_t d = rb[st][s][i];
                                const uint32_t lo = d & 0x7fffu, hi = (d >> 16) & 0x7fffu;
                                m = m > lo ? m : lo;
                                m = m > hi ? m : hi;
                            }
#pragma unroll
                    for (int o = 32; o >= 1; o >>= 1) {
                        const uint32_t other = static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o, kWave));
                        m = m > other ? m : other;
                    }
                    if (m != 0) {
                        // |h| 2^kr < 1 at the row's maximum
                        const int kr = -__builtin_amdgcn_frexp_expf(as_f32(m << 16));
#pragma unroll
                        for (int st = 0; st < NT; ++st)
#pragma unroll
                            for (int s = 0; s < kSub; ++s)
#pragma unroll
                                for (int i = 0; i < 4; ++i) {
                                    const uint32_t d = rb[st][s][i];
                                    rb[st][s][i] = bf16_pair_hi(ldexpf(as_f32(d << 16), kr),
                                                                ldexpf(as_f32(d & 0xffff0000u), kr));
                                }
                        eps_d = ldexp(eps_d, 2 * kr);
                        row_stats(rb, s2, var, mean, mu, mu_lo);
                    }
                }
            }
            const double inv64 = 1.0 / sqrt(var + eps_d);
            const float inv = static_cast<float>(inv64);
            const uint32_t nrec = gpr / 4;
            const auto crsrc = TILED ? row_rsrc(a.codes + (r >> 4) * nrec * 1024, nrec * 1024)
                                     : row_rsrc(a.codes + r * a.gpr * 16, gpr * 16);
            const auto srsrc = TILED ? row_rsrc(a.scales + (r >> 4) * nrec * 64, nrec * 64)
                                     : row_rsrc(a.scales + r * a.gpr, gpr);
            const uint32_t r16 = static_cast<uint32_t>(r & 15);
#pragma unroll
            for (int st = 0; st < NT; ++st) {
                uint32_t word[kSub], sc[kSub];
#pragma unroll
                for (int s = 0; s < kSub; ++s) {
                    const int ss = st * kSub + s;
                    const f32x4_t m0 = fm[(ss * 2 + 0) * kWave + lane];
                    const f32x4_t m1 = fm[(ss * 2 + 1) * kWave + lane];
                    const f32x4_t b0 = fb[(ss * 2 + 0) * kWave + lane];
                    const f32x4_t b1 = fb[(ss * 2 + 1) * kWave + lane];
                    float f[8], xp[8], v[8];
                    widen8<kFp16>(rb[st][s], f);
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const float d0 = NORM == kLayer ? ((f[t] - mu) - mu_lo) * inv : f[t] * inv;
                        const float d1 = NORM == kLayer ? ((f[4 + t] - mu) - mu_lo) * inv : f[4 + t] * inv;
                        xp[t] = __builtin_fmaf(d0, m0[t], b0[t]);
                        xp[4 + t] = __builtin_fmaf(d1, m1[t], b1[t]);
                    }
                    rotate3(xp, v);
                    uint32_t sbits = e8m0_scale_bits(group_amax8(v)), cbits = sbits;
                    int ksh = 0;
                    const bool tiny = sbits < kTinyScaleBits;
                    if (any_lane(tiny)) {
                        const int k = tiny ? tiny_shift(group_amax8(xp)) : 0;
                        const float inv_k = static_cast<float>(ldexp(inv64, k));
                        const float up = as_f32(static_cast<uint32_t>(127 + k) << 23);
                        float xs[8], w[8];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const float d0 = NORM == kLayer ? ((f[t] - mu) - mu_lo) * inv_k : f[t] * inv_k;
                            const float d1 = NORM == kLayer ? ((f[4 + t] - mu) - mu_lo) * inv_k : f[4 + t] * inv_k;
                            xs[t] = __builtin_fmaf(d0, m0[t], b0[t] * up);
                            xs[4 + t] = __builtin_fmaf(d1, m1[t], b1[t] * up);
                        }
                        rotate3(xs, w);
                        uint32_t s2b, c2b;
                        shifted_scale_bits(group_amax8(w), k, s2b, c2b);
#pragma unroll
                        for (int t = 0; t < 8; ++t) v[t] = tiny ? w[t] : v[t];
                        sbits = tiny ? s2b : sbits;
                        cbits = tiny ? c2b : cbits;
                        ksh = k;
                    }
                    sc[s] = sbits >> 23;
                    word[s] = encode8(v, as_f32(cbits));
                    if constexpr (YOUT) {
                        const float down = pow2_neg(ksh);
                        const auto yrsrc = row_rsrc(a.y + r * a.gpr * kGroup, gpr * kGroup * 4);
                        const uint32_t off = (static_cast<uint32_t>(kTileGroups * st + 16 * s + j) * kGroup + 8 * q) * 4;
                        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{as_u32(v[0] * down), as_u32(v[1] * down),
                                                                       as_u32(v[2] * down), as_u32(v[3] * down)},
                                                               yrsrc, off, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{as_u32(v[4] * down), as_u32(v[5] * down),
                                                                       as_u32(v[6] * down), as_u32(v[7] * down)},
                                                               yrsrc, off + 16, 0, 0);
                    }
                }
                transpose_words(word);
                const uint32_t S = q == 0 ? sc[0] : q == 1 ? sc[1] : q == 2 ? sc[2] : sc[3];
                const uint32_t g = static_cast<uint32_t>(kTileGroups * st + lane);
                const uint32_t slot = TILED ? (g >> 2) * 64 + (g & 3) * 16 + r16 : g;
                __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{word[0], word[1], word[2], word[3]}, crsrc, slot * 16, 0,
                                                       0);
                __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(S), srsrc, slot, 0, 0);
            }
        }
    }
}

bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// Resident blocks per CU the instance allows (registers, LDS), queried once.
template <int XT, int NORM, int NT, bool YOUT, bool TILED, int BW>
int blocks_per_cu() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, norm_quant_kernel<XT, NORM, NT, YOUT, TILED, BW>, kWave * BW,
                                                     0) != hipSuccess ||
        v <= 0)
        v = 1;
    cached.store(v, std::memory_order_relaxed);
    return v;
}

template <int XT, int NORM, int NT, bool YOUT, bool TILED, int BW>
mxq_status launch_bw(NormArgs a, hipStream_t st) {
    constexpr int kBlockWaves = BW;
    const int per_cu = blocks_per_cu<XT, NORM, NT, YOUT, TILED, BW>();
    const int64_t want = (static_cast<int64_t>(a.tokens) + kBlockWaves - 1) / kBlockWaves;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * per_cu;
    const int blocks = static_cast<int>(want < cap ? want : cap);
    a.waves = blocks * kBlockWaves;
    hipLaunchKernelGGL((norm_quant_kernel<XT, NORM, NT, YOUT, TILED, BW>), dim3(blocks), dim3(kWave * BW), 0, st, a);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

template <int XT, int NORM, int NT, bool YOUT, bool TILED>
mxq_status launch_nt(const NormArgs& a, hipStream_t st) {
    constexpr int kBig = kBigBlockWaves<NT>;
    if constexpr (kBig == kSmallBlockWaves) {
        return launch_bw<XT, NORM, NT, YOUT, TILED, kBig>(a, st);
    } else {
        if (a.tokens >= static_cast<int64_t>(device_cu_count()) * kBig)
            return launch_bw<XT, NORM, NT, YOUT, TILED, kBig>(a, st);
        return launch_bw<XT, NORM, NT, YOUT, TILED, kSmallBlockWaves>(a, st);
    }
}

template <int XT, int NORM, bool YOUT, bool TILED>
mxq_status launch_tiles(const NormArgs& a, hipStream_t st) {
    const int tiles = (a.gpr + kTileGroups - 1) / kTileGroups;
    if (tiles <= 1) return launch_nt<XT, NORM, 1, YOUT, TILED>(a, st);
    if (tiles <= 2) return launch_nt<XT, NORM, 2, YOUT, TILED>(a, st);
    if (tiles <= 4) return launch_nt<XT, NORM, 4, YOUT, TILED>(a, st);
    return launch_nt<XT, NORM, 8, YOUT, TILED>(a, st);
}

// The rotated-value output is a template parameter: a runtime branch around
// its stores would cut the unrolled sub-tiles into separate basic blocks
// that the scheduler cannot interleave.
template <int XT, int NORM>
mxq_status launch_norm(const NormArgs& a, hipStream_t st, bool tiled) {
    if (tiled) return launch_tiles<XT, NORM, false, true>(a, st);
    return a.y ? launch_tiles<XT, NORM, true, false>(a, st) : launch_tiles<XT, NORM, false, false>(a, st);
}

mxq_status norm_impl(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels, int64_t x_row_stride,
                     int32_t norm_kind, const float* gamma, const float* beta, float eps, const float* lambda,
                     const uint16_t* r_hat, uint8_t* codes, uint8_t* scales, float* y_rot, void* stream,
                     bool tiled) {
    if (x_dtype != MXQ_BF16 && x_dtype != MXQ_FP16) return MXQ_ERR_DTYPE;
    if (norm_kind != MXQ_NORM_RMS && norm_kind != MXQ_NORM_LAYER) return MXQ_ERR_DTYPE;
    if (tokens < 0 || channels < 0 || channels % kGroup || channels > kMaxTiles * kTileGroups * kGroup ||
        tokens >= (int64_t(1) << 31) || (tiled && channels % 128))
        return MXQ_ERR_SHAPE;
    if (!(eps >= 0.0f) || !(eps <= 3.4028234663852886e38f)) return MXQ_ERR_SHAPE;  // NaN, negative, inf
    if (tokens == 0 || channels == 0) return MXQ_OK;
    if (!x || !gamma || !r_hat || !codes || !scales) return MXQ_ERR_NULL;
    if (x_row_stride < channels) return MXQ_ERR_STRIDE;
    if (!aligned_to(x, 16) || (x_row_stride * 2) % 16 || !aligned_to(codes, 16) || !aligned_to(r_hat, 2) ||
        (tiled && !aligned_to(scales, 16)) ||
        !aligned_to(gamma, 4) || (beta && !aligned_to(beta, 4)) || (lambda && !aligned_to(lambda, 4)) ||
        (y_rot && !aligned_to(y_rot, 16)))
        return MXQ_ERR_ALIGN;
    NormArgs a{x,      x_row_stride, gamma, beta, lambda, r_hat, codes, scales, y_rot, eps,
               static_cast<int32_t>(tokens), static_cast<int32_t>(channels),
               static_cast<int32_t>(channels / kGroup), 0};
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (x_dtype == MXQ_BF16)
        return norm_kind == MXQ_NORM_RMS ? launch_norm<MXQ_BF16, kRms>(a, st, tiled)
                                         : launch_norm<MXQ_BF16, kLayer>(a, st, tiled);
    return norm_kind == MXQ_NORM_RMS ? launch_norm<MXQ_FP16, kRms>(a, st, tiled)
                                     : launch_norm<MXQ_FP16, kLayer>(a, st, tiled);
}

}  // namespace norm
}  // namespace mxq

using namespace mxq::norm;

extern "C" mxq_status mxq_norm_rotate_quant(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                            int64_t x_row_stride, int32_t norm_kind, const float* gamma,
                                            const float* beta, float eps, const float* lambda,
                                            const uint16_t* r_hat, uint8_t* codes, uint8_t* scales, float* y_rot,
                                            void* stream) {
    return norm_impl(x, x_dtype, tokens, channels, x_row_stride, norm_kind, gamma, beta, eps, lambda, r_hat, codes,
                     scales, y_rot, stream, false);
}

extern "C" mxq_status mxq_norm_rotate_quant_tiled(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                                  int64_t x_row_stride, int32_t norm_kind, const float* gamma,
                                                  const float* beta, float eps, const float* lambda,
                                                  const uint16_t* r_hat, uint8_t* tiled_codes,
                                                  uint8_t* tiled_scales, void* stream) {
    return norm_impl(x, x_dtype, tokens, channels, x_row_stride, norm_kind, gamma, beta, eps, lambda, r_hat,
                     tiled_codes, tiled_scales, nullptr, stream, true);
}
