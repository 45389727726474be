// Rotation by a B x B block for B = 16, 32, 64, 128, then MXFP4 of every
// 32-element group: the block sizes of the DuQuant++ page's ablation
// (sec. 4.3), which keeps MXFP4 groups 32 wide and varies the rotation
// block.  B = 32 is the main path (mxq_rotate_quant, a separate tuned
// kernel); this kernel serves the error study of the other sizes.
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

template <int XT, bool LAM, int KB, bool HALF>
__global__ __launch_bounds__(kBlockThreads) void block_quant_kernel(BlockArgs a) {
    constexpr bool kFp16 = XT == MXQ_FP16;
    constexpr int kSubs = 4 / KB;  // sub-tiles per super-tile
    constexpr int kB = HALF ? 16 : 32 * KB;
    constexpr int kTerms = (XT == MXQ_BF16 && !LAM) ? 1 : ((XT == MXQ_FP16 && !LAM) ? 2 : 3);
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int w = static_cast<int>(blockIdx.x) * kBlockWaves + wave;
    if (w >= a.tcols * a.row_step) return;
    const int tc = w % a.tcols;
    const int r0 = w / a.tcols;
    const int j = lane & 15;
    const int q = lane >> 4;
    const uint32_t gpr = static_cast<uint32_t>(a.gpr);
    const int p0 = tc * kTileGroups;

    // A operands: A[gamma][h][kappa][t] = R[32 kappa + 8 q + t][32 gamma + 8 (j / 4) + 4 h + j % 4]
    bf16x8_t A[KB][2][KB];
#pragma unroll
    for (int g = 0; g < KB; ++g)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int k = 0; k < KB; ++k)
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int row = 32 * k + 8 * q + t;
                    const int col = 32 * g + 8 * (j >> 2) + 4 * h + (j & 3);
                    uint16_t bits;
                    if constexpr (HALF)
                        bits = (row >> 4) == (col >> 4) ? a.r[(row & 15) * 16 + (col & 15)] : uint16_t(0);
                    else
                        bits = a.r[row * kB + col];
                    A[g][h][k][t] = __builtin_bit_cast(__bf16, bits);
                }

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
    for (int r_loop = r0; r_loop < a.tokens; r_loop += a.row_step) {
        const int64_t r = __builtin_amdgcn_readfirstlane(r_loop);
        const auto rsrc = row_rsrc(xb + r * a.stride * 2, row_bytes);
        u32x4_t xin[kSubs][KB];
#pragma unroll
        for (int s = 0; s < kSubs; ++s)
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const uint32_t grp = static_cast<uint32_t>(p0 + KB * (16 * s + j) + k);
                xin[s][k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (grp * kGroup + 8 * q) * 2, 0, kAuxNT);
            }
        uint32_t word[4], sc[4];
#pragma unroll
        for (int s = 0; s < kSubs; ++s) {
            f32x4_t d0[KB], d1[KB];
#pragma unroll
            for (int g = 0; g < KB; ++g) d0[g] = d1[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (kTerms == 1) {
#pragma unroll
                for (int k = 0; k < KB; ++k) {
                    const bf16x8_t b = __builtin_bit_cast(bf16x8_t, xin[s][k]);
#pragma unroll
                    for (int g = 0; g < KB; ++g) {
                        d0[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][0][k], b, d0[g], 0, 0, 0);
                        d1[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][1][k], b, d1[g], 0, 0, 0);
                    }
                }
            } else {
                float f[KB][8];
#pragma unroll
                for (int k = 0; k < KB; ++k) {
                    widen8<kFp16>(xin[s][k], f[k]);
                    if constexpr (LAM) {
#pragma unroll
                        for (int t = 0; t < 8; ++t) f[k][t] *= il[s][k][t];
                    }
                }
#pragma unroll
                for (int term = 0; term < kTerms; ++term) {
#pragma unroll
                    for (int k = 0; k < KB; ++k) {
                        u32x4_t bt;
#pragma unroll
                        for (int i = 0; i < 4; ++i) bt[i] = bf16_pair_hi(f[k][2 * i], f[k][2 * i + 1]);
                        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bt);
#pragma unroll
                        for (int g = 0; g < KB; ++g) {
                            d0[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][0][k], b, d0[g], 0, 0, 0);
                            d1[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[g][1][k], b, d1[g], 0, 0, 0);
                        }
                        if (term + 1 < kTerms) {
#pragma unroll
                            for (int t = 0; t < 8; ++t) f[k][t] = bf16_residual(f[k][t]);
                        }
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
                const uint32_t scale_bits = e8m0_scale_bits(group_amax8(v));
                sc[s * KB + g] = scale_bits >> 23;
                word[s * KB + g] = encode8(v, as_f32(scale_bits));
                if (a.y) {
                    const auto yrsrc = row_rsrc(a.y + r * a.gpr * kGroup, gpr * kGroup * 4);
                    const uint32_t grp = static_cast<uint32_t>(p0 + KB * (16 * s + j) + g);
                    const uint32_t off = (grp * kGroup + 8 * q) * 4;
                    __builtin_amdgcn_raw_buffer_store_b128(
                        u32x4_t{as_u32(v[0]), as_u32(v[1]), as_u32(v[2]), as_u32(v[3])}, yrsrc, off, 0, 0);
                    __builtin_amdgcn_raw_buffer_store_b128(
                        u32x4_t{as_u32(v[4]), as_u32(v[5]), as_u32(v[6]), as_u32(v[7])}, yrsrc, off + 16, 0, 0);
                }
            }
        }
        transpose_words(word);
        const uint32_t S = q == 0 ? sc[0] : q == 1 ? sc[1] : q == 2 ? sc[2] : sc[3];
        const uint32_t grp = static_cast<uint32_t>(p0 + KB * (16 * (q / KB) + j) + q % KB);
        const auto crsrc = row_rsrc(a.codes + r * a.gpr * 16, gpr * 16);
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{word[0], word[1], word[2], word[3]}, crsrc, grp * 16, 0,
                                               kAuxNT);
        const auto srsrc = row_rsrc(a.scales + r * a.gpr, gpr);
        __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(S), srsrc, grp, 0, 0);
    }
}

bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

template <int XT, bool LAM, int KB, bool HALF>
int waves_per_cu() {
    static std::atomic<int> cached{0};
    int v = cached.load(std::memory_order_relaxed);
    if (v > 0) return v;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, block_quant_kernel<XT, LAM, KB, HALF>, kBlockThreads,
                                                     0) != hipSuccess ||
        blocks <= 0)
        blocks = 1;
    v = blocks * kBlockWaves;
    cached.store(v, std::memory_order_relaxed);
    return v;
}

template <int XT, bool LAM, int KB, bool HALF>
mxq_status launch(BlockArgs a, hipStream_t st) {
    a.tcols = (a.gpr + kTileGroups - 1) / kTileGroups;
    const int64_t slots = static_cast<int64_t>(device_cu_count()) * waves_per_cu<XT, LAM, KB, HALF>();
    int64_t rs = slots / a.tcols;
    if (rs < 1) rs = 1;
    if (rs > a.tokens) rs = a.tokens;
    a.row_step = static_cast<int32_t>(rs);
    const int64_t waves = static_cast<int64_t>(a.tcols) * rs;
    const int blocks = static_cast<int>((waves + kBlockWaves - 1) / kBlockWaves);
    hipLaunchKernelGGL((block_quant_kernel<XT, LAM, KB, HALF>), dim3(blocks), dim3(kBlockThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

template <int XT, bool LAM>
mxq_status dispatch_block(const BlockArgs& a, int block, hipStream_t st) {
    switch (block) {
        case 16: return launch<XT, LAM, 1, true>(a, st);
        case 32: return launch<XT, LAM, 1, false>(a, st);
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
