// MXFP4 x MXFP4 product on the gfx950 scaled matrix cores: the consumer of
// the quantized activations (DuQuant++ page, sec. 3.3 and sec. 5.2: the
// rotated MXFP4 activations feed an MXFP4 linear layer whose weights carry
// the absorbed smoothing and rotation).
//
//   y[m][n] = sum_k dq(A)[m][k] * dq(B)[n][k]
//
// A (activations) and B (weights, one row per output feature) are both
// quantized along the reduction dimension K, in the library's storage
// format: codes [rows][K/2] (two E2M1 codes per byte, low nibble first) and
// E8M0 scales [rows][K/32].
//
// v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands multiplies a 16 x 128
// block of A by a 128 x 16 block of B^T.  Lane l supplies row l % 16 and the
// 32 consecutive K positions of block l / 16: 16 code bytes in the order they
// are stored, low nibble first, which is exactly one MXFP4 group, plus that
// group's scale byte.  Each operand fragment is therefore a plain 16-byte
// load per lane straight from the stored codes, with no repacking.  The sum
// over K does not care which group sits in which MFMA, so a lane loads 32
// contiguous bytes (two groups) per fragment per iteration and the two MFMAs
// of an iteration take its first and its second group; A and B use the same
// assignment, so every product pairs the same k.
//
// Tiling: a block of kWM x kWN waves computes a (16 kFM kWM) x (16 kFN kWN)
// tile of y; each wave holds kFM x kFN accumulator fragments.  Operands are
// loaded per wave through buffer resources bounded to the block's rows, so
// rows past M or N read as zero (codes 0, scale 2^-127: products 0) and
// ragged edges need no branches in the loop.  Two register sets alternate:
// the loads of iteration i + 1 are in flight while iteration i computes.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mxq.h"
#include "mxq_internal.h"

#ifndef MXQ_GEMM_FM
#define MXQ_GEMM_FM 4  // 16-row A fragments per wave
#endif
#ifndef MXQ_GEMM_FN
#define MXQ_GEMM_FN 4  // 16-row B fragments per wave
#endif
#ifndef MXQ_GEMM_WAVES_M
#define MXQ_GEMM_WAVES_M 2
#endif
#ifndef MXQ_GEMM_WAVES_N
#define MXQ_GEMM_WAVES_N 2
#endif
#ifndef MXQ_GEMM_GROUP_M
#define MXQ_GEMM_GROUP_M 8  // tile rows per band of the block order
#endif

namespace mxq {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4g_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4g_t;

constexpr int kWave = 64;
constexpr int kFM = MXQ_GEMM_FM, kFN = MXQ_GEMM_FN;
constexpr int kWM = MXQ_GEMM_WAVES_M, kWN = MXQ_GEMM_WAVES_N;
constexpr int kThreads = kWave * kWM * kWN;
constexpr int kBM = 16 * kFM * kWM;
constexpr int kBN = 16 * kFN * kWN;
constexpr int kKIter = 256;  // K positions per loop iteration
constexpr int kFmtE2M1 = 4;  // operand format code of the scaled MFMA for FP4
constexpr int kXcds = 8;     // MI355X: 8 accelerator dies, each with its own L2
constexpr int64_t kMaxK = int64_t(1) << 24;

struct GemmArgs {
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    void* y;
    int64_t ldy;
    int32_t M, N, K;
    int32_t tiles_m, tiles_n;
};

// One operand fragment of one lane for one iteration: the 16 code bytes of
// two consecutive groups and their two scale bytes (low byte first).
struct Frag {
    u32x4g_t c[2];
    uint32_t s;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ void load_frag(Frag& f, __amdgpu_buffer_rsrc_t codes, __amdgpu_buffer_rsrc_t scales,
                                          uint32_t coff, uint32_t soff, int it) {
    f.c[0] = __builtin_amdgcn_raw_buffer_load_b128(codes, coff, kKIter / 2 * it, 0);
    f.c[1] = __builtin_amdgcn_raw_buffer_load_b128(codes, coff + 16, kKIter / 2 * it, 0);
    f.s = __builtin_amdgcn_raw_buffer_load_b16(scales, soff, kKIter / 32 * it, 0);
}

__device__ __forceinline__ i32x8_t operand(const u32x4g_t& c) {
    return i32x8_t{static_cast<int>(c[0]), static_cast<int>(c[1]), static_cast<int>(c[2]), static_cast<int>(c[3]),
                   0, 0, 0, 0};
}

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int wm = wave / kWN;
    const int wn = wave % kWN;

    // Block order: dispatch ids go round-robin over the dies, so renumber
    // them to give each die a contiguous range of tiles; then walk bands of
    // kGroupM tile rows column by column, so the tiles resident at one time
    // on a die share A rows and B rows in its L2.
    const int nblk = static_cast<int>(gridDim.x);
    int bid = static_cast<int>(blockIdx.x);
    if (nblk % kXcds == 0) bid = (bid % kXcds) * (nblk / kXcds) + bid / kXcds;
    const int band = MXQ_GEMM_GROUP_M * g.tiles_n;
    const int first_m = (bid / band) * MXQ_GEMM_GROUP_M;
    const int band_rows = min(g.tiles_m - first_m, MXQ_GEMM_GROUP_M);
    const int in_band = bid % band;
    // (the tile indices are uniform; readfirstlane tells the compiler so, or
    // it would wrap every buffer load in a loop over distinct descriptors)
    const int tm = __builtin_amdgcn_readfirstlane(first_m + in_band % band_rows);
    const int tn = __builtin_amdgcn_readfirstlane(in_band / band_rows);

    const int64_t m0 = static_cast<int64_t>(tm) * kBM;
    const int64_t n0 = static_cast<int64_t>(tn) * kBN;
    const uint32_t cpr = static_cast<uint32_t>(g.K) / 2;   // code bytes per row
    const uint32_t spr = static_cast<uint32_t>(g.K) / 32;  // scale bytes per row
    const uint32_t rows_a = static_cast<uint32_t>(min<int64_t>(kBM, g.M - m0));
    const uint32_t rows_b = static_cast<uint32_t>(min<int64_t>(kBN, g.N - n0));
    const auto ra = rsrc(g.a_codes + m0 * cpr, rows_a * cpr);
    const auto rsa = rsrc(g.a_scales + m0 * spr, rows_a * spr);
    const auto rb = rsrc(g.b_codes + n0 * cpr, rows_b * cpr);
    const auto rsb = rsrc(g.b_scales + n0 * spr, rows_b * spr);

    const uint32_t r16 = static_cast<uint32_t>(lane & 15);
    const uint32_t h = static_cast<uint32_t>(lane >> 4);
    uint32_t ca[kFM], sa[kFM], cb[kFN], sb[kFN];
#pragma unroll
    for (int f = 0; f < kFM; ++f) {
        const uint32_t row = static_cast<uint32_t>(wm * 16 * kFM + 16 * f) + r16;
        ca[f] = row * cpr + 32 * h;
        sa[f] = row * spr + 2 * h;
    }
#pragma unroll
    for (int f = 0; f < kFN; ++f) {
        const uint32_t row = static_cast<uint32_t>(wn * 16 * kFN + 16 * f) + r16;
        cb[f] = row * cpr + 32 * h;
        sb[f] = row * spr + 2 * h;
    }

    f32x4g_t acc[kFM][kFN];
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j) acc[i][j] = f32x4g_t{0.f, 0.f, 0.f, 0.f};

    auto load = [&](Frag (&A)[kFM], Frag (&B)[kFN], int it) {
#pragma unroll
        for (int f = 0; f < kFM; ++f) load_frag(A[f], ra, rsa, ca[f], sa[f], it);
#pragma unroll
        for (int f = 0; f < kFN; ++f) load_frag(B[f], rb, rsb, cb[f], sb[f], it);
    };
    auto compute = [&](const Frag (&A)[kFM], const Frag (&B)[kFN]) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int i = 0; i < kFM; ++i)
#pragma unroll
                for (int j = 0; j < kFN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        operand(A[i].c[k]), operand(B[j].c[k]), acc[i][j], kFmtE2M1, kFmtE2M1, 0,
                        static_cast<int>((A[i].s >> (8 * k)) & 0xffu), 0,
                        static_cast<int>((B[j].s >> (8 * k)) & 0xffu));
    };

    const int nit = g.K / kKIter;
    Frag A0[kFM], B0[kFN], A1[kFM], B1[kFN];
    load(A0, B0, 0);
    int it = 0;
    for (; it + 2 <= nit; it += 2) {
        load(A1, B1, it + 1);
        compute(A0, B0);
        if (it + 2 < nit) load(A0, B0, it + 2);
        compute(A1, B1);
    }
    if (it < nit) compute(A0, B0);

    // Accumulator layout: lane l, register r holds row 4 (l / 16) + r,
    // column l % 16 of its 16 x 16 fragment.
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + wm * 16 * kFM + 16 * i + 4 * static_cast<int>(h) + r;
            if (row >= g.M) continue;
#pragma unroll
            for (int j = 0; j < kFN; ++j) {
                const int64_t col = n0 + wn * 16 * kFN + 16 * j + static_cast<int>(r16);
                if (col >= g.N) continue;
                if constexpr (OUT_BF16)
                    static_cast<__bf16*>(g.y)[row * g.ldy + col] = static_cast<__bf16>(acc[i][j][r]);
                else
                    static_cast<float*>(g.y)[row * g.ldy + col] = acc[i][j][r];
            }
        }
    }
}

bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace
}  // namespace mxq

using namespace mxq;

extern "C" {

mxq_status mxq_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* y, int32_t y_dtype,
                          int64_t ldy, void* stream) {
    if (y_dtype != MXQ_FP32 && y_dtype != MXQ_BF16) return MXQ_ERR_DTYPE;
    if (M < 0 || N < 0 || K < 0 || K % kKIter || K > kMaxK || M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31))
        return MXQ_ERR_SHAPE;
    if (M == 0 || N == 0) return MXQ_OK;
    if (!y) return MXQ_ERR_NULL;
    if (ldy < N) return MXQ_ERR_STRIDE;
    const uintptr_t ysz = y_dtype == MXQ_FP32 ? 4 : 2;
    if (!aligned_to(y, ysz)) return MXQ_ERR_ALIGN;
    const int64_t tiles_m = (M + kBM - 1) / kBM;
    const int64_t tiles_n = (N + kBN - 1) / kBN;
    // K == 0 is an empty reduction: the kernel reads nothing and writes zeros.
    if (K > 0 && (!a_codes || !a_scales || !b_codes || !b_scales)) return MXQ_ERR_NULL;
    if (!aligned_to(a_codes, 16) || !aligned_to(b_codes, 16) || !aligned_to(a_scales, 2) || !aligned_to(b_scales, 2))
        return MXQ_ERR_ALIGN;
    if (tiles_m * tiles_n >= (int64_t(1) << 31)) return MXQ_ERR_SHAPE;
    GemmArgs g{a_codes, a_scales, b_codes, b_scales, y, ldy, static_cast<int32_t>(M), static_cast<int32_t>(N),
               static_cast<int32_t>(K), static_cast<int32_t>(tiles_m), static_cast<int32_t>(tiles_n)};
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(static_cast<unsigned>(tiles_m * tiles_n));
    if (y_dtype == MXQ_BF16)
        hipLaunchKernelGGL((gemm_kernel<true>), grid, dim3(kThreads), 0, st, g);
    else
        hipLaunchKernelGGL((gemm_kernel<false>), grid, dim3(kThreads), 0, st, g);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

}  // extern "C"
