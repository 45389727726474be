// gfx950 kernels and the C ABI declared in include/mxq.h.
//
// The online path of the DuQuant++ page ("DuQuant++: block-aligned rotation
// quantization for MXFP4 activation outliers"): X * Lambda^-1 * R with R block
// diagonal (one shared 32x32 block, sec. 3.2-3.3), followed by MXFP4 encoding
// of every 32-element group (sec. 2.1), in a single pass over HBM (the fused
// operator of sec. 5.2 item 1 and sec. 5.4 item 3, extended with the
// quantization).
//
// Work decomposition.  A tile is 32 consecutive groups (1024 channels) of one
// token row; one wave64 owns a tile at a time.  Lane l handles group j = l % 32
// of the tile and half h = l / 32 of it.  The grid is persistent: each wave
// keeps one tile column (so its lambda values stay in registers) and walks
// down the rows with a fixed row step, prefetching the next batch of rows
// while it computes the current one.
//
// Rotation on the matrix cores (sec. 3.3 asks for the small dense product to
// run on matrix hardware, and the pitfalls list, item 4, for a batched GEMM
// over the [..., groups, 32] view rather than one big sparse product).  Per
// tile we form Y^T = R^T X^T with v_mfma_f32_32x32x16_bf16, twice (k = 0..15,
// 16..31):
//   A operand = R^T with its rows permuted, register-resident for the kernel;
//   B operand = the tile's activations, lane l supplying group l % 32 and
//               channels 16 s + 8 h + (0..7) in step s -- exactly the two
//               16-byte loads the lane makes;
//   D         = lane (j, h), register r holds y[group j][16 h + r], because
//               row i of A carries output channel pi(i), where the MFMA result
//               layout puts row 8 (r / 4) + 4 h + (r % 4) in lane half h,
//               register r.
// So each lane ends with 16 contiguous rotated values of one group: the group
// maximum is an in-lane max plus one v_permlane32_swap, and the lane packs 8
// contiguous code bytes for a single 8-byte store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/mxq.h"
#include "mxq_device.h"

#ifndef MXQ_WAVES_PER_CU
#define MXQ_WAVES_PER_CU 16
#endif
#ifndef MXQ_BATCH
#define MXQ_BATCH 2
#endif

namespace mxq {

constexpr int kGroup = 32;
constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlockThreads = kWave * kWavesPerBlock;
constexpr int kBatch = MXQ_BATCH;  // rows in flight per wave

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
    int32_t tcols;    // tile columns = ceil(gpr / 32)
    int32_t row_step; // waves per tile column
    int32_t waves;    // tcols * row_step
};

// Output channel carried by row i of the A operand (see file comment).
__device__ __forceinline__ int a_row_channel(int i) {
    return ((i >> 2) & 1) * 16 + (i >> 3) * 4 + (i & 3);
}

template <int XT, int MODE>
struct Loads {
    // 16-byte loads per lane per tile and their element offsets in the row.
    static constexpr int kN = (XT == kFP32) ? 4 : 2;
    __device__ static int64_t base(int p, int h) {
        return static_cast<int64_t>(p) * kGroup + (MODE == kRotate ? 8 * h : 16 * h);
    }
    __device__ static int step(int s) {
        if constexpr (MODE == kRotate) return 16 * s;
        else if constexpr (XT == kFP32) return 4 * s;
        else return 8 * s;
    }
};

template <int XT, int MODE, bool LAM, bool YOUT>
__global__ __launch_bounds__(kBlockThreads) void quant_kernel(Args a) {
    using L = Loads<XT, MODE>;
    constexpr int kN = L::kN;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int w = static_cast<int>(blockIdx.x) * kWavesPerBlock + wave;
    if (w >= a.waves) return;
    const int tc = w % a.tcols;
    const int64_t r0 = w / a.tcols;
    const int64_t rs = a.row_step;
    const int j = lane & 31;
    const int h = lane >> 5;
    const int p = tc * kGroup + j;  // group index within the row
    const bool valid = p < a.gpr;

    // Rotation block as the MFMA A operand (two k-halves), bf16 bits.
    bf16x8_t A0, A1;
    if constexpr (MODE == kRotate) {
        const int n = a_row_channel(j);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            A0[t] = __builtin_bit_cast(__bf16, a.r_hat[(8 * h + t) * kGroup + n]);
            A1[t] = __builtin_bit_cast(__bf16, a.r_hat[(16 + 8 * h + t) * kGroup + n]);
        }
    }
    // 1 / lambda for the 16 channels this lane feeds (fixed tile column).
    float il[16];
    if constexpr (LAM) {
        const int64_t c0 = L::base(p, h);
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int t = 0; t < 8; ++t)
                il[8 * s + t] = valid ? 1.0f / a.lambda[c0 + 16 * s + t] : 0.0f;
    }

    const char* xb = static_cast<const char*>(a.x);
    constexpr int esz = (XT == kFP32) ? 4 : 2;
    const int64_t lane_off = L::base(p, h);

    auto load_rows = [&](u32x4_t (&buf)[kBatch][kN], int64_t r) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t rr = r + u * rs;
#pragma unroll
            for (int s = 0; s < kN; ++s) buf[u][s] = u32x4_t{0u, 0u, 0u, 0u};
            if (rr < a.tokens && valid) {
                const char* row = xb + (rr * a.stride + lane_off) * esz;
#pragma unroll
                for (int s = 0; s < kN; ++s)
                    buf[u][s] = *reinterpret_cast<const u32x4_t*>(row + static_cast<int64_t>(L::step(s)) * esz);
            }
        }
    };

    u32x4_t buf[kBatch][kN];
    load_rows(buf, r0);
    for (int64_t r = r0; r < a.tokens; r += kBatch * rs) {
        u32x4_t cur[kBatch][kN];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int s = 0; s < kN; ++s) cur[u][s] = buf[u][s];
        const int64_t rn = r + kBatch * rs;
        if (rn < a.tokens) load_rows(buf, rn);

#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t rr = r + u * rs;
            if (rr >= a.tokens) break;
            float v[16];
            if constexpr (MODE == kRotate) {
                f32x16_t acc = {};
                if constexpr (XT == kBF16 && !LAM) {
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, __builtin_bit_cast(bf16x8_t, cur[u][0]), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, __builtin_bit_cast(bf16x8_t, cur[u][1]), acc, 0, 0, 0);
                } else {
                    // x' in fp32, then exact bf16 terms: 2 for fp16 x (11-bit
                    // significand), 3 for x * (1/lambda) (24-bit significand).
                    float f[16];
                    widen8<XT == kFP16>(cur[u][0], f);
                    widen8<XT == kFP16>(cur[u][1], f + 8);
                    if constexpr (LAM) {
#pragma unroll
                        for (int t = 0; t < 16; ++t) f[t] *= il[t];
                    }
                    constexpr int kTerms = LAM ? 3 : 2;
#pragma unroll
                    for (int term = 0; term < kTerms; ++term) {
                        u32x4_t b0, b1;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            b0[i] = bf16_pair_hi(f[2 * i], f[2 * i + 1]);
                            b1[i] = bf16_pair_hi(f[8 + 2 * i], f[8 + 2 * i + 1]);
                        }
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, __builtin_bit_cast(bf16x8_t, b0), acc, 0, 0, 0);
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, __builtin_bit_cast(bf16x8_t, b1), acc, 0, 0, 0);
                        if (term + 1 < kTerms) {
#pragma unroll
                            for (int t = 0; t < 16; ++t) f[t] = bf16_residual(f[t]);
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < 16; ++t) v[t] = acc[t];
            } else {
                if constexpr (XT == kFP32) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) widen4_f32(cur[u][s], v + 4 * s);
                } else {
                    widen8<XT == kFP16>(cur[u][0], v);
                    widen8<XT == kFP16>(cur[u][1], v + 8);
                }
            }

            const float m = group_amax(v);
            const uint32_t S = e8m0_of_amax(m);
            const float scale = as_f32(S << 23);
            const uint32_t lo = encode8(v, scale);
            const uint32_t hi = encode8(v + 8, scale);
            if (valid) {
                const int64_t g = rr * a.gpr + p;
                *reinterpret_cast<u32x2_t*>(a.codes + g * 16 + 8 * h) = u32x2_t{lo, hi};
                if (h == 0) a.scales[g] = static_cast<uint8_t>(S);
                if constexpr (YOUT) {
                    float* yp = a.y + g * kGroup + 16 * h;
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        *reinterpret_cast<float4*>(yp + 4 * s) = float4{v[4 * s], v[4 * s + 1], v[4 * s + 2], v[4 * s + 3]};
                }
            }
        }
    }
}

// Decode: one lane per half group (16 codes, one 8-byte load).
template <bool OUT_BF16>
__global__ __launch_bounds__(kBlockThreads) void dequant_kernel(const uint8_t* codes, const uint8_t* scales,
                                                               void* y, int64_t halves) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; q < halves; q += stride) {
        const int64_t g = q >> 1;
        const u32x2_t c = *reinterpret_cast<const u32x2_t*>(codes + q * 8);
        const int S = scales[g];
        uint32_t out[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t code = (c[i >> 3] >> (4 * (i & 7))) & 0xfu;
            const uint32_t mag = code & 7u;
            // E2M1 magnitude as fp32: codes 2..7 are 2^(mag/2 - 1) * (1 + (mag & 1) / 2),
            // whose fp32 pattern is (mag + 252) << 22; code 1 is 0.5, code 0 is 0.
            const uint32_t bits = mag >= 2u ? (mag + 252u) << 22 : (mag == 1u ? 0x3f000000u : 0u);
            float v = __builtin_amdgcn_ldexpf(as_f32(bits), S - 127);
            uint32_t u = as_u32(v) | ((code & 8u) << 28);
            if (S == 255) u = 0x7fc00000u;
            out[i] = u;
        }
        if constexpr (OUT_BF16) {
            u32x4_t o0, o1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                o0[i] = (out[2 * i] >> 16) | (out[2 * i + 1] & 0xffff0000u);
                o1[i] = (out[8 + 2 * i] >> 16) | (out[8 + 2 * i + 1] & 0xffff0000u);
            }
            u32x4_t* yp = reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(y) + q * 16);
            yp[0] = o0;
            yp[1] = o1;
        } else {
            u32x4_t* yp = reinterpret_cast<u32x4_t*>(static_cast<float*>(y) + q * 16);
#pragma unroll
            for (int s = 0; s < 4; ++s) yp[s] = u32x4_t{out[4 * s], out[4 * s + 1], out[4 * s + 2], out[4 * s + 3]};
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.

struct Plan {
    int32_t blocks, waves, tcols, row_step;
};

constexpr int64_t kMaxI32 = 2147483647;

// Grid for tokens x channels on cu_count CUs.  Target: MXQ_WAVES_PER_CU
// resident waves per CU.  Waves share a tile column in groups of row_step;
// among row steps between half and all of the target, pick the one whose
// last round of rows leaves the fewest waves idle.
static bool make_plan(int64_t tokens, int64_t channels, int cu_count, Plan* out) {
    if (tokens <= 0 || channels <= 0 || channels % kGroup) return false;
    if (tokens > kMaxI32 || channels > kMaxI32 - kGroup) return false;
    const int64_t gpr = channels / kGroup;
    const int64_t tcols = (gpr + kGroup - 1) / kGroup;
    if (tokens * tcols > kMaxI32) return false;
    const int64_t target = static_cast<int64_t>(cu_count > 0 ? cu_count : 1) * MXQ_WAVES_PER_CU;
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

// Compute-unit count of the current device, queried once per device.
static int device_cu_count() {
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

template <int XT, int MODE, bool LAM, bool YOUT>
static mxq_status launch(const Plan& pl, const Args& a, hipStream_t st) {
    hipLaunchKernelGGL((quant_kernel<XT, MODE, LAM, YOUT>), dim3(pl.blocks), dim3(kBlockThreads), 0, st, a);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

template <int XT>
static mxq_status dispatch_rotate(const Plan& pl, const Args& a, hipStream_t st) {
    if (a.lambda) {
        return a.y ? launch<XT, kRotate, true, true>(pl, a, st) : launch<XT, kRotate, true, false>(pl, a, st);
    }
    return a.y ? launch<XT, kRotate, false, true>(pl, a, st) : launch<XT, kRotate, false, false>(pl, a, st);
}

static mxq_status check_common(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                               int64_t stride, bool allow_fp32) {
    if (x_dtype != MXQ_BF16 && x_dtype != MXQ_FP16 && !(allow_fp32 && x_dtype == MXQ_FP32)) return MXQ_ERR_DTYPE;
    if (tokens < 0 || channels < 0 || channels % kGroup) return MXQ_ERR_SHAPE;
    (void)x;
    (void)stride;
    return MXQ_OK;
}

static mxq_status rotate_impl(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                              int64_t stride, const float* lambda, const uint16_t* r_hat, uint8_t* codes,
                              uint8_t* scales, float* y, void* stream) {
    mxq_status s = check_common(x, x_dtype, tokens, channels, stride, false);
    if (s != MXQ_OK) return s;
    if (tokens == 0 || channels == 0) return MXQ_OK;
    if (!x || !r_hat || !codes || !scales) return MXQ_ERR_NULL;
    if (stride < channels) return MXQ_ERR_STRIDE;
    if (!aligned(x, 16) || (stride * 2) % 16 || !aligned(codes, 16) || !aligned(r_hat, 2) ||
        (lambda && !aligned(lambda, 16)) || (y && !aligned(y, 16)))
        return MXQ_ERR_ALIGN;
    Plan pl;
    if (!make_plan(tokens, channels, device_cu_count(), &pl)) return MXQ_ERR_SHAPE;
    Args a{x, stride, lambda, r_hat, codes, scales, y, static_cast<int32_t>(tokens),
           static_cast<int32_t>(channels / kGroup), pl.tcols, pl.row_step, pl.waves};
    hipStream_t st = static_cast<hipStream_t>(stream);
    return x_dtype == MXQ_BF16 ? dispatch_rotate<kBF16>(pl, a, st) : dispatch_rotate<kFP16>(pl, a, st);
}

}  // namespace mxq

using namespace mxq;

extern "C" {

mxq_status mxq_rotate_quant(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                            int64_t x_row_stride, const float* lambda, const uint16_t* r_hat,
                            uint8_t* codes, uint8_t* scales, void* stream) {
    return rotate_impl(x, x_dtype, tokens, channels, x_row_stride, lambda, r_hat, codes, scales, nullptr,
                       stream);
}

mxq_status mxq_rotate_quant_ex(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                               int64_t x_row_stride, const float* lambda, const uint16_t* r_hat,
                               uint8_t* codes, uint8_t* scales, float* y_rot, void* stream) {
    return rotate_impl(x, x_dtype, tokens, channels, x_row_stride, lambda, r_hat, codes, scales, y_rot,
                       stream);
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
    Plan pl;
    if (!make_plan(tokens, channels, device_cu_count(), &pl)) return MXQ_ERR_SHAPE;
    Args a{x, x_row_stride, nullptr, nullptr, codes, scales, nullptr, static_cast<int32_t>(tokens),
           static_cast<int32_t>(channels / kGroup), pl.tcols, pl.row_step, pl.waves};
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (x_dtype) {
        case MXQ_BF16: return launch<kBF16, kQuant, false, false>(pl, a, st);
        case MXQ_FP16: return launch<kFP16, kQuant, false, false>(pl, a, st);
        default: return launch<kFP32, kQuant, false, false>(pl, a, st);
    }
}

mxq_status mxq_dequant(const uint8_t* codes, const uint8_t* scales, int64_t tokens, int64_t channels, void* y,
                       int32_t y_dtype, void* stream) {
    if (y_dtype != MXQ_BF16 && y_dtype != MXQ_FP32) return MXQ_ERR_DTYPE;
    if (tokens < 0 || channels < 0 || channels % kGroup) return MXQ_ERR_SHAPE;
    if (tokens == 0 || channels == 0) return MXQ_OK;
    if (tokens > kMaxI32 || channels > kMaxI32 - kGroup) return MXQ_ERR_SHAPE;
    if (!codes || !scales || !y) return MXQ_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(y, 16)) return MXQ_ERR_ALIGN;
    const int64_t halves = tokens * (channels / kGroup) * 2;
    int64_t blocks = (halves + kBlockThreads - 1) / kBlockThreads;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * 32;
    if (blocks > cap) blocks = cap;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (y_dtype == MXQ_BF16)
        hipLaunchKernelGGL((dequant_kernel<true>), dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads), 0, st,
                           codes, scales, y, halves);
    else
        hipLaunchKernelGGL((dequant_kernel<false>), dim3(static_cast<unsigned>(blocks)), dim3(kBlockThreads), 0, st,
                           codes, scales, y, halves);
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
    if (!make_plan(tokens, channels, cu_count, &pl)) return MXQ_ERR_SHAPE;
    out[0] = pl.blocks;
    out[1] = pl.waves;
    out[2] = pl.tcols;
    out[3] = pl.row_step;
    out[4] = kWavesPerBlock;
    return MXQ_OK;
}

int32_t mxq_version(void) { return 1; }

}  // extern "C"
