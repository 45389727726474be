// Offline calibration of the shared 32x32 rotation block on gfx950, in fp64.
//
// DuQuant++ page ("DuQuant++: block-aligned rotation quantization for MXFP4
// activation outliers"), sec. 3.2: pick the 32-channel group of the (smoothed,
// sec. 5.1 item 3) calibration activations with the largest L-infinity norm
// (X_worst, all calibration tokens of that group), then grow a rotation
// greedily: at each of up to 128 steps take the dimension d holding the
// largest |value|, try a Givens rotation of d with each of the other 31
// dimensions, and keep the one that leaves the smallest L-infinity norm.  The
// page asks for double precision (sec. 3 pitfalls, item 3); every product and
// sum below is a separately rounded fp64 operation (no contraction), in a
// fixed order, so the result is reproducible bit for bit.
//
// Readings where the page is silent: a Givens rotation by theta maps
// (x_d, x_j) to (c x_d - s x_j, s x_d + c x_j), c = cos theta, s = sin theta.
// The angle is pi/4 for every candidate (mxq_calib_givens), or each candidate
// also picks the best angle of a fixed grid (mxq_calib_givens_angles): pi/4,
// then the angles with tan(theta / 2) = k / M, k = 1 .. M - 1, whose
// c = (M^2 - k^2) / (M^2 + k^2) and s = 2 k M / (M^2 + k^2) are correctly
// rounded divisions of exact integers (the half-angle substitution), so no
// trigonometric function enters.  The norm has period pi/2 in theta, so the
// grid spans (0, pi/2).  Ties go to the lowest column / candidate / grid
// angle / group index; a step is taken while the best candidate does not
// raise the norm, and the search stops when every candidate would raise it
// or X_worst is zero.
//
// Work layout.  X_worst is [T][32] fp64 (256 bytes per token).  In the scan
// kernel lane l of a wave holds column l % 32 of token 2 p + l / 32, so one
// load instruction reads two whole tokens (512 bytes).  Each step is a scan
// launch over all tokens (apply the previous step's rotation in place, and
// for the current d accumulate, per candidate j, the maxima of both rotated
// columns) followed by a one-block decide launch.  Because the maxima of the
// two rotated columns are exactly the new column maxima of the chosen
// candidate, one pass over X_worst per step suffices.  With an angle grid a
// step is three launches: apply the previous step's rotation, scan every
// (candidate, angle) pair (blockIdx.y picks a chunk of kAngChunk angles; the
// per-block maxima meet in an array by atomic max, which is order-free), and
// decide.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/mxq.h"
#include "mxq_device.h"
#include "mxq_internal.h"

#pragma clang fp contract(off)

namespace mxq {
namespace calib {

constexpr int kW = 32;               // block width
constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWave * kWavesPerBlock;
constexpr int kUnroll = 8;           // token pairs per scan iteration
constexpr int kSlices = 32;          // decide kernel: threads per candidate
constexpr double kC = 0x1.6a09e667f3bcdp-1;  // sqrt(1/2), correctly rounded
constexpr double kS = 0x1.6a09e667f3bcdp-1;
constexpr int kMaxAngles = 1024;     // largest angle grid
constexpr int kAngChunk = 8;         // angles per block of the angle scan
constexpr int kAngUnroll = 4;        // token pairs per angle-scan iteration

struct State {
    int32_t d;           // dimension holding the current maximum
    int32_t pd, pj;      // rotation accepted but not yet applied to X_worst (-1: none)
    int32_t steps_done;
    int32_t stopped;
    int32_t pa;          // grid index of the pending rotation's angle
    double linf;
    double pc, ps;       // cos and sin of the pending rotation
    double colmax[kW];
};

__device__ __forceinline__ double shfl_d(double v, int src) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(u & 0xffffffffu));
    const int hi = __builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(u >> 32));
    return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                          static_cast<uint32_t>(lo));
}

// ---- worst group ----------------------------------------------------------

__global__ void fill_u64(uint64_t* p, int64_t n, uint64_t v) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

// |x / lambda| maxima per group.  Thread layout: one thread per (token, group)
// pair within a grid-stride loop; each thread reads its group's 32 values of
// one token (64 or 128 bytes), so a wave covers 64 consecutive groups.
template <int XT, bool LAM>
__global__ __launch_bounds__(kThreads) void group_max_kernel(const void* x, int64_t stride, const float* lambda,
                                                            int64_t tokens, int64_t gpr, uint64_t* gmax) {
    const int64_t total = tokens * gpr;
    const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += step) {
        const int64_t t = i / gpr;
        const int64_t g = i - t * gpr;
        double m = 0.0;
        for (int k = 0; k < kW; ++k) {
            const int64_t c = g * kW + k;
            double v;
            if constexpr (XT == MXQ_BF16) {
                const uint16_t b = static_cast<const uint16_t*>(x)[t * stride + c];
                v = static_cast<double>(as_f32(static_cast<uint32_t>(b) << 16));
            } else if constexpr (XT == MXQ_FP16) {
                const uint16_t b = static_cast<const uint16_t*>(x)[t * stride + c];
                v = static_cast<double>(static_cast<float>(__builtin_bit_cast(_Float16, b)));
            } else {
                v = static_cast<double>(static_cast<const float*>(x)[t * stride + c]);
            }
            if constexpr (LAM) v = v / static_cast<double>(lambda[c]);
            const double a = fabs(v);
            m = a > m ? a : m;
        }
        // non-negative doubles order like their bit patterns
        atomicMax(reinterpret_cast<unsigned long long*>(gmax + g),
                  static_cast<unsigned long long>(__builtin_bit_cast(uint64_t, m)));
    }
}

// First group with the largest maximum (one block).
__global__ void pick_group_kernel(const uint64_t* gmax, int64_t gpr, int64_t* group, double* linf) {
    __shared__ uint64_t best_v[kThreads];
    __shared__ int64_t best_i[kThreads];
    uint64_t bv = 0;
    int64_t bi = 0;
    bool have = false;
    for (int64_t g = threadIdx.x; g < gpr; g += blockDim.x) {
        const uint64_t v = gmax[g];
        if (!have || v > bv) {
            bv = v;
            bi = g;
            have = true;
        }
    }
    best_v[threadIdx.x] = have ? bv : 0;
    best_i[threadIdx.x] = have ? bi : INT64_MAX;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t v = 0;
        int64_t i = INT64_MAX;
        for (int k = 0; k < static_cast<int>(blockDim.x); ++k) {
            if (best_i[k] == INT64_MAX) continue;
            if (i == INT64_MAX || best_v[k] > v || (best_v[k] == v && best_i[k] < i)) {
                v = best_v[k];
                i = best_i[k];
            }
        }
        *group = i;
        *linf = __builtin_bit_cast(double, v);
    }
}

template <int XT, bool LAM>
__global__ __launch_bounds__(kThreads) void extract_kernel(const void* x, int64_t stride, const float* lambda,
                                                          int64_t tokens, const int64_t* group, double* xw) {
    const int64_t g = *group;
    const int64_t total = tokens * kW;
    const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += step) {
        const int64_t t = i / kW;
        const int64_t c = g * kW + (i - t * kW);
        double v;
        if constexpr (XT == MXQ_BF16) {
            v = static_cast<double>(as_f32(static_cast<uint32_t>(static_cast<const uint16_t*>(x)[t * stride + c]) << 16));
        } else if constexpr (XT == MXQ_FP16) {
            v = static_cast<double>(
                static_cast<float>(__builtin_bit_cast(_Float16, static_cast<const uint16_t*>(x)[t * stride + c])));
        } else {
            v = static_cast<double>(static_cast<const float*>(x)[t * stride + c]);
        }
        if constexpr (LAM) v = v / static_cast<double>(lambda[c]);
        xw[i] = v;
    }
}

// ---- greedy Givens search --------------------------------------------------

enum : int { kModeInit = 0, kModeStep = 1, kModeApply = 2 };

// One pass over X_worst.  Apply the pending rotation (pd, pj) in place, then
// (kModeStep) for the current d accumulate per candidate j the maxima of
// |c x_d - s x_j| and |s x_d + c x_j|, or (kModeInit) the column maxima.
// Per-block partial maxima go to partials[block][32][2].
template <int MODE>
__global__ __launch_bounds__(kThreads) void scan_kernel(double* xw, int64_t tokens, const State* st,
                                                       double* partials) {
    __shared__ double red[kWavesPerBlock][kW][2];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int k = lane & (kW - 1);
    const int half = lane >> 5;
    int pd = -1, pj = -1, d = 0;
    if (MODE != kModeInit) {
        if (st->stopped && st->pd < 0) return;  // nothing left to do (uniform for the grid)
        pd = st->pd;
        pj = st->pj;
        d = st->d;
        if (MODE == kModeApply && pd < 0) return;
    }
    const double pc = MODE != kModeInit ? st->pc : 0.0;
    const double ps = MODE != kModeInit ? st->ps : 0.0;
    const bool eval = MODE == kModeStep && !st->stopped;
    double m1 = 0.0, m2 = 0.0;
    const int64_t pairs = (tokens + 1) / 2;
    const int64_t wstep = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
    // kUnroll token pairs per iteration, all loads issued before any is used
    for (int64_t p0 = (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave) * kUnroll; p0 < pairs;
         p0 += wstep * kUnroll) {
        double v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t t = 2 * (p0 + u) + half;
            v[u] = t < tokens ? xw[t * kW + k] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t t = 2 * (p0 + u) + half;
            const bool row_ok = t < tokens;
            if (pd >= 0) {
                const double xd = shfl_d(v[u], pd + kW * half);
                const double xj = shfl_d(v[u], pj + kW * half);
                if (k == pd) v[u] = pc * xd - ps * xj;
                if (k == pj) v[u] = ps * xd + pc * xj;
                if (row_ok && (k == pd || k == pj)) xw[t * kW + k] = v[u];
            }
            if (MODE == kModeInit) {
                const double a = fabs(v[u]);
                m1 = a > m1 ? a : m1;
            } else if (eval) {
                const double xd = shfl_d(v[u], d + kW * half);
                if (row_ok && k != d) {
                    const double a1 = fabs(kC * xd - kS * v[u]);
                    const double a2 = fabs(kS * xd + kC * v[u]);
                    m1 = a1 > m1 ? a1 : m1;
                    m2 = a2 > m2 ? a2 : m2;
                }
            }
        }
    }
    if (MODE == kModeApply) return;
    // combine the two token halves of the wave, then the waves of the block
    const double o1 = shfl_d(m1, lane ^ 32);
    const double o2 = shfl_d(m2, lane ^ 32);
    m1 = o1 > m1 ? o1 : m1;
    m2 = o2 > m2 ? o2 : m2;
    if (half == 0) {
        red[wave][k][0] = m1;
        red[wave][k][1] = m2;
    }
    __syncthreads();
    if (threadIdx.x < kW) {
        double a = red[0][threadIdx.x][0], b = red[0][threadIdx.x][1];
        for (int w = 1; w < kWavesPerBlock; ++w) {
            a = red[w][threadIdx.x][0] > a ? red[w][threadIdx.x][0] : a;
            b = red[w][threadIdx.x][1] > b ? red[w][threadIdx.x][1] : b;
        }
        partials[(static_cast<int64_t>(blockIdx.x) * kW + threadIdx.x) * 2] = a;
        partials[(static_cast<int64_t>(blockIdx.x) * kW + threadIdx.x) * 2 + 1] = b;
    }
}

// One block of 32 x 32 threads: thread (slice, j) reduces every 32nd block's
// partial maxima of candidate j, slice 0 combines the slices, and thread 0
// takes (or refuses) the step and writes the scalar state.  Values shared
// between threads go through LDS.
template <int MODE>
__global__ __launch_bounds__(kW * kSlices) void decide_kernel(State* st, const double* partials, int nblocks,
                                                             double* r, double* history, int32_t* pairs_out,
                                                             int32_t* steps_done) {
    __shared__ double M1[kW], M2[kW], cm[kW];
    __shared__ double part[kSlices][kW][2];
    __shared__ int acc_d, acc_j;  // accepted pair (acc_j < 0: none)
    const int j = threadIdx.x & (kW - 1);
    const int slice = threadIdx.x / kW;
    if (MODE == kModeStep && st->stopped) return;  // uniform
    double a = 0.0, b = 0.0;
    for (int blk = slice; blk < nblocks; blk += kSlices) {
        const double pa = partials[(static_cast<int64_t>(blk) * kW + j) * 2];
        const double pb = partials[(static_cast<int64_t>(blk) * kW + j) * 2 + 1];
        a = pa > a ? pa : a;
        b = pb > b ? pb : b;
    }
    part[slice][j][0] = a;
    part[slice][j][1] = b;
    __syncthreads();
    if (slice == 0) {
        for (int sl = 1; sl < kSlices; ++sl) {
            a = part[sl][j][0] > a ? part[sl][j][0] : a;
            b = part[sl][j][1] > b ? part[sl][j][1] : b;
        }
        M1[j] = a;
        M2[j] = b;
        cm[j] = MODE == kModeInit ? a : st->colmax[j];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        acc_j = -1;
        if (MODE == kModeInit) {
            double m = 0.0;
            int dd = 0;
            for (int c = 0; c < kW; ++c)
                if (cm[c] > m) {
                    m = cm[c];
                    dd = c;
                }
            st->linf = m;
            st->d = dd;
            st->pd = -1;
            st->pj = -1;
            st->pa = 0;
            st->pc = kC;
            st->ps = kS;
            st->steps_done = 0;
            st->stopped = m == 0.0;
            history[0] = m;
            *steps_done = 0;
        } else {
            const int d = st->d;
            const double linf = st->linf;
            double best = 0.0;
            int bj = -1;
            if (linf > 0.0) {
                for (int c = 0; c < kW; ++c) {
                    if (c == d) continue;
                    double rest = 0.0;
                    for (int k2 = 0; k2 < kW; ++k2)
                        if (k2 != d && k2 != c && cm[k2] > rest) rest = cm[k2];
                    double norm = M1[c] > M2[c] ? M1[c] : M2[c];
                    norm = rest > norm ? rest : norm;
                    if (bj < 0 || norm < best) {
                        best = norm;
                        bj = c;
                    }
                }
            }
            if (bj < 0 || best > linf) {  // zero block, or every candidate raises the norm
                st->stopped = 1;
                st->pd = -1;
                st->pj = -1;
            } else {
                cm[d] = M1[bj];
                cm[bj] = M2[bj];
                double m = 0.0;
                int dd = 0;
                for (int c = 0; c < kW; ++c)
                    if (cm[c] > m) {
                        m = cm[c];
                        dd = c;
                    }
                const int s = st->steps_done;
                history[s + 1] = m;
                if (pairs_out) {
                    pairs_out[2 * s] = d;
                    pairs_out[2 * s + 1] = bj;
                }
                st->linf = m;
                st->pd = d;
                st->pj = bj;
                st->d = dd;
                st->steps_done = s + 1;
                *steps_done = s + 1;
                acc_d = d;
                acc_j = bj;
            }
        }
    }
    __syncthreads();
    if (slice != 0) return;
    st->colmax[j] = cm[j];
    if (MODE == kModeInit) {
        for (int i = 0; i < kW; ++i) r[i * kW + j] = (i == j) ? 1.0 : 0.0;
    } else if (acc_j >= 0) {
        // R <- R G: columns d and j of row `j` (thread j owns row j)
        const int d = acc_d, c = acc_j;
        const double rd = r[j * kW + d], rc = r[j * kW + c];
        r[j * kW + d] = kC * rd - kS * rc;
        r[j * kW + c] = kS * rd + kC * rc;
    }
}

// ---- greedy search with a per-candidate angle -------------------------------

// (c, s) of the angle grid, index 0 = pi/4, index k = tan(theta / 2) = k / M.
// Integers below 2^21 and their products are exact in fp64; each quotient is
// one correctly rounded division.
__global__ void angle_table_kernel(double* table, int grid) {
    const int k = static_cast<int>(blockIdx.x * blockDim.x + threadIdx.x);
    if (k >= grid) return;
    double c = kC, s = kS;
    if (k > 0) {
        const double m = static_cast<double>(grid), kk = static_cast<double>(k);
        const double den = m * m + kk * kk;
        c = (m * m - kk * kk) / den;
        s = (2.0 * kk * m) / den;
    }
    table[2 * k] = c;
    table[2 * k + 1] = s;
}

// For the current d and the grid angles a0 .. a0 + kAngChunk - 1 (a0 =
// blockIdx.y * kAngChunk), the maxima over this block's tokens of
// |c x_d - s x_j| and |s x_d + c x_j| for every j != d, merged into
// acc[j][a][2] (bit patterns of non-negative doubles, which order like the
// values) by atomic max.  Lane layout as scan_kernel: lane l holds column
// l % 32 of token 2 p + l / 32.
__global__ __launch_bounds__(kThreads) void scan_angles_kernel(const double* xw, int64_t tokens, const State* st,
                                                              const double* table, int nang, uint64_t* acc) {
    __shared__ double red[kWavesPerBlock][2][kAngChunk][kW];
    if (st->stopped) return;  // uniform for the grid
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int k = lane & (kW - 1);
    const int half = lane >> 5;
    const int d = st->d;
    const int a0 = static_cast<int>(blockIdx.y) * kAngChunk;
    double cc[kAngChunk], ss[kAngChunk], m1[kAngChunk], m2[kAngChunk];
#pragma unroll
    for (int a = 0; a < kAngChunk; ++a) {
        const int idx = a0 + a < nang ? a0 + a : nang - 1;  // past the grid: repeats, not merged
        cc[a] = table[2 * idx];
        ss[a] = table[2 * idx + 1];
        m1[a] = 0.0;
        m2[a] = 0.0;
    }
    const int64_t pairs = (tokens + 1) / 2;
    const int64_t wstep = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
    for (int64_t p0 = (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave) * kAngUnroll; p0 < pairs;
         p0 += wstep * kAngUnroll) {
        double v[kAngUnroll];
#pragma unroll
        for (int u = 0; u < kAngUnroll; ++u) {
            const int64_t t = 2 * (p0 + u) + half;
            v[u] = t < tokens ? xw[t * kW + k] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < kAngUnroll; ++u) {
            const int64_t t = 2 * (p0 + u) + half;
            const double xd = shfl_d(v[u], d + kW * half);
            if (t < tokens && k != d) {
#pragma unroll
                for (int a = 0; a < kAngChunk; ++a) {
                    const double a1 = fabs(cc[a] * xd - ss[a] * v[u]);
                    const double a2 = fabs(ss[a] * xd + cc[a] * v[u]);
                    m1[a] = a1 > m1[a] ? a1 : m1[a];
                    m2[a] = a2 > m2[a] ? a2 : m2[a];
                }
            }
        }
    }
#pragma unroll
    for (int a = 0; a < kAngChunk; ++a) {
        const double o1 = shfl_d(m1[a], lane ^ 32);
        const double o2 = shfl_d(m2[a], lane ^ 32);
        m1[a] = o1 > m1[a] ? o1 : m1[a];
        m2[a] = o2 > m2[a] ? o2 : m2[a];
        if (half == 0) {
            red[wave][0][a][k] = m1[a];
            red[wave][1][a][k] = m2[a];
        }
    }
    __syncthreads();
    static_assert(kAngChunk * kW == kThreads, "one thread per (angle, column) of the chunk");
    const int j = threadIdx.x & (kW - 1);
    const int a = threadIdx.x / kW;
    if (j == d || a0 + a >= nang) return;
    double b1 = red[0][0][a][j], b2 = red[0][1][a][j];
    for (int w = 1; w < kWavesPerBlock; ++w) {
        b1 = red[w][0][a][j] > b1 ? red[w][0][a][j] : b1;
        b2 = red[w][1][a][j] > b2 ? red[w][1][a][j] : b2;
    }
    uint64_t* dst = acc + (static_cast<int64_t>(j) * nang + a0 + a) * 2;
    atomicMax(reinterpret_cast<unsigned long long*>(dst), static_cast<unsigned long long>(__builtin_bit_cast(uint64_t, b1)));
    atomicMax(reinterpret_cast<unsigned long long*>(dst + 1),
              static_cast<unsigned long long>(__builtin_bit_cast(uint64_t, b2)));
}

// One block of 32 x 32 threads.  Thread (slice, j) reads (and clears, for the
// next step) the merged maxima of candidate j at angles slice, slice + 32, ...
// and keeps its best (smallest norm, then earliest angle); slice 0 reduces
// the slices per candidate, thread 0 the candidates (smallest norm, then
// lowest j), takes or refuses the step, and writes the scalar state; slice 0
// then updates R.
__global__ __launch_bounds__(kW * kSlices) void decide_angles_kernel(State* st, uint64_t* acc, const double* table,
                                                                    int nang, double* r, double* history,
                                                                    int32_t* pairs_out, int32_t* angles_out,
                                                                    int32_t* steps_done) {
    __shared__ double cm[kW];
    __shared__ double bn[kSlices][kW], b1[kSlices][kW], b2[kSlices][kW];
    __shared__ int ba[kSlices][kW];
    __shared__ int acc_d, acc_j;
    __shared__ double acc_c, acc_s;
    if (st->stopped) return;  // uniform
    const int j = threadIdx.x & (kW - 1);
    const int slice = threadIdx.x / kW;
    const int d = st->d;
    if (slice == 0) cm[j] = st->colmax[j];
    __syncthreads();
    double rest = 0.0;
    for (int k2 = 0; k2 < kW; ++k2)
        if (k2 != d && k2 != j && cm[k2] > rest) rest = cm[k2];
    double best = 0.0, bm1 = 0.0, bm2 = 0.0;
    int besta = -1;
#pragma unroll 1
    for (int a = slice; a < nang; a += kSlices) {
        uint64_t* p = acc + (static_cast<int64_t>(j) * nang + a) * 2;
        const double m1 = __builtin_bit_cast(double, p[0]);
        const double m2 = __builtin_bit_cast(double, p[1]);
        p[0] = 0;
        p[1] = 0;
        double norm = m1 > m2 ? m1 : m2;
        norm = rest > norm ? rest : norm;
        if (besta < 0 || norm < best) {
            best = norm;
            besta = a;
            bm1 = m1;
            bm2 = m2;
        }
    }
    bn[slice][j] = best;
    ba[slice][j] = j == d ? -1 : besta;
    b1[slice][j] = bm1;
    b2[slice][j] = bm2;
    __syncthreads();
    if (slice == 0) {  // best over the slices of candidate j: smallest norm, then earliest angle
#pragma unroll 1
        for (int sl = 1; sl < kSlices; ++sl) {
            const int a = ba[sl][j];
            if (a < 0) continue;
            if (ba[0][j] < 0 || bn[sl][j] < bn[0][j] || (bn[sl][j] == bn[0][j] && a < ba[0][j])) {
                bn[0][j] = bn[sl][j];
                ba[0][j] = a;
                b1[0][j] = b1[sl][j];
                b2[0][j] = b2[sl][j];
            }
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        acc_j = -1;
        const double linf = st->linf;
        double bnorm = 0.0;
        int bj = -1;
        if (linf > 0.0) {
            for (int c = 0; c < kW; ++c) {
                if (c == d || ba[0][c] < 0) continue;
                if (bj < 0 || bn[0][c] < bnorm) {
                    bnorm = bn[0][c];
                    bj = c;
                }
            }
        }
        if (bj < 0 || bnorm > linf) {  // zero block, or every candidate raises the norm
            st->stopped = 1;
            st->pd = -1;
            st->pj = -1;
        } else {
            const int a = ba[0][bj];
            cm[d] = b1[0][bj];
            cm[bj] = b2[0][bj];
            double m = 0.0;
            int dd = 0;
            for (int c = 0; c < kW; ++c)
                if (cm[c] > m) {
                    m = cm[c];
                    dd = c;
                }
            const int s = st->steps_done;
            history[s + 1] = m;
            if (pairs_out) {
                pairs_out[2 * s] = d;
                pairs_out[2 * s + 1] = bj;
            }
            if (angles_out) angles_out[s] = a;
            st->linf = m;
            st->pd = d;
            st->pj = bj;
            st->pa = a;
            st->pc = table[2 * a];
            st->ps = table[2 * a + 1];
            st->d = dd;
            st->steps_done = s + 1;
            *steps_done = s + 1;
            acc_d = d;
            acc_j = bj;
            acc_c = table[2 * a];
            acc_s = table[2 * a + 1];
        }
    }
    __syncthreads();
    if (slice != 0) return;
    st->colmax[j] = cm[j];
    if (acc_j >= 0) {
        // R <- R G: columns d and j of row `j` (thread j owns row j)
        const int dd = acc_d, c = acc_j;
        const double cs = acc_c, sn = acc_s;
        const double rd = r[j * kW + dd], rc = r[j * kW + c];
        r[j * kW + dd] = cs * rd - sn * rc;
        r[j * kW + c] = sn * rd + cs * rc;
    }
}

}  // namespace calib

// ---- host entry points ------------------------------------------------------

using calib::State;

static constexpr int64_t kCalibMaxBlocks = 1024;

static int64_t scan_blocks(int64_t tokens) {
    const int64_t pairs = (tokens + 1) / 2;
    const int64_t per_block = static_cast<int64_t>(calib::kWavesPerBlock) * calib::kUnroll;
    int64_t b = (pairs + per_block - 1) / per_block;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * 4;
    if (b > cap) b = cap;
    if (b > kCalibMaxBlocks) b = kCalibMaxBlocks;
    return b < 1 ? 1 : b;
}

static size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// Workspace layout: State | per-block partial maxima | angle table | merged
// (candidate, angle) maxima | per-group maxima of the worst-group scan.
static size_t ws_partials() { return align256(sizeof(State)); }
static size_t ws_table() {
    return ws_partials() + align256(static_cast<size_t>(kCalibMaxBlocks) * calib::kW * 2 * sizeof(double));
}
static size_t ws_acc() { return ws_table() + align256(static_cast<size_t>(calib::kMaxAngles) * 2 * sizeof(double)); }
static size_t ws_gmax() {
    return ws_acc() + align256(static_cast<size_t>(calib::kW) * calib::kMaxAngles * 2 * sizeof(uint64_t));
}

static size_t calib_workspace_bytes(int64_t channels) {
    const int64_t gpr = channels > 0 ? channels / calib::kW : 0;
    return ws_gmax() + align256(static_cast<size_t>(gpr) * sizeof(uint64_t));
}

template <int XT, bool LAM>
static void launch_worst(const void* x, int64_t stride, const float* lambda, int64_t tokens, int64_t gpr,
                         uint64_t* gmax, int64_t* group, double* linf, double* xw, hipStream_t st) {
    const int64_t fill_blocks = (gpr + 255) / 256;
    hipLaunchKernelGGL(calib::fill_u64, dim3(static_cast<unsigned>(fill_blocks)), dim3(256), 0, st, gmax, gpr,
                       uint64_t(0));
    int64_t blocks = (tokens * gpr + calib::kThreads - 1) / calib::kThreads;
    const int64_t cap = static_cast<int64_t>(device_cu_count()) * 16;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL((calib::group_max_kernel<XT, LAM>), dim3(static_cast<unsigned>(blocks)),
                       dim3(calib::kThreads), 0, st, x, stride, lambda, tokens, gpr, gmax);
    hipLaunchKernelGGL(calib::pick_group_kernel, dim3(1), dim3(calib::kThreads), 0, st, gmax, gpr, group, linf);
    int64_t eblocks = (tokens * calib::kW + calib::kThreads - 1) / calib::kThreads;
    if (eblocks > cap) eblocks = cap;
    hipLaunchKernelGGL((calib::extract_kernel<XT, LAM>), dim3(static_cast<unsigned>(eblocks)),
                       dim3(calib::kThreads), 0, st, x, stride, lambda, tokens, group, xw);
}

static mxq_status calib_worst_group(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels, int64_t stride,
                             const float* lambda, double* x_worst, int64_t* group, double* linf, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (x_dtype != MXQ_BF16 && x_dtype != MXQ_FP16 && x_dtype != MXQ_FP32) return MXQ_ERR_DTYPE;
    if (tokens <= 0 || channels <= 0 || channels % calib::kW || tokens > (int64_t(1) << 40) / channels)
        return MXQ_ERR_SHAPE;
    if (!x || !x_worst || !group || !linf || !workspace) return MXQ_ERR_NULL;
    if (stride < channels) return MXQ_ERR_STRIDE;
    if (workspace_bytes < calib_workspace_bytes(channels) || (reinterpret_cast<uintptr_t>(workspace) & 255) ||
        (reinterpret_cast<uintptr_t>(x_worst) & 7) || (reinterpret_cast<uintptr_t>(group) & 7) ||
        (reinterpret_cast<uintptr_t>(linf) & 7))
        return MXQ_ERR_ALIGN;
    const int64_t gpr = channels / calib::kW;
    char* ws = static_cast<char*>(workspace);
    uint64_t* gmax = reinterpret_cast<uint64_t*>(ws + ws_gmax());
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (x_dtype * 2 + (lambda ? 1 : 0)) {
        case MXQ_BF16 * 2: launch_worst<MXQ_BF16, false>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
        case MXQ_BF16 * 2 + 1: launch_worst<MXQ_BF16, true>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
        case MXQ_FP16 * 2: launch_worst<MXQ_FP16, false>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
        case MXQ_FP16 * 2 + 1: launch_worst<MXQ_FP16, true>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
        case MXQ_FP32 * 2: launch_worst<MXQ_FP32, false>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
        default: launch_worst<MXQ_FP32, true>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
    }
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

static mxq_status calib_givens(double* x_worst, int64_t tokens, int32_t max_steps, double* r, double* history,
                        int32_t* steps_done, int32_t* pairs, void* workspace, size_t workspace_bytes, void* stream) {
    if (tokens <= 0 || tokens > (int64_t(1) << 40) || max_steps < 0 || max_steps > 1000000) return MXQ_ERR_SHAPE;
    if (!x_worst || !r || !history || !steps_done || !workspace) return MXQ_ERR_NULL;
    if (workspace_bytes < calib_workspace_bytes(0) || (reinterpret_cast<uintptr_t>(workspace) & 255) ||
        (reinterpret_cast<uintptr_t>(x_worst) & 7) || (reinterpret_cast<uintptr_t>(r) & 7) ||
        (reinterpret_cast<uintptr_t>(history) & 7) || (reinterpret_cast<uintptr_t>(steps_done) & 3) ||
        (reinterpret_cast<uintptr_t>(pairs) & 3))
        return MXQ_ERR_ALIGN;
    char* ws = static_cast<char*>(workspace);
    State* state = reinterpret_cast<State*>(ws);
    double* partials = reinterpret_cast<double*>(ws + ws_partials());
    const int64_t nb = scan_blocks(tokens);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(static_cast<unsigned>(nb)), block(calib::kThreads);
    hipLaunchKernelGGL(calib::scan_kernel<calib::kModeInit>, grid, block, 0, st, x_worst, tokens, state, partials);
    const dim3 dblock(calib::kW * calib::kSlices);
    hipLaunchKernelGGL(calib::decide_kernel<calib::kModeInit>, dim3(1), dblock, 0, st, state, partials,
                       static_cast<int>(nb), r, history, pairs, steps_done);
    for (int32_t s = 0; s < max_steps; ++s) {
        hipLaunchKernelGGL(calib::scan_kernel<calib::kModeStep>, grid, block, 0, st, x_worst, tokens, state,
                           partials);
        hipLaunchKernelGGL(calib::decide_kernel<calib::kModeStep>, dim3(1), dblock, 0, st, state,
                           partials, static_cast<int>(nb), r, history, pairs, steps_done);
    }
    hipLaunchKernelGGL(calib::scan_kernel<calib::kModeApply>, grid, block, 0, st, x_worst, tokens, state, partials);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

static mxq_status calib_givens_angles(double* x_worst, int64_t tokens, int32_t max_steps, int32_t angle_grid,
                                      double* r, double* history, int32_t* steps_done, int32_t* pairs,
                                      int32_t* angles, void* workspace, size_t workspace_bytes, void* stream) {
    if (tokens <= 0 || tokens > (int64_t(1) << 40) || max_steps < 0 || max_steps > 1000000 || angle_grid < 1 ||
        angle_grid > calib::kMaxAngles)
        return MXQ_ERR_SHAPE;
    if (!x_worst || !r || !history || !steps_done || !workspace) return MXQ_ERR_NULL;
    if (workspace_bytes < calib_workspace_bytes(0) || (reinterpret_cast<uintptr_t>(workspace) & 255) ||
        (reinterpret_cast<uintptr_t>(x_worst) & 7) || (reinterpret_cast<uintptr_t>(r) & 7) ||
        (reinterpret_cast<uintptr_t>(history) & 7) || (reinterpret_cast<uintptr_t>(steps_done) & 3) ||
        (reinterpret_cast<uintptr_t>(pairs) & 3) || (reinterpret_cast<uintptr_t>(angles) & 3))
        return MXQ_ERR_ALIGN;
    char* ws = static_cast<char*>(workspace);
    State* state = reinterpret_cast<State*>(ws);
    double* partials = reinterpret_cast<double*>(ws + ws_partials());
    double* table = reinterpret_cast<double*>(ws + ws_table());
    uint64_t* acc = reinterpret_cast<uint64_t*>(ws + ws_acc());
    const int64_t nb = scan_blocks(tokens);
    const int chunks = (angle_grid + calib::kAngChunk - 1) / calib::kAngChunk;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const dim3 grid(static_cast<unsigned>(nb)), block(calib::kThreads);
    const dim3 agrid(static_cast<unsigned>(nb), static_cast<unsigned>(chunks));
    const dim3 dblock(calib::kW * calib::kSlices);
    const int64_t nacc = static_cast<int64_t>(calib::kW) * angle_grid * 2;
    hipLaunchKernelGGL(calib::fill_u64, dim3(static_cast<unsigned>((nacc + 255) / 256)), dim3(256), 0, st, acc, nacc,
                       uint64_t(0));
    hipLaunchKernelGGL(calib::angle_table_kernel, dim3(static_cast<unsigned>((angle_grid + 255) / 256)), dim3(256), 0,
                       st, table, angle_grid);
    hipLaunchKernelGGL(calib::scan_kernel<calib::kModeInit>, grid, block, 0, st, x_worst, tokens, state, partials);
    hipLaunchKernelGGL(calib::decide_kernel<calib::kModeInit>, dim3(1), dblock, 0, st, state, partials,
                       static_cast<int>(nb), r, history, pairs, steps_done);
    for (int32_t s = 0; s < max_steps; ++s) {
        hipLaunchKernelGGL(calib::scan_kernel<calib::kModeApply>, grid, block, 0, st, x_worst, tokens, state,
                           partials);
        hipLaunchKernelGGL(calib::scan_angles_kernel, agrid, block, 0, st, x_worst, tokens, state, table,
                           angle_grid, acc);
        hipLaunchKernelGGL(calib::decide_angles_kernel, dim3(1), dblock, 0, st, state, acc, table, angle_grid, r,
                           history, pairs, angles, steps_done);
    }
    hipLaunchKernelGGL(calib::scan_kernel<calib::kModeApply>, grid, block, 0, st, x_worst, tokens, state, partials);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

// ---- the worst-group scan without a workspace ---------------------------------
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc): the per-group maxima live
// in a file-scope device array instead of the caller's workspace.  Each GPU
// the library runs on holds its own copy (64 KiB, kept until the process
// ends); its address is looked up once per device, with that device current,
// and every call on that GPU shares it: the scan's fill kernel clears the
// entries a call uses before the call reads them, and calls that overlap on
// one GPU race.
constexpr int64_t kScratchGroups = 8192;  // channels <= 262144
static __device__ __align__(256) uint64_t scratch[kScratchGroups];
constexpr int kMaxDevices = 64;

static mxq_status scratch_ptr(uint64_t** out) {
    static std::atomic<uint64_t*> ptrs[kMaxDevices];
    static std::mutex lookup;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXQ_ERR_HIP;
    uint64_t* p = ptrs[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> guard(lookup);
        p = ptrs[dev].load(std::memory_order_relaxed);
        if (!p) {
            void* addr = nullptr;
            if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return MXQ_ERR_HIP;
            p = static_cast<uint64_t*>(addr);
            ptrs[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MXQ_OK;
}

static mxq_status calib_worst_group_noalloc(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                            int64_t stride, const float* lambda, double* x_worst, int64_t* group,
                                            double* linf, void* stream) {
    if (x_dtype != MXQ_BF16 && x_dtype != MXQ_FP16 && x_dtype != MXQ_FP32) return MXQ_ERR_DTYPE;
    if (tokens <= 0 || channels <= 0 || channels % calib::kW || channels > kScratchGroups * calib::kW ||
        tokens > (int64_t(1) << 40) / channels)
        return MXQ_ERR_SHAPE;
    if (!x || !x_worst || !group || !linf) return MXQ_ERR_NULL;
    if (stride < channels) return MXQ_ERR_STRIDE;
    if ((reinterpret_cast<uintptr_t>(x_worst) & 7) || (reinterpret_cast<uintptr_t>(group) & 7) ||
        (reinterpret_cast<uintptr_t>(linf) & 7))
        return MXQ_ERR_ALIGN;
    uint64_t* gmax = nullptr;
    const mxq_status s = scratch_ptr(&gmax);
    if (s != MXQ_OK) return s;
    const int64_t gpr = channels / calib::kW;
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (x_dtype * 2 + (lambda ? 1 : 0)) {
        case MXQ_BF16 * 2: launch_worst<MXQ_BF16, false>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
        case MXQ_BF16 * 2 + 1: launch_worst<MXQ_BF16, true>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
        case MXQ_FP16 * 2: launch_worst<MXQ_FP16, false>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
        case MXQ_FP16 * 2 + 1: launch_worst<MXQ_FP16, true>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
        case MXQ_FP32 * 2: launch_worst<MXQ_FP32, false>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
        default: launch_worst<MXQ_FP32, true>(x, stride, lambda, tokens, gpr, gmax, group, linf, x_worst, st); break;
    }
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

}  // namespace mxq

extern "C" {

size_t mxq_calib_workspace_bytes(int64_t channels) { return mxq::calib_workspace_bytes(channels); }

mxq_status mxq_calib_worst_group_noalloc(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                         int64_t x_row_stride, const float* lambda, double* x_worst,
                                         int64_t* group, double* linf, void* stream) {
    return mxq::calib_worst_group_noalloc(x, x_dtype, tokens, channels, x_row_stride, lambda, x_worst, group, linf,
                                          stream);
}

mxq_status mxq_calib_worst_group(const void* x, int32_t x_dtype, int64_t tokens, int64_t channels,
                                 int64_t x_row_stride, const float* lambda, double* x_worst, int64_t* group,
                                 double* linf, void* workspace, size_t workspace_bytes, void* stream) {
    return mxq::calib_worst_group(x, x_dtype, tokens, channels, x_row_stride, lambda, x_worst, group, linf,
                                  workspace, workspace_bytes, stream);
}

mxq_status mxq_calib_givens_angles(double* x_worst, int64_t tokens, int32_t max_steps, int32_t angle_grid,
                                   double* r_block, double* linf_history, int32_t* steps_done, int32_t* pairs,
                                   int32_t* angles, void* workspace, size_t workspace_bytes, void* stream) {
    return mxq::calib_givens_angles(x_worst, tokens, max_steps, angle_grid, r_block, linf_history, steps_done, pairs,
                                    angles, workspace, workspace_bytes, stream);
}

mxq_status mxq_calib_givens(double* x_worst, int64_t tokens, int32_t max_steps, double* r_block,
                            double* linf_history, int32_t* steps_done, int32_t* pairs, void* workspace,
                            size_t workspace_bytes, void* stream) {
    return mxq::calib_givens(x_worst, tokens, max_steps, r_block, linf_history, steps_done, pairs, workspace,
                             workspace_bytes, stream);
}

}  // extern "C"
