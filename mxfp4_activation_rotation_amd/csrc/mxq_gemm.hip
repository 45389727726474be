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
// 32 consecutive K positions of group l / 16 of the 128: 16 code bytes in the
// order they are stored, low nibble first, which is exactly one MXFP4 group,
// plus that group's scale byte.  Each operand fragment is therefore 64 plain
// 16-byte pieces of the stored codes, with no repacking.
//
// Two storage layouts are accepted, and each kernel is one template over
// them: the row layout the quantizer writes by default, and fragment-tiled
// records (16 rows x 128 positions, slot l = row l % 16, group l / 16), in
// which a fragment is one contiguous 1 KB record.  The MFMA sequence is the
// same for both, so the outputs are bit-identical.
//
// Large products (M > 64): a block of 8 waves (2 per SIMD) computes a
// 256 x 256 tile of y, each wave 128 x 64 (8 x 4 accumulator fragments).  K
// advances 128 positions per stage through a 4-deep LDS ring filled three
// stages ahead by buffer loads with the lds modifier (no staging registers),
// with one bare s_barrier per stage; scales travel in a 3-chunk ring of 4
// stages each.  The operands of the next stage are read from LDS between
// the MFMAs of the current one (software pipelining in registers).  In LDS every fragment sits in a 1 KB slot read by a
// conflict-free ds_read_b128.  Global loads go through buffer resources
// bounded to the tile's rows (or records), so rows past M or N read as zero
// (codes 0, scale 2^-127: products 0) and ragged edges need no branches.
//
// Mid-size products on tiled operands whose 256 x 256 grid has fewer tiles
// than the chip has CUs: 256 x 128 tiles, two blocks per CU (gemm2_kernel).
//
// Decode-shaped products (M <= 64): split-K over the 16 waves of a block
// that owns 16 output columns (see gemm_small_kernel).  From 65 to
// MXQ_GEMM_CHUNKED_MAX_M rows, while the 256 x 256 grid has fewer tiles
// than CUs, the same kernel with one block row per 64 activation rows.  The
// choice depends on the shape only, so both storage layouts give the same
// bits.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mxq.h"
#include "mxq_internal.h"

#ifndef MXQ_GEMM_GROUP_M
#define MXQ_GEMM_GROUP_M 4  // tile rows per band of the block order
#endif
#ifndef MXQ_GEMM_CHUNKED_MAX_M
#define MXQ_GEMM_CHUNKED_MAX_M 128  // above 64 and up to this many rows: the decode kernel in 64-row block rows
#endif
#ifndef MXQ_GEMM_STAGES
#define MXQ_GEMM_STAGES 4  // LDS ring of K stages; loads run MXQ_GEMM_STAGES - 1 stages ahead
#endif

namespace mxq {
namespace {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4g_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4g_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2g_t;

constexpr int kWave = 64;
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kThreads = kWave * kWavesM * kWavesN;  // 512
constexpr int kFragM = 8, kFragN = 4;                // 16-row fragments per wave
constexpr int kBM = 16 * kFragM * kWavesM;           // 256
constexpr int kBN = 16 * kFragN * kWavesN;           // 256
constexpr int kStageK = 128;                         // K positions per stage: one MFMA deep
constexpr int kRowBytes = kStageK / 2;               // code bytes per row per stage
constexpr int kCodeTile = kBM * kRowBytes;           // 16 KB (kBM == kBN)
constexpr int kSlots = kCodeTile / (16 * kWave);     // 1 KB slots per operand tile: 16
constexpr int kLoadsPerThread = kSlots / (kThreads / kWave);  // 2
constexpr int kChunkStages = 4;                      // stages per scale chunk
constexpr int kChunkRowBytes = kChunkStages * kStageK / 32;  // 16 scale bytes per row per chunk
constexpr int kScaleChunk = kBM * kChunkRowBytes;    // 4 KB per operand
constexpr int kNst = MXQ_GEMM_STAGES;
constexpr int kAhead = kNst - 1;
constexpr int kLoadsPerStage = 2 * kLoadsPerThread + 1;  // direct loads per wave per stage
constexpr int kFmtE2M1 = 4;  // operand format code of the scaled MFMA for FP4
constexpr int kXcds = 8;     // MI355X: 8 accelerator dies, each with its own L2
constexpr int64_t kMaxK = int64_t(1) << 24;
static_assert(kBM == kBN, "one staging map serves both operands");
static_assert(kThreads / 2 * 4 == kScaleChunk / kChunkStages,
              "a quarter chunk of an operand is one dword per lane of half the waves");
constexpr int kChunks = 3;  // scale chunk ring: the chunk in use, the next, and one being filled
static_assert(kAhead >= 1 && kAhead <= 7 && kAhead * kLoadsPerStage < 64, "vmcnt is a 6-bit counter");

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

struct Stage {
    uint8_t a[kCodeTile];
    uint8_t b[kCodeTile];
};

struct ScaleChunk {
    uint8_t a[kScaleChunk];
    uint8_t b[kScaleChunk];
};

// Buffer resource over [base, base + bytes); base and bytes are the same in
// every lane (a resource lives in scalar registers) and are read from the
// first active lane, so the compiler never wraps an access in a loop over
// distinct descriptors.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(p & 0xffffffffu)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(p >> 32)));
    void* u = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(u, 0, __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), 0x00020000);
}

__device__ __forceinline__ i32x8_t operand(const u32x4g_t& c) {
    return i32x8_t{static_cast<int>(c[0]), static_cast<int>(c[1]), static_cast<int>(c[2]), static_cast<int>(c[3]),
                   0, 0, 0, 0};
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt left unconstrained; vmcnt is
// split into bits 3:0 and 15:14 of the immediate).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// Wait until at most `later` stages' worth of this wave's direct loads are
// outstanding (a smaller count than needed only waits longer).
__device__ __forceinline__ void wait_stage_loads(int later) {
    switch (later) {
        case 1: wait_vmcnt<kLoadsPerStage>(); break;
        case 2: wait_vmcnt<2 * kLoadsPerStage>(); break;
        case 3: wait_vmcnt<3 * kLoadsPerStage>(); break;
        case 4: wait_vmcnt<4 * kLoadsPerStage>(); break;
        case 5: wait_vmcnt<5 * kLoadsPerStage>(); break;
        case 6: wait_vmcnt<6 * kLoadsPerStage>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

template <bool OUT_BF16, bool TILED>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) Stage st[kNst];
    __shared__ __attribute__((aligned(16))) ScaleChunk sc[kChunks];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int wm = wave / kWavesN;
    const int wn = wave % kWavesN;

    // Block order: dispatch ids go round-robin over the dies, so renumber
    // them to give each die a contiguous range of tiles; then walk bands of
    // MXQ_GEMM_GROUP_M tile rows column by column, so the tiles resident at
    // one time on a die share A rows and B rows in its L2.  (The tile indices
    // are uniform; readfirstlane tells the compiler so, or it would wrap
    // every buffer load in a loop over distinct descriptors.)
    const int nblk = static_cast<int>(gridDim.x);
    int bid = static_cast<int>(blockIdx.x);
    if (nblk % kXcds == 0) bid = (bid % kXcds) * (nblk / kXcds) + bid / kXcds;
    const int band = MXQ_GEMM_GROUP_M * g.tiles_n;
    const int first_m = (bid / band) * MXQ_GEMM_GROUP_M;
    const int band_rows = min(g.tiles_m - first_m, MXQ_GEMM_GROUP_M);
    const int in_band = bid % band;
    const int tm = __builtin_amdgcn_readfirstlane(first_m + in_band % band_rows);
    const int tn = __builtin_amdgcn_readfirstlane(in_band / band_rows);

    const int64_t m0 = static_cast<int64_t>(tm) * kBM;
    const int64_t n0 = static_cast<int64_t>(tn) * kBN;
    const uint32_t cpr = static_cast<uint32_t>(g.K) / 2;   // code bytes per row
    const uint32_t spr = static_cast<uint32_t>(g.K) / 32;  // scale bytes per row
    const uint32_t nk32 = static_cast<uint32_t>(g.K) / kStageK;  // stages = records per record row
    __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
    if constexpr (TILED) {
        // the tile's 16 record rows (fewer at the bottom/right edge)
        const uint32_t recs_a = static_cast<uint32_t>(min<int64_t>(kBM / 16, (g.M + 15) / 16 - m0 / 16));
        const uint32_t recs_b = static_cast<uint32_t>(min<int64_t>(kBN / 16, (g.N + 15) / 16 - n0 / 16));
        ra = rsrc(g.a_codes + (m0 / 16) * nk32 * 1024, recs_a * nk32 * 1024);
        rb = rsrc(g.b_codes + (n0 / 16) * nk32 * 1024, recs_b * nk32 * 1024);
        rsa = rsrc(g.a_scales + (m0 / 16) * nk32 * 64, recs_a * nk32 * 64);
        rsb = rsrc(g.b_scales + (n0 / 16) * nk32 * 64, recs_b * nk32 * 64);
    } else {
        const uint32_t rows_a = static_cast<uint32_t>(min<int64_t>(kBM, g.M - m0));
        const uint32_t rows_b = static_cast<uint32_t>(min<int64_t>(kBN, g.N - n0));
        ra = rsrc(g.a_codes + m0 * cpr, rows_a * cpr);
        rb = rsrc(g.b_codes + n0 * cpr, rows_b * cpr);
        rsa = rsrc(g.a_scales + m0 * spr, rows_a * spr);
        rsb = rsrc(g.b_scales + n0 * spr, rows_b * spr);
    }

    // Code staging (direct global -> LDS loads, no registers): wave w fills
    // slots w and w + 8 of each operand tile, slot f holding the 16 x 64
    // code bytes of rows 16 f .. 16 f + 15 for the stage, as 64 chunks of
    // 16 bytes (chunk c of row r = the 32 K positions of group c).  A direct
    // load puts lane l's 16 bytes at position l of the slot, so the lane
    // decides the layout: lane l fetches row l / 4, chunk (l - l / 16) mod 4,
    // i.e. position p(r, c) = 4 r + (c + r / 4) mod 4.  Each quad of lanes
    // then reads one row's 64 contiguous bytes (one cache-line half per quad
    // for the address unit), and the MFMA lane L, which needs row L % 16 and
    // group L / 16, reads position p(L % 16, L / 16): every 16 lanes of a
    // ds_read_b128 cover the 64 LDS banks once.
    // Fragment-tiled operands are stored in the MFMA lane order already:
    // slot f of stage kt is the contiguous 1 KB record (f, kt), lane l loads
    // its bytes 16 l .. 16 l + 15 and the MFMA lane L reads position L.
    const uint32_t ld_r = static_cast<uint32_t>(lane >> 2);
    const uint32_t ld_c = static_cast<uint32_t>((lane - (lane >> 4)) & 3);
    const uint32_t goff = TILED ? 16 * static_cast<uint32_t>(lane) + static_cast<uint32_t>(wave) * nk32 * 1024
                                : (static_cast<uint32_t>(16 * wave) + ld_r) * cpr + 16 * ld_c;
    // Scale staging: chunk j holds the 16 scale bytes of stages 4 j .. 4 j + 3
    // for every row ([row][16] per operand, a ring of three chunks in LDS).
    // The loads of stage s carry a quarter of chunk s / 4 + 1: waves 0-3
    // fetch A rows 64 q .. 64 q + 63 (q = s mod 4) and waves 4-7 the same
    // rows of B, 4 lanes per row (one 16-byte row slice per quad).  Since
    // stage s is loaded while stage s - 3 computes, the ring slot of chunk
    // s / 4 + 1 last held chunk s / 4 - 2, whose final stage precedes s - 4.
    // Tiled scales: the chunk of record row f is the 4 consecutive 64-byte
    // scale records (f, 4 j .. 4 j + 3), 256 contiguous bytes, stored as
    // [stage][lane] (the row layout stores [row][stage][group]); either way
    // the chunk of fragment f occupies bytes 256 f .. 256 f + 255.
    const bool scale_of_b = wave >= kWavesM * kWavesN / 2;
    const auto rs = scale_of_b ? rsb : rsa;
    const uint32_t s_row = static_cast<uint32_t>(16 * (wave & 3)) + static_cast<uint32_t>(lane >> 2);
    const uint32_t s_goff = TILED ? 4 * static_cast<uint32_t>(lane) + static_cast<uint32_t>(wave & 3) * nk32 * 64
                                  : s_row * spr + 4 * static_cast<uint32_t>(lane & 3);
    typedef __attribute__((address_space(3))) void* lds_ptr;
    auto load_scale_quarter = [&](int chunk, int q) {
        uint8_t* dst = (scale_of_b ? sc[chunk % kChunks].b : sc[chunk % kChunks].a) + (64 * q + 16 * (wave & 3)) * kChunkRowBytes;
        const int so = TILED ? (4 * q * static_cast<int>(nk32) + kChunkStages * chunk) * 64
                             : kChunkRowBytes * chunk + 64 * q * static_cast<int>(spr);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)dst, 4, s_goff, so, 0, 0);
    };
    // Loads of stage kt: its codes, plus one quarter of scale chunk kt / 4 + 1.
    auto load = [&](int kt, int buf) {
        Stage& S = st[buf];
#pragma unroll
        for (int u = 0; u < kLoadsPerThread; ++u) {
            // the slot's rows advance by 128 per u: the step goes into the
            // scalar offset
            const int so = TILED ? 1024 * kt + u * 8 * static_cast<int>(nk32) * 1024
                                 : kRowBytes * kt + u * 128 * static_cast<int>(cpr);
            const int slot = wave + (kThreads / kWave) * u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(S.a + slot * 1024), 16, goff, so, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)(S.b + slot * 1024), 16, goff, so, 0, 0);
        }
        load_scale_quarter(kt / kChunkStages + 1, kt % kChunkStages);
    };

    f32x4g_t acc[kFragM][kFragN];
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j) acc[i][j] = f32x4g_t{0.f, 0.f, 0.f, 0.f};

    // Operand position of lane l in a slot (see the staging map) and its
    // scale byte in a chunk row: group l / 16 of the stage.
    const uint32_t op_off = TILED ? 16 * static_cast<uint32_t>(lane)
                                  : 16 * static_cast<uint32_t>(4 * (lane & 15) + (((lane >> 4) + ((lane & 15) >> 2)) & 3));
    const uint32_t sl = TILED ? static_cast<uint32_t>(lane)
                              : static_cast<uint32_t>((lane & 15) * kChunkRowBytes + (lane >> 4));
    // Operand registers: A fragment f is refilled with the next stage's as
    // soon as its last MFMA of the current stage has issued; B has two sets
    // that alternate between stages.
    u32x4g_t aop[kFragM], bop0[kFragN], bop1[kFragN];
    int sa[kFragM], sb0[kFragN], sb1[kFragN];
    auto read_a = [&](int kt, int f) {
        const Stage& S = st[kt % kNst];
        const ScaleChunk& C = sc[(kt / kChunkStages) % kChunks];
        const uint32_t sq = (TILED ? 64 : 4) * static_cast<uint32_t>(kt % kChunkStages);
        aop[f] = *reinterpret_cast<const u32x4g_t*>(S.a + (wm * kFragM + f) * 1024 + op_off);
        sa[f] = C.a[(wm * kFragM + f) * 16 * kChunkRowBytes + sl + sq];
    };
    auto read_b = [&](int kt, int j, u32x4g_t* bop, int* sb) {
        const Stage& S = st[kt % kNst];
        const ScaleChunk& C = sc[(kt / kChunkStages) % kChunks];
        const uint32_t sq = (TILED ? 64 : 4) * static_cast<uint32_t>(kt % kChunkStages);
        bop[j] = *reinterpret_cast<const u32x4g_t*>(S.b + (wn * kFragN + j) * 1024 + op_off);
        sb[j] = C.b[(wn * kFragN + j) * 16 * kChunkRowBytes + sl + sq];
    };

    // Pipeline.  Stage kt + kAhead is loaded into the ring slot that stage
    // kt - 1 used, and the operands of stage kt + 1 are read while stage kt
    // computes.  Before the barrier of step kt each wave waits for its own
    // loads of stage kt + 1: all but the (at most kAhead - 2) later stages it
    // has issued (vmcnt counts this wave's direct loads, which complete in
    // order).  After the barrier stage kt + 1 is in LDS for every wave, and
    // every wave's reads of stage kt - 1 have returned (its MFMAs consumed
    // them in step kt - 1), so that slot can be refilled.  The barrier is a
    // bare s_barrier: __syncthreads() would add a workgroup fence, which
    // waits for every outstanding direct load (vmcnt(0)) and so would drain
    // the stages in flight; the "memory" clobber keeps the compiler from
    // moving LDS accesses across it.
    static_assert(kAhead >= 2, "stage kt + 1 is read during step kt");
    const int nk = g.K / kStageK;
    if (nk > 0) {
        // scale chunk 0 whole, then the first kAhead stages
#pragma unroll
        for (int q = 0; q < kChunkStages; ++q) load_scale_quarter(0, q);
    }
#pragma unroll
    for (int s0 = 0; s0 < kAhead; ++s0)
        if (s0 < nk) load(s0, s0);
    auto step = [&](int kt, const u32x4g_t* cb, const int* csb, u32x4g_t* nb, int* nsb) {
        if (kt + 1 < nk) wait_stage_loads(min(kAhead - 2, nk - 2 - kt));
        asm volatile("s_barrier" ::: "memory");
        if (kt + kAhead < nk) load(kt + kAhead, (kt + kAhead) % kNst);
        // The scheduling barriers pin the order: four MFMAs of fragment row
        // f, then the reads that refill its registers (and one B fragment).
        // The reads are unconditional, so the step stays one basic block; in
        // the last step they read an in-bounds slot whose values go unused.
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < kFragM; ++f) {
#pragma unroll
            for (int j = 0; j < kFragN; ++j)
                acc[f][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    operand(aop[f]), operand(cb[j]), acc[f][j], kFmtE2M1, kFmtE2M1, 0, sa[f], 0, csb[j]);
            read_a(kt + 1, f);
            if (f < kFragN) read_b(kt + 1, f, nb, nsb);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (nk > 0) {
        wait_stage_loads(min(kAhead - 1, nk - 1));
        asm volatile("s_barrier" ::: "memory");
#pragma unroll
        for (int f = 0; f < kFragM; ++f) read_a(0, f);
#pragma unroll
        for (int j = 0; j < kFragN; ++j) read_b(0, j, bop0, sb0);
    }
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, bop0, sb0, bop1, sb1);
        if (kt + 1 < nk) step(kt + 1, bop1, sb1, bop0, sb0);
    }

    // Accumulator layout: lane l, register r holds row 4 (l / 16) + r,
    // column l % 16 of its 16 x 16 fragment.
    const int h = lane >> 4;
    const int c16 = lane & 15;
#pragma unroll
    for (int f = 0; f < kFragM; ++f) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + (wm * kFragM + f) * 16 + 4 * h + r;
            if (row >= g.M) continue;
#pragma unroll
            for (int j = 0; j < kFragN; ++j) {
                const int64_t col = n0 + (wn * kFragN + j) * 16 + c16;
                if (col >= g.N) continue;
                if constexpr (OUT_BF16)
                    static_cast<__bf16*>(g.y)[row * g.ldy + col] = static_cast<__bf16>(acc[f][j][r]);
                else
                    static_cast<float*>(g.y)[row * g.ldy + col] = acc[f][j][r];
            }
        }
    }
}

// Mid-size products on fragment-tiled operands, whose grid of 256 x 256
// tiles would leave CUs idle (fewer tiles than CUs, e.g. 2048 tokens by 4096
// outputs): a 256 x 128 tile over 4 waves (one per SIMD, each 128 x 64 as
// above, the same MFMA sequence, so the same bits) with two blocks resident
// per CU.  The ring is 3 stages deep and each stage carries its own scale
// records (A 16 KB + B 8 KB of codes, 1 KB + 512 B of scales: 76.5 KB per
// block, so two fit in the 160 KB of LDS).  Stage kt + 2 is loaded while
// stage kt computes, so before the barrier of step kt a wave's only loads in
// flight are those of stage kt + 1 and it waits for all of them.  On grids
// that already fill the chip the 256 x 256 kernel is faster: per flop, a CU
// pulls 1.5x the operand bytes here.
constexpr int k2WavesN = 2;
constexpr int k2Waves = kWavesM * k2WavesN;  // 4
constexpr int k2Threads = kWave * k2Waves;   // 256
constexpr int k2BN = 16 * kFragN * k2WavesN; // 128
constexpr int k2Nst = 3;
constexpr int k2LoadsA = (kBM / 16) / k2Waves;   // 4
constexpr int k2LoadsB = (k2BN / 16) / k2Waves;  // 2
constexpr int k2LoadsPerStage = k2LoadsA + k2LoadsB + 2;

struct Stage2 {
    uint8_t a[kBM * kRowBytes];
    uint8_t b[k2BN * kRowBytes];
    uint8_t sa[kBM / 16 * 64];
    uint8_t sb[k2BN / 16 * 64];
};

template <bool OUT_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(1, k2Threads), amdgpu_waves_per_eu(2))) void gemm2_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) Stage2 st[k2Nst];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int wm = wave / k2WavesN;
    const int wn = wave % k2WavesN;
    const int nblk = static_cast<int>(gridDim.x);
    int bid = static_cast<int>(blockIdx.x);
    if (nblk % kXcds == 0) bid = (bid % kXcds) * (nblk / kXcds) + bid / kXcds;
    const int band = MXQ_GEMM_GROUP_M * g.tiles_n;
    const int first_m = (bid / band) * MXQ_GEMM_GROUP_M;
    const int band_rows = min(g.tiles_m - first_m, MXQ_GEMM_GROUP_M);
    const int in_band = bid % band;
    const int tm = __builtin_amdgcn_readfirstlane(first_m + in_band % band_rows);
    const int tn = __builtin_amdgcn_readfirstlane(in_band / band_rows);
    const int64_t m0 = static_cast<int64_t>(tm) * kBM;
    const int64_t n0 = static_cast<int64_t>(tn) * k2BN;
    const uint32_t nk32 = static_cast<uint32_t>(g.K) / kStageK;
    const uint32_t recs_a = static_cast<uint32_t>(min<int64_t>(kBM / 16, (g.M + 15) / 16 - m0 / 16));
    const uint32_t recs_b = static_cast<uint32_t>(min<int64_t>(k2BN / 16, (g.N + 15) / 16 - n0 / 16));
    const auto ra = rsrc(g.a_codes + (m0 / 16) * nk32 * 1024, recs_a * nk32 * 1024);
    const auto rb = rsrc(g.b_codes + (n0 / 16) * nk32 * 1024, recs_b * nk32 * 1024);
    const auto rsa = rsrc(g.a_scales + (m0 / 16) * nk32 * 64, recs_a * nk32 * 64);
    const auto rsb = rsrc(g.b_scales + (n0 / 16) * nk32 * 64, recs_b * nk32 * 64);
    typedef __attribute__((address_space(3))) void* lds_ptr;
    const uint32_t goff = 16 * static_cast<uint32_t>(lane) + static_cast<uint32_t>(wave) * nk32 * 1024;
    // Each stage slot gets one 1 KB record per load (A records w, w + 4, ...;
    // B records w, w + 4) and the stage's scale records: wave w fetches A
    // records 4 w .. 4 w + 3 (16 lanes x 4 bytes each) and, with lanes 0-31,
    // B records 2 w and 2 w + 1.  Every wave issues the same number of loads
    // per stage (a partial-lane load still counts once in vmcnt).
    const uint32_t sa_goff = (static_cast<uint32_t>(4 * wave + (lane >> 4)) * nk32) * 64 + 4 * static_cast<uint32_t>(lane & 15);
    const uint32_t sb_goff = (static_cast<uint32_t>(2 * wave + ((lane >> 4) & 1)) * nk32) * 64 + 4 * static_cast<uint32_t>(lane & 15);
    auto load = [&](int kt, int buf) {
        Stage2& S = st[buf];
#pragma unroll
        for (int u = 0; u < k2LoadsA; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr)(S.a + (wave + k2Waves * u) * 1024), 16, goff,
                                                     1024 * kt + u * k2Waves * static_cast<int>(nk32) * 1024, 0, 0);
#pragma unroll
        for (int u = 0; u < k2LoadsB; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr)(S.b + (wave + k2Waves * u) * 1024), 16, goff,
                                                     1024 * kt + u * k2Waves * static_cast<int>(nk32) * 1024, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr)(S.sa + wave * 256), 4, sa_goff, 64 * kt, 0, 0);
        if (lane < 32)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr)(S.sb + wave * 128), 4, sb_goff, 64 * kt, 0, 0);
    };
    f32x4g_t acc[kFragM][kFragN];
#pragma unroll
    for (int i = 0; i < kFragM; ++i)
#pragma unroll
        for (int j = 0; j < kFragN; ++j) acc[i][j] = f32x4g_t{0.f, 0.f, 0.f, 0.f};
    const uint32_t op_off = 16 * static_cast<uint32_t>(lane);
    u32x4g_t aop[kFragM], bop0[kFragN], bop1[kFragN];
    int sa[kFragM], sb0[kFragN], sb1[kFragN];
    auto read_a = [&](int kt, int f) {
        const Stage2& S = st[kt % k2Nst];
        aop[f] = *reinterpret_cast<const u32x4g_t*>(S.a + (wm * kFragM + f) * 1024 + op_off);
        sa[f] = S.sa[(wm * kFragM + f) * 64 + lane];
    };
    auto read_b = [&](int kt, int j, u32x4g_t* bop, int* sb) {
        const Stage2& S = st[kt % k2Nst];
        bop[j] = *reinterpret_cast<const u32x4g_t*>(S.b + (wn * kFragN + j) * 1024 + op_off);
        sb[j] = S.sb[(wn * kFragN + j) * 64 + lane];
    };
    const int nk = g.K / kStageK;
#pragma unroll
    for (int s0 = 0; s0 < k2Nst - 1; ++s0)
        if (s0 < nk) load(s0, s0);
    auto step = [&](int kt, const u32x4g_t* cb, const int* csb, u32x4g_t* nb, int* nsb) {
        if (kt + 1 < nk) wait_vmcnt<0>();
        asm volatile("s_barrier" ::: "memory");
        if (kt + k2Nst - 1 < nk) load(kt + k2Nst - 1, (kt + k2Nst - 1) % k2Nst);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int f = 0; f < kFragM; ++f) {
#pragma unroll
            for (int j = 0; j < kFragN; ++j)
                acc[f][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    operand(aop[f]), operand(cb[j]), acc[f][j], kFmtE2M1, kFmtE2M1, 0, sa[f], 0, csb[j]);
            read_a(kt + 1, f);
            if (f < kFragN) read_b(kt + 1, f, nb, nsb);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (nk > 0) {
        if (nk > 1)
            wait_vmcnt<k2LoadsPerStage>();
        else
            wait_vmcnt<0>();
        asm volatile("s_barrier" ::: "memory");
#pragma unroll
        for (int f = 0; f < kFragM; ++f) read_a(0, f);
#pragma unroll
        for (int j = 0; j < kFragN; ++j) read_b(0, j, bop0, sb0);
    }
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, bop0, sb0, bop1, sb1);
        if (kt + 1 < nk) step(kt + 1, bop1, sb1, bop0, sb0);
    }
    const int h = lane >> 4;
    const int c16 = lane & 15;
#pragma unroll
    for (int f = 0; f < kFragM; ++f) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = m0 + (wm * kFragM + f) * 16 + 4 * h + r;
            if (row >= g.M) continue;
#pragma unroll
            for (int j = 0; j < kFragN; ++j) {
                const int64_t col = n0 + (wn * kFragN + j) * 16 + c16;
                if (col >= g.N) continue;
                if constexpr (OUT_BF16)
                    static_cast<__bf16*>(g.y)[row * g.ldy + col] = static_cast<__bf16>(acc[f][j][r]);
                else
                    static_cast<float*>(g.y)[row * g.ldy + col] = acc[f][j][r];
            }
        }
    }
}

// Decode-shaped products (M <= 64 activation rows).  The weights dominate
// the bytes, and a 256 x 256 tile would leave most of the chip idle, so a
// block owns 16 weight rows (output columns) and its 16 waves split K: wave
// w walks stages w, w + 16, ... (128 K positions each) with the same
// 16 x 16 x 128 scaled MFMA, loading its operands straight into registers
// (lane l: row l % 16, group l / 16 of the stage; the activation rows are
// re-read from L2 by every block).  The 16 partial tiles are summed through
// LDS in wave order, so results are deterministic.
//
// In the row layout a fragment is 16 rows x 64 bytes, 16 separate pieces
// per load instruction; in the fragment-tiled layout it is one contiguous
// 1 KB record, which streams at a much higher rate (the activations, read
// by every block, gain the most).  The tiled weights are read with the
// non-temporal policy (each byte is used once); for the row layout the
// default policy is faster, as the two halves of each 128-byte line are
// fetched by different waves.
//
// Small batches above 64 rows (CHUNKED): block row y of a 2-D grid takes
// activation rows 64 y .. 64 y + 63 with the 64-row code.  Dispatch ids go
// round-robin over the dies, so when the column-group count is a multiple
// of 8 (N a multiple of 128) the blocks of one column group land on one die
// and share its L2 copy of the weight records (read with the default policy
// here).  A 256-row tile would run one tile row of blocks on a mostly idle
// chip.
constexpr int kSmallWaves = 16;
constexpr int kAuxNonTemporal = 2;  // cache policy bits of buffer ops
constexpr int kSmallMaxM = 64;
typedef __attribute__((ext_vector_type(4))) float f32x4s_t;

template <bool OUT_BF16, int FM, bool TILED, bool CHUNKED>
__global__ __launch_bounds__(kWave * kSmallWaves) void gemm_small_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) f32x4s_t red[kSmallWaves][FM][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
    const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
    const uint32_t cpr = static_cast<uint32_t>(g.K) / 2;
    const uint32_t spr = static_cast<uint32_t>(g.K) / 32;
    const uint32_t nk32 = static_cast<uint32_t>(g.K) / 128;
    // CHUNKED: block row blockIdx.y owns activation rows 64 y .. 64 y + 63
    const int64_t m_off = CHUNKED ? static_cast<int64_t>(blockIdx.y) * 64 : 0;
    const int64_t rows_a = CHUNKED ? min<int64_t>(64, g.M - m_off) : g.M;
    __amdgpu_buffer_rsrc_t ra, rsa, rb, rsb;
    if constexpr (TILED) {
        const uint32_t recs_a = static_cast<uint32_t>((rows_a + 15) / 16);
        ra = rsrc(g.a_codes + (m_off / 16) * nk32 * 1024, recs_a * nk32 * 1024);
        rsa = rsrc(g.a_scales + (m_off / 16) * nk32 * 64, recs_a * nk32 * 64);
        rb = rsrc(g.b_codes + (n0 / 16) * nk32 * 1024, nk32 * 1024);
        rsb = rsrc(g.b_scales + (n0 / 16) * nk32 * 64, nk32 * 64);
    } else {
        const uint32_t rows_b = static_cast<uint32_t>(min<int64_t>(16, g.N - n0));
        ra = rsrc(g.a_codes + m_off * cpr, static_cast<uint32_t>(rows_a) * cpr);
        rsa = rsrc(g.a_scales + m_off * spr, static_cast<uint32_t>(rows_a) * spr);
        rb = rsrc(g.b_codes + n0 * cpr, rows_b * cpr);
        rsb = rsrc(g.b_scales + n0 * spr, rows_b * spr);
    }
    // (chunked launches reuse each weight record across block rows: default policy)
    constexpr int kAuxB = (TILED && !CHUNKED) ? kAuxNonTemporal : 0;
    const uint32_t r16 = static_cast<uint32_t>(lane & 15);
    const uint32_t q = static_cast<uint32_t>(lane >> 4);
    f32x4s_t acc[FM];
#pragma unroll
    for (int f = 0; f < FM; ++f) acc[f] = f32x4s_t{0.f, 0.f, 0.f, 0.f};
    const int nk = g.K / 128;
    // Stages in flight per wave (all loads of a group issue before its
    // MFMAs): as many as the 128 registers a 1024-thread block leaves each
    // lane allow (8 for 16 rows, 4 for 32, 2 for 64).
    constexpr int kDepth = FM >= 4 ? 2 : (FM == 2 ? 4 : 8);
    for (int s0 = wave; s0 < nk; s0 += kSmallWaves * kDepth) {
        u32x4g_t av[kDepth][FM], bv[kDepth];
        uint32_t sav[kDepth][FM], sbv[kDepth];
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            const int st = s0 + d * kSmallWaves;  // uniform across the wave
            if (st >= nk) break;
            if constexpr (TILED) {
                // record (f, st) of A, record st of this block's B record row
#pragma unroll
                for (int f = 0; f < FM; ++f) {
                    const uint32_t rec = static_cast<uint32_t>(f) * nk32 + static_cast<uint32_t>(st);
                    av[d][f] = __builtin_amdgcn_raw_buffer_load_b128(ra, rec * 1024 + 16 * lane, 0, 0);
                    sav[d][f] = __builtin_amdgcn_raw_buffer_load_b8(rsa, rec * 64 + lane, 0, 0);
                }
                bv[d] = __builtin_amdgcn_raw_buffer_load_b128(rb, static_cast<uint32_t>(st) * 1024 + 16 * lane, 0,
                                                              kAuxB);
                sbv[d] = __builtin_amdgcn_raw_buffer_load_b8(rsb, static_cast<uint32_t>(st) * 64 + lane, 0, kAuxB);
            } else {
                const uint32_t cb = static_cast<uint32_t>(st) * 64 + 16 * q;
                const uint32_t sbyte = static_cast<uint32_t>(st) * 4 + q;
#pragma unroll
                for (int f = 0; f < FM; ++f) {
                    const uint32_t row = 16 * f + r16;
                    av[d][f] = __builtin_amdgcn_raw_buffer_load_b128(ra, row * cpr + cb, 0, 0);
                    sav[d][f] = __builtin_amdgcn_raw_buffer_load_b8(rsa, row * spr + sbyte, 0, 0);
                }
                bv[d] = __builtin_amdgcn_raw_buffer_load_b128(rb, r16 * cpr + cb, 0, kAuxB);
                sbv[d] = __builtin_amdgcn_raw_buffer_load_b8(rsb, r16 * spr + sbyte, 0, kAuxB);
            }
        }
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
            if (s0 + d * kSmallWaves >= nk) break;
#pragma unroll
            for (int f = 0; f < FM; ++f)
                acc[f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    operand(av[d][f]), operand(bv[d]), acc[f], kFmtE2M1, kFmtE2M1, 0, static_cast<int>(sav[d][f]), 0,
                    static_cast<int>(sbv[d]));
        }
    }
#pragma unroll
    for (int f = 0; f < FM; ++f) red[wave][f][lane] = acc[f];
    __syncthreads();
    // Thread t sums element t of the FM x 256 partial tiles over the waves
    // (fixed order) and stores it: lane l, register r of fragment f is row
    // 16 f + 4 (l / 16) + r, column l % 16.
    for (int t = threadIdx.x; t < FM * kWave * 4; t += kWave * kSmallWaves) {
        const int f = t / (kWave * 4);
        const int l = (t / 4) % kWave;
        const int r = t % 4;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kSmallWaves; ++w) sum += red[w][f][l][r];
        const int64_t row = 16 * f + 4 * (l >> 4) + r;
        const int64_t col = n0 + (l & 15);
        if (row < rows_a && col < g.N) {
            if constexpr (OUT_BF16)
                static_cast<__bf16*>(g.y)[(row + m_off) * g.ldy + col] = static_cast<__bf16>(sum);
            else
                static_cast<float*>(g.y)[(row + m_off) * g.ldy + col] = sum;
        }
    }
}

template <bool OUT_BF16, bool TILED>
void launch_small(const GemmArgs& g, hipStream_t st) {
    const dim3 grid(static_cast<unsigned>((g.N + 15) / 16));
    const dim3 block(kWave * kSmallWaves);
    if (g.M <= 16)
        hipLaunchKernelGGL((gemm_small_kernel<OUT_BF16, 1, TILED, false>), grid, block, 0, st, g);
    else if (g.M <= 32)
        hipLaunchKernelGGL((gemm_small_kernel<OUT_BF16, 2, TILED, false>), grid, block, 0, st, g);
    else if (g.M <= kSmallMaxM)
        hipLaunchKernelGGL((gemm_small_kernel<OUT_BF16, 4, TILED, false>), grid, block, 0, st, g);
    else
        hipLaunchKernelGGL((gemm_small_kernel<OUT_BF16, 4, TILED, true>),
                           dim3(grid.x, static_cast<unsigned>((g.M + kSmallMaxM - 1) / kSmallMaxM)), block, 0, st, g);
}

template <bool TILED>
mxq_status launch_gemm(const GemmArgs& g, bool out_bf16, hipStream_t st) {
    const int64_t cus = device_cu_count();
    const bool underfilled = static_cast<int64_t>(g.tiles_m) * g.tiles_n < cus;
    if (g.M <= kSmallMaxM || (underfilled && g.M <= MXQ_GEMM_CHUNKED_MAX_M)) {
        if (out_bf16)
            launch_small<true, TILED>(g, st);
        else
            launch_small<false, TILED>(g, st);
    } else {
        if constexpr (TILED) {
            if (underfilled) {
                GemmArgs g2 = g;
                g2.tiles_n = (g.N + k2BN - 1) / k2BN;
                const dim3 grid2(static_cast<unsigned>(static_cast<int64_t>(g2.tiles_m) * g2.tiles_n));
                if (out_bf16)
                    hipLaunchKernelGGL((gemm2_kernel<true>), grid2, dim3(k2Threads), 0, st, g2);
                else
                    hipLaunchKernelGGL((gemm2_kernel<false>), grid2, dim3(k2Threads), 0, st, g2);
                return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
            }
        }
        const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(g.tiles_m) * g.tiles_n));
        if (out_bf16)
            hipLaunchKernelGGL((gemm_kernel<true, TILED>), grid, dim3(kThreads), 0, st, g);
        else
            hipLaunchKernelGGL((gemm_kernel<false, TILED>), grid, dim3(kThreads), 0, st, g);
    }
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

// Fragment-tiled storage: one thread per 16-byte slot, in record order, so
// each wave writes one 1 KB code record; padding rows get zero bytes.
__global__ __launch_bounds__(256) void tile_kernel(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                                   int32_t K, uint8_t* tcodes, uint8_t* tscales, int64_t slots) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= slots) return;
    const int64_t nk = K / kStageK;
    const int64_t rec = i >> 6;
    const int l = static_cast<int>(i & 63);
    const int64_t row = 16 * (rec / nk) + (l & 15);
    const int64_t grp = 4 * (rec % nk) + (l >> 4);
    u32x4g_t v = {0u, 0u, 0u, 0u};
    uint8_t sc = 0;
    if (row < rows) {
        v = *reinterpret_cast<const u32x4g_t*>(codes + row * (K / 2) + 16 * grp);
        sc = scales[row * (K / 32) + grp];
    }
    *reinterpret_cast<u32x4g_t*>(tcodes + 16 * i) = v;
    tscales[i] = sc;
}

bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

mxq_status gemm_impl(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                            const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* y, int32_t y_dtype,
                            int64_t ldy, void* stream, bool tiled) {
    if (y_dtype != MXQ_FP32 && y_dtype != MXQ_BF16) return MXQ_ERR_DTYPE;
    if (M < 0 || N < 0 || K < 0 || K % kStageK || K > kMaxK || M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31))
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
    const uintptr_t salign = tiled ? 4 : 2;
    if (!aligned_to(a_codes, 16) || !aligned_to(b_codes, 16) || !aligned_to(a_scales, salign) ||
        !aligned_to(b_scales, salign))
        return MXQ_ERR_ALIGN;
    if (tiles_m * tiles_n >= (int64_t(1) << 31)) return MXQ_ERR_SHAPE;
    GemmArgs g{a_codes, a_scales, b_codes, b_scales, y, ldy, static_cast<int32_t>(M), static_cast<int32_t>(N),
               static_cast<int32_t>(K), static_cast<int32_t>(tiles_m), static_cast<int32_t>(tiles_n)};
    hipStream_t st = static_cast<hipStream_t>(stream);
    return tiled ? launch_gemm<true>(g, y_dtype == MXQ_BF16, st) : launch_gemm<false>(g, y_dtype == MXQ_BF16, st);
}

}  // namespace
}  // namespace mxq

using namespace mxq;

extern "C" {

mxq_status mxq_gemm_mxfp4(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                          const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* y, int32_t y_dtype,
                          int64_t ldy, void* stream) {
    return gemm_impl(a_codes, a_scales, b_codes, b_scales, M, N, K, y, y_dtype, ldy, stream, false);
}

mxq_status mxq_gemm_mxfp4_tiled(const uint8_t* a_tcodes, const uint8_t* a_tscales, const uint8_t* b_tcodes,
                                const uint8_t* b_tscales, int64_t M, int64_t N, int64_t K, void* y,
                                int32_t y_dtype, int64_t ldy, void* stream) {
    return gemm_impl(a_tcodes, a_tscales, b_tcodes, b_tscales, M, N, K, y, y_dtype, ldy, stream, true);
}

mxq_status mxq_tile_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t K,
                          uint8_t* tiled_codes, uint8_t* tiled_scales, void* stream) {
    if (rows < 0 || K < 0 || K % kStageK || K > kMaxK || rows >= (int64_t(1) << 31)) return MXQ_ERR_SHAPE;
    if (rows == 0 || K == 0) return MXQ_OK;
    if (!codes || !scales || !tiled_codes || !tiled_scales) return MXQ_ERR_NULL;
    if (!aligned_to(codes, 16) || !aligned_to(tiled_codes, 16)) return MXQ_ERR_ALIGN;
    const int64_t slots = (rows + 15) / 16 * (K / kStageK) * 64;
    const int64_t blocks = (slots + 255) / 256;
    if (blocks >= (int64_t(1) << 31)) return MXQ_ERR_SHAPE;
    hipLaunchKernelGGL(tile_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), codes, scales, rows, static_cast<int32_t>(K), tiled_codes,
                       tiled_scales, slots);
    return hipGetLastError() == hipSuccess ? MXQ_OK : MXQ_ERR_HIP;
}

}  // extern "C"
