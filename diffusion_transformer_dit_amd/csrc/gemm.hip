// bf16, int8 and fp32 MFMA GEMM for gfx950 with the block's fused epilogues.
//
// C[m, n] = sum_k A[m, k] * W[n, k]: A is [M, K] row-major (activations), W is
// [N, K] row-major (weights as [out, in]), both K-contiguous, so both operand
// tiles are copied to LDS row by row and read back as MFMA fragments without a
// transpose.  One workgroup computes a BM x BN tile with WM x WN waves; each
// wave owns a (BM/WM) x (BN/WN) sub-tile built from 16x16 MFMA blocks
// (v_mfma_f32_16x16x32_bf16 with fp32 accumulators; for the W8A8 H256 format
// of the zml-flow-rs page §VII v_mfma_i32_16x16x64_i8 with exact int32
// accumulators, dequantized by the row scales of A and W before the epilogue;
// for fp32 operands four v_mfma_f32_16x16x4f32 per 16-byte fragment pair).  K
// advances 128 bytes of each operand row at a time (64 bf16, 128 int8 or 32
// fp32) through two or three LDS stages: while one stage feeds the MFMAs, the
// next tiles are already in flight from global memory.
//
// Epilogues (run on the fp32 accumulators, no extra pass over memory):
//   * residual : out = resid + gate[n] * acc + bias[n]   (gated residual, ERNIE
//                page §VII Decision 1; out-projection / down-projection)
//   * swiglu   : u = act(acc_gate) * acc_up              (the tile's W rows
//                interleave gate rows and the matching up rows)
//   * qkv      : per-(token, head) LayerNorm or RMSNorm over head_dim with
//                gamma/beta and the RoPE rotation from cos/sin tables, in either
//                order, scatter to head-major q/k and transposed v (zml-flow-rs
//                page §VI "QKV + norm + RoPE"; ERNIE page §IV draws RoPE first)
#include <type_traits>

#include "common.h"
#include "trace.h"

namespace dit {

// Tile shape: BM x BN outputs per workgroup of WM x WN waves, K consumed BK
// elements of ES bytes (2: bf16, 1: int8) at a time through NS LDS stages.
template <int BM_, int BN_, int WM_, int WN_, int BK_ = 64, int NS_ = 2, int ES_ = 2>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NS = NS_, ES = ES_;
    static constexpr int kWaves = WM * WN;
    static constexpr bool kAgpr = false;   // accumulators in AGPRs (the persistent 4-wave kernel's tiles)
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
    static constexpr int TM = kWaveM / 16, TN = kWaveN / 16;    // 16 x 16 MFMA blocks per wave
    static constexpr int kRowBytes = BK * ES;                   // one tile row (BK elements) in LDS
    static constexpr int kChunks = kRowBytes / 16;              // 16-byte chunks per row
    static constexpr int kRowsPerLine = 256 / kRowBytes;        // rows sharing one 64-bank line
    static constexpr int kRowsPerLoad = 1024 / kRowBytes;       // rows one wave-wide 1 KiB load fills
    static constexpr int kALoads = BM / kRowsPerLoad / kWaves;  // buffer->LDS loads per wave per stage
    static constexpr int kBLoads = BN / kRowsPerLoad / kWaves;
    static constexpr int kLoads = kALoads + kBLoads;
    static constexpr int kStageBytes = (BM + BN) * kRowBytes;
    static_assert(BM % (kRowsPerLoad * kWaves) == 0 && BN % (kRowsPerLoad * kWaves) == 0, "tile vs loads");
    static_assert(kWaveM % 16 == 0 && kWaveN % 16 == 0 && kRowBytes % 128 == 0, "wave tile");
    static_assert((NS - 2) * kLoads <= 63, "vmcnt range");
    // Two waves per SIMD leave 256 registers per wave: when the accumulators
    // and double-buffered A and B fragments would not fit (the 320-row tile),
    // the A fragments are single-buffered, each reloaded right after the MFMAs
    // of its row block.
    static constexpr bool kSingleA = kWaves > 4 && TM * TN * 4 + 2 * (TM + TN) * 4 > 224;
    // Chunk c of tile row r lives at slot c ^ swz(r).  gfx950 LDS has 64 banks
    // (256 B per cycle) and a ds_read_b128 serves 16 lanes per cycle; the
    // fragment reads of those 16 lanes are 16 consecutive rows at one logical
    // chunk.  kRowsPerLine rows share a bank line, so rotating the chunk by the
    // line index spreads the 16 rows over all 64 banks.
    static __device__ __forceinline__ int swz(int r) { return (r / kRowsPerLine) & (kChunks - 1); }
    static __device__ __forceinline__ uint32_t off(int r, int c) { return r * kRowBytes + ((c ^ swz(r)) << 4); }
};

// Maps the launch index to a (row-tile, col-tile).  Workgroups are dispatched
// round-robin over the 8 XCDs, so index p runs on XCD p % 8; remap so that
// each XCD receives one contiguous range of tiles, then walk that range in
// groups of kGroupM row-tiles so the tiles resident together on one XCD share
// their W columns (and A rows) in that XCD's L2.
__device__ __forceinline__ void tile_coords(int pid, int num, int tiles_m, int tiles_n, int &tm, int &tn) {
    if ((num & 7) == 0) {
        const int per = num >> 3;
        pid = (pid & 7) * per + (pid >> 3);
    }
    constexpr int kGroupM = 4;
    const int group = kGroupM * tiles_n;
    const int gid = pid / group;
    const int first = gid * kGroupM;
    const int gm = min(tiles_m - first, kGroupM);
    const int in = pid - gid * group;
    tm = first + in % gm;
    tn = in / gm;
}

// Tile widths are template parameters, so the per-tile row arithmetic (done
// for every tile a persistent workgroup takes) has no run-time division.
template <int BN>
struct RowsIdentity {
    __device__ __forceinline__ int operator()(int tile_n, int t) const { return tile_n * BN + t; }
};

// SwiGLU tile rows: each wave's WAVE_N columns are WAVE_N/2 gate rows followed by
// the up rows (offset F) of the same features.
template <int BN, int WAVE_N>
struct RowsSwiglu {
    int F;
    __device__ __forceinline__ int operator()(int tile_n, int t) const {
        constexpr int half = WAVE_N / 2;
        const int w = t / WAVE_N, within = t - w * WAVE_N;
        const int feat = tile_n * (BN / 2) + w * half + (within % half);
        return within >= half ? feat + F : feat;
    }
};

// one 16x16 MFMA block, k = 64 bytes of each operand row (32 bf16 or 64 int8):
// lane l feeds row l % 16 with the 16 bytes of chunk l / 16 and receives
// output rows 4 (l / 16) .. + 3 of column l % 16.  The int8 form keeps its
// int32 accumulators in the same float registers (bit patterns; 0.0f is int
// 0), so the dequantization below converts them in place.  16 x 16 blocks
// rather than 32 x 32 ones: with the same bytes of LDS fragments per MFMA cycle
// the 8-wave main loop runs 6-7 % faster (4096 x 24576 x 4096: 681 -> 638 us).
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(intx4 a, intx4 b, floatx4 c) {
    return __builtin_bit_cast(floatx4,
                              __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, __builtin_bit_cast(intx4, c), 0, 0, 0));
}
// fp32 operands (the fp32 parity path): a 16-byte fragment holds 4 k values per
// lane, consumed by four v_mfma_f32_16x16x4_f32 (value u of both operands: the
// same k in A and B, so every k of the 64-byte step is summed once)
__device__ __forceinline__ floatx4 mfma16(floatx4 a, floatx4 b, floatx4 c) {
#pragma unroll
    for (int u = 0; u < 4; ++u) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], b[u], c, 0, 0, 0);
    return c;
}

// Accumulator element (i, j, r) of a wave sits at wave-tile row i*16 +
// (lane/16)*4 + r and wave-tile column j*16 + lane%16.
__device__ __forceinline__ int acc_row(int i, int r, int lq) { return i * 16 + (lq << 2) + r; }

// a_scale [M] / w_scale [w_rows]: the int8 operands' row scales (ES == 1 only)
template <class T, class RowMap, class Epi>
__global__ __launch_bounds__(T::kThreads, 1)
void gemm_kernel(const void *__restrict__ A, const void *__restrict__ W, int M, int K, int w_rows,
                 int tiles_m, int tiles_n, RowMap rowmap, Epi epi, const float *a_scale, const float *w_scale,
                 int m_base) {
#if defined(__HIP_DEVICE_COMPILE__)   // buffer resources exist only in the device pass
    constexpr int kMain = T::NS * T::kStageBytes;
    constexpr int kLds = Epi::template lds_bytes<T>() > kMain ? Epi::template lds_bytes<T>() : kMain;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = m_base + tm * T::BM;   // m_base: first row of this launch (tail launches)

    const int tid = threadIdx.x;
    // wave index as a scalar: the LDS destinations of the buffer->LDS loads (M0)
    // are then computed on the scalar unit
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;
    const int l16 = lane & 15, lq = lane >> 4;

    // Global -> LDS without registers: buffer_load_dwordx4 ... lds moves 64 x 16
    // bytes of one wave into a contiguous 1 KiB of LDS (lane l at +16 l).  Load
    // q of wave w fills tile rows kRowsPerLoad (q waves + w) ..; lane l brings
    // row + l / kChunks into physical slot l % kChunks, i.e. the logical chunk
    // (l % kChunks) ^ swz(row).
    using Frag = typename std::conditional<T::ES == 2, bf16x8,
                                           typename std::conditional<T::ES == 1, intx4, floatx4>::type>::type;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)M * (uint32_t)K * (uint32_t)T::ES);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(W, (uint32_t)w_rows * (uint32_t)K * (uint32_t)T::ES);
    const int lr = lane / T::kChunks, ls = lane % T::kChunks;
    uint32_t a_off[T::kALoads], b_off[T::kBLoads];
#pragma unroll
    for (int q = 0; q < T::kALoads; ++q) {
        const int r = (q * T::kWaves + wave) * T::kRowsPerLoad + lr;
        const int grow = min(m0 + r, M - 1);              // ragged M: clamp reads, mask stores
        a_off[q] = (uint32_t)grow * (uint32_t)K * (uint32_t)T::ES + (uint32_t)((ls ^ T::swz(r)) << 4);
    }
#pragma unroll
    for (int q = 0; q < T::kBLoads; ++q) {
        const int r = (q * T::kWaves + wave) * T::kRowsPerLoad + lr;
        b_off[q] = (uint32_t)rowmap(tn, r) * (uint32_t)K * (uint32_t)T::ES + (uint32_t)((ls ^ T::swz(r)) << 4);
    }
#define DIT_ISSUE(stage, k0)                                                                             \
    do {                                                                                                 \
        uint8_t *base_ = smem + (stage) * T::kStageBytes;                                                \
        const uint32_t kb_ = (uint32_t)(k0) * (uint32_t)T::ES;                                           \
        _Pragma("unroll") for (int q = 0; q < T::kALoads; ++q) __builtin_amdgcn_raw_ptr_buffer_load_lds( \
            ra, (lds_void *)(base_ + (q * T::kWaves + wave) * 1024), 16, a_off[q], kb_, 0, 0);           \
        _Pragma("unroll") for (int q = 0; q < T::kBLoads; ++q) __builtin_amdgcn_raw_ptr_buffer_load_lds( \
            rw, (lds_void *)(base_ + T::BM * T::kRowBytes + (q * T::kWaves + wave) * 1024), 16, b_off[q], \
            kb_, 0, 0);                                                                                  \
    } while (0)

    floatx4 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j) acc[i][j] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // NS-stage ring: stage s holds K tile kt with kt % NS == s.  Tiles past the
    // end re-load the last tile (never read) so that every iteration issues the
    // same number of loads and the vmcnt bookkeeping stays uniform.
    const int KT = K / T::BK;
    static_assert(T::NS == 2 || T::NS == 3, "the K loop is unrolled over 2 or 3 stages");
    // the unrolled loop keeps more addresses live: only where two waves per
    // SIMD still leave room (at most 16 accumulator blocks per wave), or with
    // one wave per SIMD; the larger 8-wave tiles spill with it
    constexpr bool kUnrollStages = T::kWaves == 4 || T::TM * T::TN <= 16;
    constexpr int KS = T::kRowBytes / 64;   // MFMA k-steps per stage (even: k-step 0 always uses buffer 0)
    static_assert(KS % 2 == 0, "fragment double buffer");
#pragma unroll
    for (int s0 = 0; s0 < T::NS; ++s0) DIT_ISSUE(s0, min(s0, KT - 1) * T::BK);

    if constexpr (!T::kSingleA) {
    Frag af[2][T::TM], bfr[2][T::TN];
    // fragment reads in the order the MFMAs consume them: A0, B0 .. B(TN-1), A1 .. A(TM-1)
#define DIT_LOAD_FRAGS(buf, sa_, sb_, kk)                                                           \
    do {                                                                                          \
        const int c_ = (kk) * 4 + lq;                                                             \
        af[buf][0] = *(const Frag *)((sa_) + T::off(wm * T::kWaveM + l16, c_));                   \
        _Pragma("unroll") for (int j = 0; j < T::TN; ++j)                                        \
            bfr[buf][j] = *(const Frag *)((sb_) + T::off(wn * T::kWaveN + j * 16 + l16, c_));     \
        _Pragma("unroll") for (int i = 1; i < T::TM; ++i)                                        \
            af[buf][i] = *(const Frag *)((sa_) + T::off(wm * T::kWaveM + i * 16 + l16, c_));      \
    } while (0)
#define DIT_MFMAS(buf)                                                                             \
    do {                                                                                          \
        _Pragma("unroll") for (int i = 0; i < T::TM; ++i)                                        \
            _Pragma("unroll") for (int j = 0; j < T::TN; ++j)                                    \
                acc[i][j] = mfma16(af[buf][i], bfr[buf][j], acc[i][j]);                                \
    } while (0)

    wait_vmcnt<(T::NS - 1) * T::kLoads>();   // tile 0 landed
    barrier_only();
    DIT_LOAD_FRAGS(0, smem, smem + T::BM * T::kRowBytes, 0);

    // The workgroup barrier sits inside the MFMA stream: the last k-step's
    // MFMAs run after it, from fragments already in registers, and cover the
    // barrier, the loads of a later tile and the first fragment reads of the
    // next stage, so the matrix pipe does not drain at every K tile.
    // K tile kt uses stage ST = kt % NS.  Where the registers allow (see
    // kUnrollStages) the loop is unrolled over the NS stages, so that ST, and
    // every LDS address of the tile, is a constant
    auto k_tile = [&](int kt, int ST) __attribute__((always_inline)) {
        const uint8_t *sa = smem + ST * T::kStageBytes;
        const uint8_t *sb = sa + T::BM * T::kRowBytes;
#pragma unroll
        for (int kk = 0; kk < KS - 1; ++kk) {
            DIT_LOAD_FRAGS((kk + 1) & 1, sa, sb, kk + 1);   // fetch k-step kk+1 while kk runs
            DIT_MFMAS(kk & 1);
        }
        // the next k-step's reads go out early in each k-step (two per MFMA), so
        // they land long before the MFMAs that need them
#pragma unroll
        for (int kk = 0; kk < KS - 1; ++kk) {
#pragma unroll
            for (int r = 0; r < (T::TM + T::TN + 1) / 2; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // DS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, T::TM * T::TN - (T::TM + T::TN + 1) / 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // tile kt+1 has landed once at most NS-2 later tiles are in flight, and this
        // wave's reads of stage kt are done; after the barrier that holds for every
        // wave, so stage kt may be refilled with tile kt + NS
        wait_vmcnt<(T::NS - 2) * T::kLoads, 0>();
        barrier_only();
        {
            // next stage's first fragments (before the loads: LDS reads are not
            // reordered across the LDS-writing loads)
            const uint8_t *na = smem + ((ST + 1) % T::NS) * T::kStageBytes;
            DIT_LOAD_FRAGS(0, na, na + T::BM * T::kRowBytes, 0);
        }
        DIT_ISSUE(ST, min(kt + T::NS, KT - 1) * T::BK);
        DIT_MFMAS((KS - 1) & 1);
        // after the barrier: fragment reads, then the tile loads spread between
        // the MFMAs of the last k-step
        constexpr int kPer = (T::kLoads + T::TM * T::TN - 1) / (T::TM * T::TN);
        __builtin_amdgcn_sched_group_barrier(0x100, T::TM + T::TN, 0);       // DS read
#pragma unroll
        for (int r = 0; r < T::TM * T::TN; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
            __builtin_amdgcn_sched_group_barrier(0x020, kPer, 0);            // VMEM
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    if constexpr (kUnrollStages) {
        for (int kt = 0;;) {
            k_tile(kt, 0);
            if (++kt >= KT) break;
            k_tile(kt, 1 % T::NS);
            if (++kt >= KT) break;
            if constexpr (T::NS == 3) {
                k_tile(kt, 2);
                if (++kt >= KT) break;
            }
        }
    } else {
        for (int kt = 0; kt < KT; ++kt) k_tile(kt, kt % T::NS);
    }
#undef DIT_MFMAS
#undef DIT_LOAD_FRAGS
    } else {
    // single-buffered A: B fragments of the next k-step first, then per row
    // block i its TN MFMAs followed by the reload of A fragment i
    Frag af[T::TM], bfr[2][T::TN];
#define DIT_LOAD_B(buf, sb_, kk)                                                                     \
    do {                                                                                          \
        const int c_ = (kk) * 4 + lq;                                                             \
        _Pragma("unroll") for (int j = 0; j < T::TN; ++j)                                        \
            bfr[buf][j] = *(const Frag *)((sb_) + T::off(wn * T::kWaveN + j * 16 + l16, c_));     \
    } while (0)
#define DIT_STEP_RELOAD(buf, sa_, kk)                                                              \
    do {                                                                                          \
        const int c_ = (kk) * 4 + lq;                                                             \
        _Pragma("unroll") for (int i = 0; i < T::TM; ++i) {                                      \
            _Pragma("unroll") for (int j = 0; j < T::TN; ++j)                                    \
                acc[i][j] = mfma16(af[i], bfr[buf][j], acc[i][j]);                                 \
            af[i] = *(const Frag *)((sa_) + T::off(wm * T::kWaveM + i * 16 + l16, c_));           \
        }                                                                                         \
    } while (0)
#define DIT_SCHED_ROWS()                                                                           \
    do {                                                                                          \
        __builtin_amdgcn_sched_group_barrier(0x100, T::TN, 0);               /* DS read: B */     \
        _Pragma("unroll") for (int r = 0; r < T::TM; ++r) {                                      \
            __builtin_amdgcn_sched_group_barrier(0x008, T::TN, 0);           /* MFMA */           \
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);               /* DS read: A */     \
        }                                                                                         \
    } while (0)

    wait_vmcnt<(T::NS - 1) * T::kLoads>();   // tile 0 landed
    barrier_only();
#pragma unroll
    for (int i = 0; i < T::TM; ++i) af[i] = *(const Frag *)(smem + T::off(wm * T::kWaveM + i * 16 + l16, lq));
    DIT_LOAD_B(0, smem + T::BM * T::kRowBytes, 0);

    auto k_tile = [&](int kt, int ST) __attribute__((always_inline)) {   // ST = kt % NS (see above)
        const uint8_t *sa = smem + ST * T::kStageBytes;
        const uint8_t *sb = sa + T::BM * T::kRowBytes;
#pragma unroll
        for (int kk = 0; kk < KS - 1; ++kk) {
            DIT_LOAD_B((kk + 1) & 1, sb, kk + 1);
            DIT_STEP_RELOAD(kk & 1, sa, kk + 1);
        }
#pragma unroll
        for (int kk = 0; kk < KS - 1; ++kk) DIT_SCHED_ROWS();
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(T::NS - 2) * T::kLoads, 0>();
        barrier_only();
        {
            // the last k-step reloads from the next stage; every LDS read of it
            // precedes the LDS-writing tile loads, which go out at the end
            const uint8_t *na = smem + ((ST + 1) % T::NS) * T::kStageBytes;
            DIT_LOAD_B(0, na + T::BM * T::kRowBytes, 0);
            DIT_STEP_RELOAD((KS - 1) & 1, na, 0);
        }
        DIT_SCHED_ROWS();
        __builtin_amdgcn_sched_barrier(0);
        DIT_ISSUE(ST, min(kt + T::NS, KT - 1) * T::BK);
    };
    if constexpr (kUnrollStages) {
        for (int kt = 0;;) {
            k_tile(kt, 0);
            if (++kt >= KT) break;
            k_tile(kt, 1 % T::NS);
            if (++kt >= KT) break;
            if constexpr (T::NS == 3) {
                k_tile(kt, 2);
                if (++kt >= KT) break;
            }
        }
    } else {
        for (int kt = 0; kt < KT; ++kt) k_tile(kt, kt % T::NS);
    }
#undef DIT_LOAD_B
#undef DIT_STEP_RELOAD
#undef DIT_SCHED_ROWS
    }
#undef DIT_ISSUE
    wait_vmcnt<0>();      // retire the trailing (never read) loads before LDS is reused
    __syncthreads();

    if constexpr (T::ES != 1 || Epi::kDequant) {
        // bf16, or an epilogue that dequantizes row block by row block itself
        epi.template apply<T>(acc, m0 + wm * T::kWaveM, tn, wn, lane, M, smem);
    } else {
        // dequantize in place: C[m, n] = acc * (a_scale[m] w_scale[n]), the int32
        // sum converted to fp32 (rounded once)
        const int row0 = m0 + wm * T::kWaveM;
        float sw[T::TN];
#pragma unroll
        for (int j = 0; j < T::TN; ++j) sw[j] = w_scale[rowmap(tn, wn * T::kWaveN + j * 16 + l16)];
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            float sa[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) sa[e] = a_scale[min(row0 + acc_row(i, e, lq), M - 1)];
#pragma unroll
            for (int j = 0; j < T::TN; ++j) {
                // whole-vector bit cast: clang mis-lowers a bit cast of one vector element
                const intx4 iv = __builtin_bit_cast(intx4, acc[i][j]);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = (float)iv[e] * (sa[e] * sw[j]);
            }
            // compiler fence (a_scale is not restrict-qualified): the row scales of
            // later blocks are not hoisted next to all 128 accumulators
            asm volatile("" ::: "memory");
        }
        epi.template apply<T>(acc, m0 + wm * T::kWaveM, tn, wn, lane, M, smem);
    }
#endif
}


// ---------------------------------------------------------------------------
// 4-wave 256 x 256 tile for the gated-residual, SwiGLU and split-form QKV
// GEMMs, over bf16 or int8 operands: one wave per SIMD with a 128 x 128 wave
// tile (8 x 8 MFMA blocks of 16 x 16; an int8 block is the same 16 x 16 output
// over 64 instead of 32 k, with int32 sums in the accumulators).  Every
// K fragment read from LDS then feeds 8 MFMAs, so the LDS read traffic per
// MFMA is two thirds of the 8-wave tile's (0.25 instead of 0.375 fragment
// reads per MFMA), which is what bounds the 8-wave loop.  The 256 fp32 (or
// int32) accumulators of a wave fill its AGPRs.  With a single wave per SIMD nothing
// else hides a gap in its MFMA stream, so the K loop is written as inline
// assembly blocks of 16 MFMAs (one pair of A row blocks against the 8 B column
// blocks), each with its share of the other work between the MFMAs:
//   k-step 0 of a K tile  : the LDS reads of four fragments of k-step 1;
//   k-step 1, first block : 8 MFMAs, then the wait for the next K tile's
//                           copies and the workgroup barrier (the matrix pipe
//                           still busy), then the next K tile's fragment reads
//                           and four buffer->LDS copies;
//   k-step 1, other blocks: four reads and four copies, one of each per four
//                           MFMAs (issued together the copies slow the loop).
// LDS holds the A tiles of two K tiles and the W tiles of three (5 x 32 KiB):
// after the barrier of K tile kt the A tile of K tile kt + 2 and the W tile
// of K tile kt + 3 are copied (into the slots of tile kt), so the W copies,
// which more often come from memory than the A rows an XCD's CUs share in L2,
// have two K tiles to land and the barrier waits only for the others.
// Every block waits for its own LDS reads before it ends, so no load that
// writes a register is in flight outside a block; the buffer->LDS copies
// write no register and are counted by the vmcnt wait before the barrier.
// The accumulators stay in AGPRs: the compiler never moves them, since every
// block takes them as tied operands; a tile's first k-step starts them from an
// inline zero.  The workgroups are persistent (one per CU): after a tile's K
// loop the first K tiles of its next tile (A and W of K tiles 0 and 1, W of
// K tile 2) are copied into LDS, then the
// epilogue runs (reading each accumulator from its AGPR where it is used), so
// the copies' latency and the workgroup launch are off the critical path.
// ---------------------------------------------------------------------------
// its tiles: bf16 (BK 64: a K tile's A and W rows are 32 KiB each) and int8
// operands (BK 128, int32 sums in the accumulators, dequantized by the
// epilogue where read)
struct Tile4w : Tile<256, 256, 2, 2> { static constexpr bool kAgpr = true; };
struct Tile4wQ : Tile<256, 256, 2, 2, 128, 2, 1> { static constexpr bool kAgpr = true; };

// INS: the MFMA instruction, v_mfma_f32_16x16x32_bf16 (bf16 operands) or
// v_mfma_i32_16x16x64_i8 (int8 operands: int32 sums in the accumulators)
#define DIT_INS_BF16 "v_mfma_f32_16x16x32_bf16"
#define DIT_INS_I8 "v_mfma_i32_16x16x64_i8"
#define DIT_MF(INS, c, a, b) INS " %[" #c "], %[" #a "], %[" #b "], %[" #c "]\n\t"
#define DIT_RD(dst, base, off) "ds_read_b128 %[" #dst "], %[" #base "] offset:%[" #off "]\n\t"
// copy j of a block: M0 = LDS destination (the add also sets SCC, declared clobbered)
#define DIT_CP(j) "s_add_u32 m0, %[lb], %[d" #j "]\n\t"
#define DIT_LD(j) "buffer_load_dwordx4 %[v" #j "], %[rs], %[so] offen lds\n\t"
// operands: accumulators of A row blocks i0, i0 + 1; the next k-step's
// fragments written by the block (A i0, i0 + 1 and B i0, i0 + 1); the current
// fragments; the LDS addresses of the next fragments (fragment r at r * 2048)
#define DIT_K4_OPERANDS(ac_, acc_, fa_, fb_, na_, nb_, i0, adA, adB)                                            \
    [c00] ac_(acc_[i0][0]), [c01] ac_(acc_[i0][1]), [c02] ac_(acc_[i0][2]), [c03] ac_(acc_[i0][3]),    \
        [c04] ac_(acc_[i0][4]), [c05] ac_(acc_[i0][5]), [c06] ac_(acc_[i0][6]),                         \
        [c07] ac_(acc_[i0][7]), [c10] ac_(acc_[i0 + 1][0]), [c11] ac_(acc_[i0 + 1][1]),                 \
        [c12] ac_(acc_[i0 + 1][2]), [c13] ac_(acc_[i0 + 1][3]), [c14] ac_(acc_[i0 + 1][4]),             \
        [c15] ac_(acc_[i0 + 1][5]), [c16] ac_(acc_[i0 + 1][6]), [c17] ac_(acc_[i0 + 1][7]),             \
        [na0] "=&v"(na_[i0]), [na1] "=&v"(na_[i0 + 1]), [nb0] "=&v"(nb_[i0]), [nb1] "=&v"(nb_[i0 + 1])     \
        : [a0] "v"(fa_[i0]), [a1] "v"(fa_[i0 + 1]), [b0] "v"(fb_[0]), [b1] "v"(fb_[1]), [b2] "v"(fb_[2]),  \
          [b3] "v"(fb_[3]), [b4] "v"(fb_[4]), [b5] "v"(fb_[5]), [b6] "v"(fb_[6]), [b7] "v"(fb_[7]),         \
          [pa] "v"(adA), [pb] "v"(adB), [oa0] "i"((i0) * 2048), [oa1] "i"((i0 + 1) * 2048)
// copies: buffer resource, LDS base (SGPR), K byte offset (SGPR), the four
// per-lane global offsets and the first LDS offset (then + 4 KiB each)
#define DIT_K4_COPIES(rsrc_, ldsb_, soff_, vo_, doff_)                                                     \
    , [rs] "s"(rsrc_), [lb] "s"(ldsb_), [so] "s"(soff_), [v0] "v"(vo_[0]), [v1] "v"(vo_[1]),                \
        [v2] "v"(vo_[2]), [v3] "v"(vo_[3]), [d0] "i"(doff_), [d1] "i"((doff_) + 4096),                     \
        [d2] "i"((doff_) + 8192), [d3] "i"((doff_) + 12288)

// k-step 0 block: 16 MFMAs with four fragment reads
#define DIT_K4_STEP(INS, acc_, fa_, fb_, na_, nb_, i0, adA, adB)                                                \
    asm volatile(DIT_RD(na0, pa, oa0) DIT_MF(INS, c00, a0, b0) DIT_RD(na1, pa, oa1) DIT_MF(INS, c01, a0, b1)         \
                 DIT_RD(nb0, pb, oa0) DIT_MF(INS, c02, a0, b2) DIT_RD(nb1, pb, oa1) DIT_MF(INS, c03, a0, b3)         \
                 DIT_MF(INS, c04, a0, b4) DIT_MF(INS, c05, a0, b5) DIT_MF(INS, c06, a0, b6) DIT_MF(INS, c07, a0, b7)           \
                 DIT_MF(INS, c10, a1, b0) DIT_MF(INS, c11, a1, b1) DIT_MF(INS, c12, a1, b2) DIT_MF(INS, c13, a1, b3)           \
                 DIT_MF(INS, c14, a1, b4) DIT_MF(INS, c15, a1, b5) DIT_MF(INS, c16, a1, b6) DIT_MF(INS, c17, a1, b7)           \
                 "s_waitcnt lgkmcnt(0)"                                                                    \
                 : DIT_K4_OPERANDS("+a", acc_, fa_, fb_, na_, nb_, i0, adA, adB)                                 \
                 : "memory")
// the same block for k-step 0 of a tile's first K stage: each MFMA starts its
// sum from an inline zero, so no accumulator is cleared beforehand
#define DIT_MZ(INS, c, a, b) INS " %[" #c "], %[" #a "], %[" #b "], 0\n\t"
#define DIT_K4_STEP_Z(INS, acc_, fa_, fb_, na_, nb_, i0, adA, adB)                                              \
    asm volatile(DIT_RD(na0, pa, oa0) DIT_MZ(INS, c00, a0, b0) DIT_RD(na1, pa, oa1) DIT_MZ(INS, c01, a0, b1)         \
                 DIT_RD(nb0, pb, oa0) DIT_MZ(INS, c02, a0, b2) DIT_RD(nb1, pb, oa1) DIT_MZ(INS, c03, a0, b3)         \
                 DIT_MZ(INS, c04, a0, b4) DIT_MZ(INS, c05, a0, b5) DIT_MZ(INS, c06, a0, b6) DIT_MZ(INS, c07, a0, b7)           \
                 DIT_MZ(INS, c10, a1, b0) DIT_MZ(INS, c11, a1, b1) DIT_MZ(INS, c12, a1, b2) DIT_MZ(INS, c13, a1, b3)           \
                 DIT_MZ(INS, c14, a1, b4) DIT_MZ(INS, c15, a1, b5) DIT_MZ(INS, c16, a1, b6) DIT_MZ(INS, c17, a1, b7)           \
                 "s_waitcnt lgkmcnt(0)"                                                                    \
                 : DIT_K4_OPERANDS("=a", acc_, fa_, fb_, na_, nb_, i0, adA, adB)                           \
                 : "memory")
// first k-step 1 block: 8 MFMAs, the wait for all copies but the last eight
// (the W copies of the K tile after next) and the barrier, then 8 MFMAs with
// four reads and four copies
#define DIT_K4_STEP_BARRIER(INS, acc_, fa_, fb_, na_, nb_, i0, adA, adB, rsrc_, ldsb_, soff_, vo_, doff_)       \
    asm volatile(DIT_MF(INS, c00, a0, b0) DIT_MF(INS, c01, a0, b1) DIT_MF(INS, c02, a0, b2) DIT_MF(INS, c03, a0, b3)           \
                 DIT_MF(INS, c04, a0, b4) DIT_MF(INS, c05, a0, b5) DIT_MF(INS, c06, a0, b6) DIT_MF(INS, c07, a0, b7)           \
                 "s_waitcnt vmcnt(8)\n\ts_barrier\n\t"                                                     \
                 DIT_RD(na0, pa, oa0) DIT_CP(0) DIT_MF(INS, c10, a1, b0) DIT_LD(0) DIT_MF(INS, c11, a1, b1)          \
                 DIT_RD(na1, pa, oa1) DIT_CP(1) DIT_MF(INS, c12, a1, b2) DIT_LD(1) DIT_MF(INS, c13, a1, b3)          \
                 DIT_RD(nb0, pb, oa0) DIT_CP(2) DIT_MF(INS, c14, a1, b4) DIT_LD(2) DIT_MF(INS, c15, a1, b5)          \
                 DIT_RD(nb1, pb, oa1) DIT_CP(3) DIT_MF(INS, c16, a1, b6) DIT_LD(3) DIT_MF(INS, c17, a1, b7)          \
                 "s_waitcnt lgkmcnt(0)"                                                                    \
                 : DIT_K4_OPERANDS("+a", acc_, fa_, fb_, na_, nb_, i0, adA, adB)                                 \
                     DIT_K4_COPIES(rsrc_, ldsb_, soff_, vo_, doff_)                                        \
                 : "memory", "m0", "scc")
// other k-step 1 blocks: one read and one copy per four MFMAs
#define DIT_K4_STEP_COPY(INS, acc_, fa_, fb_, na_, nb_, i0, adA, adB, rsrc_, ldsb_, soff_, vo_, doff_)          \
    asm volatile(DIT_MF(INS, c00, a0, b0) DIT_RD(na0, pa, oa0) DIT_MF(INS, c01, a0, b1) DIT_CP(0)                    \
                 DIT_MF(INS, c02, a0, b2) DIT_LD(0) DIT_MF(INS, c03, a0, b3)                                         \
                 DIT_MF(INS, c04, a0, b4) DIT_RD(na1, pa, oa1) DIT_MF(INS, c05, a0, b5) DIT_CP(1)                    \
                 DIT_MF(INS, c06, a0, b6) DIT_LD(1) DIT_MF(INS, c07, a0, b7)                                         \
                 DIT_MF(INS, c10, a1, b0) DIT_RD(nb0, pb, oa0) DIT_MF(INS, c11, a1, b1) DIT_CP(2)                    \
                 DIT_MF(INS, c12, a1, b2) DIT_LD(2) DIT_MF(INS, c13, a1, b3)                                         \
                 DIT_MF(INS, c14, a1, b4) DIT_RD(nb1, pb, oa1) DIT_MF(INS, c15, a1, b5) DIT_CP(3)                    \
                 DIT_MF(INS, c16, a1, b6) DIT_LD(3) DIT_MF(INS, c17, a1, b7)                                         \
                 "s_waitcnt lgkmcnt(0)"                                                                    \
                 : DIT_K4_OPERANDS("+a", acc_, fa_, fb_, na_, nb_, i0, adA, adB)                                 \
                     DIT_K4_COPIES(rsrc_, ldsb_, soff_, vo_, doff_)                                        \
                 : "memory", "m0", "scc")

// The lane index, computed afresh by each call: a value the compiler can not
// hoist and keep live (the persistent 4-wave kernel has no register to hold
// lane-derived addresses across its K loop).
__device__ __forceinline__ int lane_now() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

template <class T, class RowMap, class Epi>
__global__ __launch_bounds__(256, 1)
void gemm4_kernel(const void *__restrict__ A, const void *__restrict__ W, int M, int K, int w_rows, int tiles_m,
                  int tiles_n, RowMap rowmap, Epi epi, int m_base) {
#if defined(__HIP_DEVICE_COMPILE__)
    static_assert(T::kAgpr && T::kWaves == 4 && T::TM == 8 && T::TN == 8 && (T::ES == 2 || T::ES == 1) &&
                      T::NS == 2 && T::kRowBytes == 128 && T::kALoads == 8 && T::kBLoads == 8 &&
                      T::kStageBytes == 65536,
                  "the 4-wave 256 x 256 tile: bf16 (64-deep K tiles) or int8 (128-deep)");
    // the next tile's first K tiles are copied into LDS while the epilogue of
    // the current one runs, so the epilogue may not use LDS
    static_assert(Epi::template lds_bytes<T>() == 0, "epilogue LDS");
    // two 32 KiB A slots (K tiles kt % 2) and three W slots (kt % 3): the W tile
    // of K tile kt + 3 is copied while tile kt + 1 is in use, two K tiles ahead
    constexpr uint32_t kA0 = 0, kW0 = 65536, kSlot = 32768;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kSlot + 3 * kSlot];

    const int ntiles = tiles_m * tiles_n;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int wm = wave / T::WN, wn = wave % T::WN;

    // Copies as in gemm_kernel: copy q (0-7: A rows, 8-15: W rows) of wave w
    // moves tile rows 8 (4 q + w) .. + 7 into 1 KiB of its stage.
    constexpr uint32_t ES = T::ES;
    const uint32_t a_bytes = (uint32_t)M * (uint32_t)K * ES, w_bytes = (uint32_t)w_rows * (uint32_t)K * ES;
    uint32_t a_off[8], b_off[8];
    auto tile_offsets = [&](int tm_, int tn_) {
        const int m0_ = m_base + tm_ * T::BM;
        // the lane terms are recomputed for each tile, not held in registers
        // across the K loop (where there are none to spare)
        const int ln = lane_now(), lr_ = ln / T::kChunks, ls_ = ln % T::kChunks;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int r = (q * 4 + wave) * T::kRowsPerLoad + lr_;
            a_off[q] = (uint32_t)min(m0_ + r, M - 1) * (uint32_t)K * ES + (uint32_t)((ls_ ^ T::swz(r)) << 4);
            b_off[q] = (uint32_t)rowmap(tn_, r) * (uint32_t)K * ES + (uint32_t)((ls_ ^ T::swz(r)) << 4);
        }
    };
    // the same two buffer resources as plain dwords for the copies inside the
    // asm blocks: base address (48 bits), no stride, size in bytes, format word
    typedef int int4v __attribute__((ext_vector_type(4)));
    const uint64_t pa64 = (uint64_t)(uintptr_t)A, pw64 = (uint64_t)(uintptr_t)W;
    const int4v ra4 = {(int)(uint32_t)pa64, (int)((pa64 >> 32) & 0xffff), (int)a_bytes, 0x00020000};
    const int4v rw4 = {(int)(uint32_t)pw64, (int)((pw64 >> 32) & 0xffff), (int)w_bytes, 0x00020000};

    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;

    const int KT = K / T::BK;
    // A and W of K tiles 0 and 1 and W of K tile 2 into their slots: copy q of
    // A rows and of W rows to + q * 4 KiB of the slot (as in the K loop, M0
    // holds the LDS destination)
    const uint32_t lbw = lds0 + wave * 1024, kb1 = (uint32_t)(min(1, KT - 1) * T::kRowBytes),
                   kb2 = (uint32_t)(min(2, KT - 1) * T::kRowBytes);
#define DIT_PCP(m0off, vo, rs, kb) \
    "s_add_u32 m0, %[lb], " #m0off "\n\tbuffer_load_dwordx4 %[" #vo "], %[" #rs "], %[" #kb "] offen lds\n\t"
    auto issue_first_stages = [&]() {
        asm volatile(
            // A0, W0 (K tile 0), A1, W1 (K tile 1), W2 (K tile 2), in this order
            DIT_PCP(0, a0, ra, k0) DIT_PCP(4096, a1, ra, k0) DIT_PCP(8192, a2, ra, k0) DIT_PCP(12288, a3, ra, k0)
            DIT_PCP(16384, a4, ra, k0) DIT_PCP(20480, a5, ra, k0) DIT_PCP(24576, a6, ra, k0) DIT_PCP(28672, a7, ra, k0)
            DIT_PCP(65536, b0, rw, k0) DIT_PCP(69632, b1, rw, k0) DIT_PCP(73728, b2, rw, k0) DIT_PCP(77824, b3, rw, k0)
            DIT_PCP(81920, b4, rw, k0) DIT_PCP(86016, b5, rw, k0) DIT_PCP(90112, b6, rw, k0) DIT_PCP(94208, b7, rw, k0)
            DIT_PCP(32768, a0, ra, k1) DIT_PCP(36864, a1, ra, k1) DIT_PCP(40960, a2, ra, k1) DIT_PCP(45056, a3, ra, k1)
            DIT_PCP(49152, a4, ra, k1) DIT_PCP(53248, a5, ra, k1) DIT_PCP(57344, a6, ra, k1) DIT_PCP(61440, a7, ra, k1)
            DIT_PCP(98304, b0, rw, k1) DIT_PCP(102400, b1, rw, k1) DIT_PCP(106496, b2, rw, k1) DIT_PCP(110592, b3, rw, k1)
            DIT_PCP(114688, b4, rw, k1) DIT_PCP(118784, b5, rw, k1) DIT_PCP(122880, b6, rw, k1) DIT_PCP(126976, b7, rw, k1)
            DIT_PCP(131072, b0, rw, k2) DIT_PCP(135168, b1, rw, k2) DIT_PCP(139264, b2, rw, k2) DIT_PCP(143360, b3, rw, k2)
            DIT_PCP(147456, b4, rw, k2) DIT_PCP(151552, b5, rw, k2) DIT_PCP(155648, b6, rw, k2) DIT_PCP(159744, b7, rw, k2)
            : : [lb] "s"(lbw), [ra] "s"(ra4), [rw] "s"(rw4), [k0] "s"(0u), [k1] "s"(kb1), [k2] "s"(kb2),
              [a0] "v"(a_off[0]), [a1] "v"(a_off[1]), [a2] "v"(a_off[2]), [a3] "v"(a_off[3]),
              [a4] "v"(a_off[4]), [a5] "v"(a_off[5]), [a6] "v"(a_off[6]), [a7] "v"(a_off[7]),
              [b0] "v"(b_off[0]), [b1] "v"(b_off[1]), [b2] "v"(b_off[2]), [b3] "v"(b_off[3]),
              [b4] "v"(b_off[4]), [b5] "v"(b_off[5]), [b6] "v"(b_off[6]), [b7] "v"(b_off[7])
            : "memory", "m0", "scc");
    };
#undef DIT_PCP

    // Persistent: workgroup b takes tiles b, b + grid, ... in the order of
    // tile_coords, so the tiles resident together on one XCD are the same as
    // with one workgroup per tile.
    int pid = blockIdx.x, tm, tn;
    tile_coords(pid, ntiles, tiles_m, tiles_n, tm, tn);
    tile_offsets(tm, tn);
    issue_first_stages();
    floatx4 acc[8][8];
    bf16x8 fa[8], fb[8], na[8], nb[8];
    for (bool first = true;; first = false) {
        // LDS byte addresses of this lane's fragments: stage s, k-step kk (chunk
        // kk * 4 + lq of the 128-byte row), fragment r at + r * 2048 (16 rows
        // on); the swizzle of rows base + 16 r + l16 depends on l16 only.  Like
        // the copy offsets they are rebuilt for each tile, so that nothing but
        // the accumulators is live across the epilogue.
        uint32_t adA[2][2], adB[3][2];
        {
            const int ln = lane_now(), l16_ = ln & 15, lq_ = ln >> 4, swl = (l16_ >> 1) & 7;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint32_t col = (uint32_t)(((kk * 4 + lq_) ^ swl) << 4);
#pragma unroll
                for (int s = 0; s < 2; ++s) adA[s][kk] = lds0 + kA0 + s * kSlot + (uint32_t)(wm * 128 + l16_) * 128u + col;
#pragma unroll
                for (int s = 0; s < 3; ++s) adB[s][kk] = lds0 + kW0 + s * kSlot + (uint32_t)(wn * 128 + l16_) * 128u + col;
            }
        }
        if (!first) tile_offsets(tm, tn);
        const uint32_t va[2][4] = {{a_off[0], a_off[1], a_off[2], a_off[3]}, {a_off[4], a_off[5], a_off[6], a_off[7]}};
        const uint32_t vb[2][4] = {{b_off[0], b_off[1], b_off[2], b_off[3]}, {b_off[4], b_off[5], b_off[6], b_off[7]}};
        // K tile 0 landed.  The first tile's later copies may still be in
        // flight; a later tile's copies went out before the previous epilogue,
        // whose stores count in the same counter, so there everything is
        // waited for.
        if (first) wait_vmcnt<24>();   // A0, W0 landed; A1, W1, W2 may be in flight
        else wait_vmcnt<0>();
        barrier_only();
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            fa[r] = *(const bf16x8 *)(smem + adA[0][0] - lds0 + r * 2048);
            fb[r] = *(const bf16x8 *)(smem + adB[0][0] - lds0 + r * 2048);
        }

        // one K tile: k-step 0 (fa, fb) || reads of its k-step 1; then k-step 1
        // (na, nb) || after the barrier (K tile kt + 1 has landed and every
        // wave is done with the slots of K tile kt): reads of k-step 0 of K tile
        // kt + 1, copies of A(kt + 2) and W(kt + 3) into the slots of K tile kt
        // (A slot SA = kt % 2, W slot SW = kt % 3).  STEP0 is the k-step 0
        // block: the zero-start one in the tile's first K tile.
#define DIT_K4_TILE(INS, kt, SA, SW, STEP0)                                                                          \
    do {                                                                                                           \
        constexpr int sa_ = (SA), sw_ = (SW), na_ = sa_ ^ 1, nw_ = (sw_ + 1) % 3;                                   \
        STEP0(INS, acc, fa, fb, na, nb, 0, adA[sa_][1], adB[sw_][1]);                                              \
        STEP0(INS, acc, fa, fb, na, nb, 2, adA[sa_][1], adB[sw_][1]);                                              \
        STEP0(INS, acc, fa, fb, na, nb, 4, adA[sa_][1], adB[sw_][1]);                                              \
        STEP0(INS, acc, fa, fb, na, nb, 6, adA[sa_][1], adB[sw_][1]);                                              \
        const uint32_t lbA = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds0 + kA0 + sa_ * kSlot + wave * 1024)); \
        const uint32_t lbW = (uint32_t)__builtin_amdgcn_readfirstlane((int)(lds0 + kW0 + sw_ * kSlot + wave * 1024)); \
        const uint32_t kbA = (uint32_t)__builtin_amdgcn_readfirstlane(min((kt) + 2, KT - 1) * T::kRowBytes);       \
        const uint32_t kbW = (uint32_t)__builtin_amdgcn_readfirstlane(min((kt) + 3, KT - 1) * T::kRowBytes);       \
        DIT_K4_STEP_BARRIER(INS, acc, na, nb, fa, fb, 0, adA[na_][0], adB[nw_][0], ra4, lbA, kbA, va[0], 0);        \
        DIT_K4_STEP_COPY(INS, acc, na, nb, fa, fb, 2, adA[na_][0], adB[nw_][0], ra4, lbA, kbA, va[1], 16384);       \
        DIT_K4_STEP_COPY(INS, acc, na, nb, fa, fb, 4, adA[na_][0], adB[nw_][0], rw4, lbW, kbW, vb[0], 0);           \
        DIT_K4_STEP_COPY(INS, acc, na, nb, fa, fb, 6, adA[na_][0], adB[nw_][0], rw4, lbW, kbW, vb[1], 16384);       \
    } while (0)
        // K tile kt uses A slot kt % 2 and W slot kt % 3: the loop is unrolled over
        // the 6 combinations so that every LDS address of a block is a constant
#define DIT_K4_LOOP(INS)                                                                                          \
    do {                                                                                                           \
        DIT_K4_TILE(INS, 0, 0, 0, DIT_K4_STEP_Z);                                                                  \
        for (int kt = 1; kt < KT;) {                                                                               \
            DIT_K4_TILE(INS, kt, 1, 1, DIT_K4_STEP); if (++kt >= KT) break;                                        \
            DIT_K4_TILE(INS, kt, 0, 2, DIT_K4_STEP); if (++kt >= KT) break;                                        \
            DIT_K4_TILE(INS, kt, 1, 0, DIT_K4_STEP); if (++kt >= KT) break;                                        \
            DIT_K4_TILE(INS, kt, 0, 1, DIT_K4_STEP); if (++kt >= KT) break;                                        \
            DIT_K4_TILE(INS, kt, 1, 2, DIT_K4_STEP); if (++kt >= KT) break;                                        \
            DIT_K4_TILE(INS, kt, 0, 0, DIT_K4_STEP); ++kt;                                                         \
        }                                                                                                          \
    } while (0)
        if constexpr (T::ES == 2) DIT_K4_LOOP(DIT_INS_BF16);
        else DIT_K4_LOOP(DIT_INS_I8);
#undef DIT_K4_LOOP
#undef DIT_K4_TILE
        wait_vmcnt<0>();      // retire the trailing (never read) copies before LDS is reused
        __syncthreads();
        // the last MFMAs' results are written back before anything reads the AGPRs
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
        const int row0 = m_base + tm * T::BM + wm * T::kWaveM, tn_cur = tn;
        pid += gridDim.x;
        const bool more = pid < ntiles;
        if (more) {
            // every wave is past its last LDS read of this tile (the barrier above)
            tile_coords(pid, ntiles, tiles_m, tiles_n, tm, tn);
            tile_offsets(tm, tn);
            issue_first_stages();
        }
        epi.template apply<T>(acc, row0, tn_cur, wn, lane_now(), M, smem);
        if (!more) break;
    }
#endif
}
#undef DIT_K4_STEP_COPY
#undef DIT_K4_STEP_BARRIER
#undef DIT_K4_STEP_Z
#undef DIT_K4_STEP
#undef DIT_MZ
#undef DIT_INS_BF16
#undef DIT_INS_I8
#undef DIT_K4_COPIES
#undef DIT_K4_OPERANDS
#undef DIT_LD
#undef DIT_CP
#undef DIT_RD
#undef DIT_MF

#undef DIT_Q4_MFMA


// An accumulator element read by an epilogue.  The persistent 4-wave kernel
// keeps its accumulators in AGPRs; there each element is read into a VGPR
// where it is used (with plain reads the compiler copies all 256 out right
// after the K loop, which takes every VGPR and spills what the persistent loop
// keeps).
template <class T>
__device__ __forceinline__ float acc_get(const floatx4 &a, int e) {
    if constexpr (T::kAgpr) {
        float x;
        asm("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(a[e]));
        return x;
    } else {
        return a[e];
    }
}

// ---------------------------------------------------------------------------
// epilogue: out = resid + gate * acc + bias
// ---------------------------------------------------------------------------
// Q8: the accumulators hold int32 sums of int8 codes; each row block is
// dequantized here with the row scales a_scale[m] w_scale[n], next to the
// residual rows it is added to (a separate pass over all 128 accumulators
// first makes the compiler hoist all 64 row-scale loads and spill).
template <typename TR, typename TO, bool Q8 = false>
struct EpiResidual {
    const TR *resid;
    const float *gate, *bias;
    TO *out;
    int N;
    int gate_fn;      // 0 identity, 1 tanh, 2 sigmoid, applied to gate[n]
    const float *a_scale = nullptr, *w_scale = nullptr;   // Q8 only
    static constexpr bool kDequant = Q8;
    template <class T> static constexpr int lds_bytes() { return 0; }
    template <class T>
    __device__ __forceinline__ void apply(floatx4 (&acc)[T::TM][T::TN], int row0, int tn, int wn, int lane, int M,
                                          uint8_t *) const {
        const int l16 = lane & 15, lq = lane >> 4;
        const int col0 = tn * T::BN + wn * T::kWaveN;
        float g[T::TN], bb[T::TN];
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int col = col0 + j * 16 + l16;
            g[j] = gate ? gate_f(gate[col], gate_fn) : 1.0f;
            if constexpr (Q8) g[j] *= w_scale[col];
            bb[j] = bias ? bias[col] : 0.0f;
        }
        // out may alias resid (in-place update), but every element is read and
        // written by this lane only, so a batch of residual loads (IB row blocks,
        // 32 elements per lane) may precede the batch of stores; without the
        // batching the compiler has to wait for each store before the next load.
        // Rows past M load row M - 1 and store nothing.
        constexpr int IB = (32 / (T::TN * 4)) > 0 ? 32 / (T::TN * 4) : 1;
        static_assert(T::TM % IB == 0, "row blocks per batch");
#pragma unroll
        for (int i0 = 0; i0 < T::TM; i0 += IB) {
            float r[IB][T::TN][4];
            if (resid) {
#pragma unroll
                for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                    for (int j = 0; j < T::TN; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int row = min(row0 + acc_row(i0 + ib, e, lq), M - 1);
                            r[ib][j][e] = to_f32<TR>(resid[(size_t)row * N + col0 + j * 16 + l16]);
                        }
            } else {
#pragma unroll
                for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                    for (int j = 0; j < T::TN; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e) r[ib][j][e] = 0.0f;
            }
            float sa[IB][4];   // Q8: row scales of the batch
            if constexpr (Q8) {
#pragma unroll
                for (int ib = 0; ib < IB; ++ib) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sa[ib][e] = a_scale[min(row0 + acc_row(i0 + ib, e, lq), M - 1)];
                    if constexpr (!T::kAgpr) {
#pragma unroll
                        for (int j = 0; j < T::TN; ++j) {
                            const intx4 iv = __builtin_bit_cast(intx4, acc[i0 + ib][j]);   // whole-vector cast (see kernel)
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[i0 + ib][j][e] = (float)iv[e] * sa[ib][e];
                        }
                    }
                }
            }
            // the product of a row and a column: the persistent 4-wave tile
            // dequantizes its AGPR-held int32 sums here, where each is read (the
            // other tiles above)
            auto val = [&](int ib, int j, int e) -> float {
                if constexpr (Q8 && T::kAgpr)
                    return (float)__builtin_bit_cast(int, acc_get<T>(acc[i0 + ib][j], e)) * sa[ib][e];
                else
                    return acc_get<T>(acc[i0 + ib][j], e);
            };
            // wave-uniform: all rows of the batch in range -> straight-line stores
            if (row0 + (i0 + IB) * 16 <= M) {
#pragma unroll
                for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                    for (int j = 0; j < T::TN; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            out[(size_t)(row0 + acc_row(i0 + ib, e, lq)) * N + col0 + j * 16 + l16] =
                                from_f32<TO>(fmaf(val(ib, j, e), g[j], bb[j]) + r[ib][j][e]);
            } else {
#pragma unroll
                for (int ib = 0; ib < IB; ++ib)
#pragma unroll
                    for (int j = 0; j < T::TN; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int row = row0 + acc_row(i0 + ib, e, lq);
                            if (row < M)
                                out[(size_t)row * N + col0 + j * 16 + l16] =
                                    from_f32<TO>(fmaf(val(ib, j, e), g[j], bb[j]) + r[ib][j][e]);
                        }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// epilogue: u = act(gate) * up, act = SiLU or the clamped GELU-tanh
// ---------------------------------------------------------------------------
template <int ACT, typename TU = bf16>     // ACT 0: SiLU (SwiGLU), 1: clamped GELU-tanh; TU: output type
struct EpiSwiglu {
    static constexpr bool kDequant = false;
    TU *u;
    int F;
    // int8 operands on the 4-wave tile: row and W-row scales, applied here (the
    // 8-wave kernels dequantize before the epilogue)
    const float *a_scale = nullptr, *w_scale = nullptr;
    template <class T> static constexpr int lds_bytes() { return 0; }
    template <class T>
    __device__ __forceinline__ void apply(floatx4 (&acc)[T::TM][T::TN], int row0, int tn, int wn, int lane, int M,
                                          uint8_t *) const {
        const int l16 = lane & 15, lq = lane >> 4;
        constexpr int HJ = T::TN / 2;
        const int f0 = tn * (T::BN / 2) + wn * (T::kWaveN / 2);
        // int32 sums in the accumulators (the 4-wave int8 tile): C[m, n] =
        // sum * (a_scale[m] w_scale[n]); column block j < HJ holds gate features
        // f0 + 16 j + l16 (W rows of the same index), j >= HJ their up rows (+ F)
        constexpr bool kQ = T::ES == 1 && T::kAgpr;
        float sw[kQ ? T::TN : 1];
        if constexpr (kQ) {
#pragma unroll
            for (int j = 0; j < T::TN; ++j) sw[j] = w_scale[(j < HJ ? 0 : F) + f0 + (j % HJ) * 16 + l16];
        }
        auto row_scales = [&](int i, float (&sa)[4]) {
            if constexpr (kQ) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sa[e] = a_scale[min(row0 + acc_row(i, e, lq), M - 1)];
            }
        };
        auto val = [&](int i, int j, int e, const float (&sa)[4]) -> float {
            if constexpr (kQ)
                return (float)__builtin_bit_cast(int, acc_get<T>(acc[i][j], e)) * (sa[e] * sw[j]);
            else
                return acc_get<T>(acc[i][j], e);
        };
        // the HJ column blocks of one output row are stored back to back, so
        // each 16 HJ-feature row segment reaches L2 whole instead of in pieces
        // far apart in time (which cost partial-line write-backs)
        auto row_block = [&](int i, bool check) {
            float sa[4];
            row_scales(i, sa);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = row0 + acc_row(i, e, lq);
                if (!check || row < M) {
#pragma unroll
                    for (int j = 0; j < HJ; ++j) {
                        const float z = val(i, j, e, sa);
                        const float g = ACT == 1 ? gelu_tanh_f(z) : silu_f(z);
                        u[(size_t)row * F + f0 + j * 16 + l16] = from_f32<TU>(g * val(i, j + HJ, e, sa));
                    }
                }
            }
        };
        // wave-uniform: all the wave's rows in range -> no per-row branches
        const bool full = row0 + T::kWaveM <= M;
        if constexpr (T::kWaves == 4 && std::is_same<TU, bf16>::value) {
            if (full) {
                // stores at a wave-uniform row-block base plus a per-lane 32-bit
                // byte offset (no per-row address arithmetic); the results of
                // rows 4 lq + e and + e + 1 share one bf16 conversion
                uint32_t off[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) off[e] = (uint32_t)((lq * 4 + e) * F + l16) * 2u;
#pragma unroll
                for (int i = 0; i < T::TM; ++i) {
                    uint8_t *base = (uint8_t *)(u + (size_t)(row0 + i * 16) * F + f0);
                    // the row block's 16 outputs as independent chains (the
                    // exponentials and reciprocals of one hide the others' latency)
                    float y[4][HJ], sa[4];
                    row_scales(i, sa);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int j = 0; j < HJ; ++j) {
                            const float z = val(i, j, e, sa);
                            y[e][j] = (ACT == 1 ? gelu_tanh_f(z) : silu_f(z)) * val(i, j + HJ, e, sa);
                        }
#pragma unroll
                    for (int e = 0; e < 4; e += 2)
#pragma unroll
                        for (int j = 0; j < HJ; ++j) {
                            uint32_t pk;   // both rounded to nearest even (the plain conversion's rounding)
                            asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(pk) : "v"(y[e][j]), "v"(y[e + 1][j]));
                            *(uint16_t *)(base + off[e] + j * 32) = (uint16_t)pk;
                            *(uint16_t *)(base + off[e + 1] + j * 32) = (uint16_t)(pk >> 16);
                        }
                    __builtin_amdgcn_sched_barrier(0);
                }
                return;
            }
        }
#pragma unroll
        for (int i = 0; i < T::TM; ++i) {
            if (full) row_block(i, false);
            else row_block(i, true);
            if constexpr (T::kWaves == 4) __builtin_amdgcn_sched_barrier(0);
        }
    }
};

// ---------------------------------------------------------------------------
// epilogue: qk-LayerNorm + RoPE, scatter to q [B,H,S,hd], k [B,Hk,S,hd],
// vt [B,Hk,hd,Spad], for the 8-wave 256 x 256 tile (wave tile 128 x 64).
// A head spans several waves' columns, so the accumulators go through LDS
// (free once the K loop has drained): each 4-wave cluster (128 rows) handles
// 64 of its rows x 256 columns at a time (two sub-passes), both clusters in
// parallel.  Per sub-pass:
//   1. the cluster's fp32 accumulators are staged in LDS;
//   2. each lane computes one unit of one head of the tile into registers:
//      q/k head: one token row, 64 values per lane (a 128-wide head row is
//                split over a lane pair that combines its LayerNorm
//                statistics with one exchange); the split keeps every RoPE
//                pair in one lane: interleaved pairs (2m, 2m+1) -> lane half
//                p holds columns [64p, 64p+64); rotate-half pairs (m, m+hd/2)
//                -> it holds [32p, 32p+32) and [hd/2+32p, hd/2+32p+32);
//      v head:   one head-dim column over the 64 staged tokens;
//   3. the bf16 results replace the staged values in LDS, laid out as they
//      are in memory (a q/k head: 64 rows x hd; a v head: hd rows x 64
//      tokens of v^T), and the cluster copies them out with lane-contiguous
//      16-byte stores (a q/k head of 64 tokens is one contiguous block, a v^T
//      row one 128-byte line).
// The LayerNorm gamma/beta of q and k sit in LDS behind the staging area
// (copied once per tile), and a lane's cos/sin row is loaded before the
// staging barrier, which waits for LDS traffic only, so those global loads
// overlap the staging.
// ---------------------------------------------------------------------------
constexpr int kQkvStride = 260;   // floats per staged row: 256 + 4, so 16 row-per-lane reads hit distinct banks

// RMS: qk-norm kind RMSNorm; RF: RoPE before the qk-norm; RH: rotate-half RoPE
// pairs (else interleaved); TQ: type of q, k, vt (fp32 on the fp32 parity path:
// written straight from registers, no LDS copy-out)
template <int HD, bool RMS, bool RF, bool RH, typename TQ = bf16>
struct EpiQkv {
    static constexpr bool kDequant = false;
    static constexpr bool kF32 = sizeof(TQ) == 4;
    QkvEpiArgs e;
    static constexpr int kStageBytes = 2 * 64 * kQkvStride * 4;
    static constexpr int kHeadBlock = 64 * HD * 2;        // bf16 bytes of one head x 64 tokens
    static constexpr int kRowChunks = HD / 8;             // 16-byte chunks per q/k output row
    template <class T> static constexpr int lds_bytes() { return kStageBytes + 4 * HD * 4; }

    // LDS slot of 16-byte chunk c of q/k output row r / of v^T row d
    static __device__ __forceinline__ int qk_slot(int r, int c) { return r * (HD * 2) + ((c ^ (r & (kRowChunks - 1))) << 4); }
    static __device__ __forceinline__ int v_slot(int d, int c) { return d * 128 + ((c ^ ((d >> 1) & 7)) << 4); }

    template <class T>
    __device__ __forceinline__ void apply(floatx4 (&acc)[T::TM][T::TN], int row0, int tn, int wn, int lane, int M,
                                          uint8_t *smem) const {
        static_assert(T::BN == 256 && T::WM == 2 && T::WN == 4 && (T::kWaveM == 128 || T::kWaveM == 64) &&
                          T::kWaveN == 64,
                      "staging assumes the 8-wave 256x256 tile or its 128-row tail variant");
        static_assert(2 * 64 * kQkvStride * 4 / 2 >= (256 / HD) * kHeadBlock, "output block fits the staging area");
        const int l16 = lane & 15, lq = lane >> 4;
        const int wave = threadIdx.x >> 6;
        const int cl = wave >> 2;                          // cluster = wm: rows cl*128 .. +128 of the tile
        const int lc = (wave & 3) * 64 + lane;             // lane within the cluster, 0..255
        float *red = (float *)smem + cl * 64 * kQkvStride;
        uint8_t *ob = (uint8_t *)red;                      // bf16 output blocks (same bytes, after the reads)
        const int qcols = e.heads * HD, kcols = e.kv_heads * HD;
        // section (0 q, 1 k, 2 v) and head index of head slot hs of this tile
        auto head_of = [&](int hs, int &sect, int &head) {
            const int c0 = tn * T::BN + hs * HD;
            sect = c0 < qcols ? 0 : (c0 < qcols + kcols ? 1 : 2);
            head = (c0 - (sect == 0 ? 0 : (sect == 1 ? qcols : qcols + kcols))) / HD;
        };
        const int hl = lc / HD, within = lc % HD;          // head slot of this lane, unit within that head
        int sect, head;
        head_of(hl, sect, head);                           // uniform per wave
        const int S = e.seq;
        // q_g, q_b, k_g, k_b (HD floats each); visible after the first staging barrier
        float *gb = (float *)(smem + kStageBytes);
        if (e.qk_norm) {
            for (int i = threadIdx.x; i < 4 * HD; i += T::kThreads) {
                const int which = i / HD, c = i - which * HD;
                const float *src = which == 0 ? e.q_g : (which == 1 ? e.q_b : (which == 2 ? e.k_g : e.k_b));
                gb[i] = src[c];
            }
        }
        constexpr int PARTS = HD / 64;                     // lanes per q/k head row
        const int rl = within / PARTS, part = within % PARTS;
        // the 32 RoPE pairs of this lane: rotate-half pairs pair0 .. pair0 + 31;
        // interleaved pairs in 4-pair runs, run q at 4 (PARTS q + part), so the
        // two lanes of a head row read chunks 32 bytes apart from the staged
        // row (distinct banks) rather than 256 bytes apart (the same banks)
        const int pair0 = part * 32;
#pragma unroll
        for (int sp = 0; sp < T::kWaveM / 64; ++sp) {
            // the K loop, or the previous sub-pass's copy-out, is done with the LDS
            if (sp > 0) { wait_vmcnt<63, 0>(); barrier_only(); }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        red[acc_row(ii, r, lq) * kQkvStride + wn * 64 + j * 16 + l16] = acc[sp * 4 + ii][j][r];
            const int rbase = row0 + sp * 64;             // token of staged row 0
            // (batch, position) of staged row r: one wave-uniform division per
            // sub-pass; with S >= 64 the 64-row window crosses at most one
            // batch boundary, so each row's position follows by a compare
            const int rb = min(rbase, M - 1);
            const int b0 = rb / S, s0 = rb - b0 * S;
            auto tok = [&](int r, int &bi, int &si) {
                if (S >= 64) {
                    si = s0 + r;
                    bi = b0;
                    if (si >= S) { si -= S; ++bi; }
                } else {
                    bi = (rb + r) / S;
                    si = rb + r - bi * S;
                }
            };
            int tb_, sp_;
            tok(min(rbase + rl, M - 1) - rb, tb_, sp_);
            const float *ct = e.cos_t + (size_t)sp_ * (HD / 2);
            const float *st = e.sin_t + (size_t)sp_ * (HD / 2);
            floatx4 cpre[8], spre[8];    // cos/sin of this lane's 32 pairs, loaded before the barrier
            if (sect < 2) {
#pragma unroll
                for (int m4 = 0; m4 < 8; ++m4) {
                    const int p4 = RH ? pair0 + m4 * 4 : (PARTS * m4 + part) * 4;
                    cpre[m4] = *(const floatx4 *)(ct + p4);
                    spre[m4] = *(const floatx4 *)(st + p4);
                }
            }
            wait_vmcnt<63, 0>();   // this wave's LDS writes done; global loads stay in flight
            barrier_only();

            bf16x8 o[8];           // this lane's 64 bf16 results, 8 at a time
            // column (within the head) of this lane's 8-value chunk q, q = 0..7
            auto qcol = [&](int q) {
                return RH ? (q < 4 ? pair0 + q * 8 : HD / 2 + pair0 + (q - 4) * 8) : (PARTS * q + part) * 8;
            };
            // fp32 path: chunk q (8 values) of this lane's q/k row straight to global memory
            auto store_f32 = [&](int q, const float (&y)[8]) {
                const int row = rbase + rl;
                if (row < M) {
                    const int bi = row / S, si = row - bi * S;
                    float *dst = (float *)(sect == 0 ? e.q : e.k) +
                                 (((size_t)bi * (sect == 0 ? e.heads : e.kv_heads) + head) * S + si) * HD + qcol(q);
                    *(floatx4 *)dst = floatx4{y[0], y[1], y[2], y[3]};
                    *(floatx4 *)(dst + 4) = floatx4{y[4], y[5], y[6], y[7]};
                }
            };
            if (sect < 2) {
                // The row is read from LDS once per pass (mean, centred variance,
                // output) instead of being held in registers.  A pair unit is one
                // 8-value chunk (interleaved pairs) or chunks q and q + 4
                // (rotate-half pairs); with rope_first the statistics and the
                // output see the rotated values.
                const float *src = red + rl * kQkvStride + hl * HD;
                constexpr bool rf = RF;
                auto raw = [&](int q, float (&y)[8]) {
                    const floatx4 v0 = *(const floatx4 *)(src + qcol(q)), v1 = *(const floatx4 *)(src + qcol(q) + 4);
#pragma unroll
                    for (int u = 0; u < 4; ++u) { y[u] = v0[u]; y[u + 4] = v1[u]; }
                };
                auto rot_il = [&](int q, float (&y)[8]) {          // pairs 4q .. 4q + 3 of this lane
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const int m = q * 4 + u;
                        const float cs = cpre[m >> 2][m & 3], sn = spre[m >> 2][m & 3];
                        const float a0 = y[2 * u], a1 = y[2 * u + 1];
                        y[2 * u] = a0 * cs - a1 * sn;
                        y[2 * u + 1] = a0 * sn + a1 * cs;
                    }
                };
                auto rot_half = [&](int q, float (&ya)[8], float (&yb)[8]) {   // pairs 8q .. 8q + 7
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int m = q * 8 + u;
                        const float cs = cpre[m >> 2][m & 3], sn = spre[m >> 2][m & 3];
                        const float a0 = ya[u], a1 = yb[u];
                        ya[u] = a0 * cs - a1 * sn;
                        yb[u] = a0 * sn + a1 * cs;
                    }
                };
                float mean = 0.f, rstd = 1.f;
                if (e.qk_norm) {
                    // pass 0: sum (LayerNorm only); pass 1: centred sum of squares
#pragma unroll
                    for (int pass = 0; pass < 2; ++pass) {
                        if (pass == 0 && RMS) continue;
                        float acc_ = 0.f;
                        auto add = [&](const float (&y)[8]) {
#pragma unroll
                            for (int u = 0; u < 8; ++u) acc_ += pass == 0 ? y[u] : (y[u] - mean) * (y[u] - mean);
                        };
                        if constexpr (!RH) {
#pragma unroll
                            for (int q = 0; q < 8; ++q) {
                                float y[8];
                                raw(q, y);
                                if (rf) rot_il(q, y);
                                add(y);
                            }
                        } else {
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                float ya[8], yb[8];
                                raw(q, ya);
                                raw(q + 4, yb);
                                if (rf) rot_half(q, ya, yb);
                                add(ya);
                                add(yb);
                            }
                        }
                        if (PARTS == 2) acc_ += __shfl_xor(acc_, 1, 64);
                        if (pass == 0) mean = acc_ * (1.0f / HD);
                        else rstd = rsqrtf(acc_ * (1.0f / HD) + e.eps);
                    }
                }
                const float *g = gb + (sect == 0 ? 0 : 2 * HD);
                const float *bb = g + HD;
                auto nrm = [&](int q, float (&y)[8]) {              // (y - mean) rstd gamma + beta
                    if (e.qk_norm) {
                        const int c = qcol(q);
                        const floatx4 g0 = *(const floatx4 *)(g + c), g1 = *(const floatx4 *)(g + c + 4);
                        const floatx4 b0 = *(const floatx4 *)(bb + c), b1 = *(const floatx4 *)(bb + c + 4);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            y[u] = (y[u] - mean) * rstd * g0[u] + b0[u];
                            y[u + 4] = (y[u + 4] - mean) * rstd * g1[u] + b1[u];
                        }
                    }
                };
                if constexpr (!RH) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        float y[8];
                        raw(q, y);
                        if (rf) { rot_il(q, y); nrm(q, y); } else { nrm(q, y); rot_il(q, y); }
                        if constexpr (kF32) {
                            store_f32(q, y);
                        } else {
#pragma unroll
                            for (int u = 0; u < 8; ++u) o[q][u] = f2bf(y[u]);
                        }
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float ya[8], yb[8];
                        raw(q, ya);
                        raw(q + 4, yb);
                        if (rf) {
                            rot_half(q, ya, yb);
                            nrm(q, ya);
                            nrm(q + 4, yb);
                        } else {
                            nrm(q, ya);
                            nrm(q + 4, yb);
                            rot_half(q, ya, yb);
                        }
                        if constexpr (kF32) {
                            store_f32(q, ya);
                            store_f32(q + 4, yb);
                        } else {
#pragma unroll
                            for (int u = 0; u < 8; ++u) { o[q][u] = f2bf(ya[u]); o[q + 4][u] = f2bf(yb[u]); }
                        }
                    }
                }
            } else {
                // v: head-dim column `within` over the 64 staged tokens
                const float *src = red + hl * HD + within;
                if constexpr (kF32) {
                    for (int r = 0; r < 64; ++r) {
                        const int row = rbase + r;
                        if (row < M) {
                            const int bi = row / S, si = row - bi * S;
                            ((float *)e.vt)[(((size_t)bi * e.kv_heads + head) * HD + within) * e.seq_pad + si] =
                                src[r * kQkvStride];
                        }
                    }
                } else {
#pragma unroll
                    for (int r8 = 0; r8 < 8; ++r8)
#pragma unroll
                        for (int u = 0; u < 8; ++u) o[r8][u] = f2bf(src[(r8 * 8 + u) * kQkvStride]);
                }
            }
            if constexpr (kF32) continue;   // fp32 results are already stored

            // 3. results into LDS in output order (after every lane's fp32 reads)
            wait_vmcnt<63, 0>();
            barrier_only();
            if (sect < 2) {
#pragma unroll
                for (int q = 0; q < 8; ++q) *(bf16x8 *)(ob + hl * kHeadBlock + qk_slot(rl, qcol(q) >> 3)) = o[q];
            } else {
#pragma unroll
                for (int r8 = 0; r8 < 8; ++r8) *(bf16x8 *)(ob + hl * kHeadBlock + v_slot(within, r8)) = o[r8];
            }
            wait_vmcnt<63, 0>();
            barrier_only();

            // copy-out: 16-byte piece pc of the cluster's (256 / HD) head blocks;
            // one wave's 64 pieces always lie in one head block
            const bool v_fast = (rbase + 63 < M) && (s0 + 63 < S) && ((s0 & 7) == 0);
#pragma unroll
            for (int it = 0; it < 8; ++it) {
                const int pc = it * 256 + lc;
                const int hs = pc / (kHeadBlock / 16), pw = pc - hs * (kHeadBlock / 16);
                int psect, phead;
                head_of(hs, psect, phead);
                if (psect < 2) {
                    const int r = pw / kRowChunks, c = pw - r * kRowChunks;
                    const int row = rbase + r;
                    if (row < M) {
                        int bi, si;
                        tok(r, bi, si);
                        bf16 *dst = (bf16 *)(psect == 0 ? e.q : e.k) +
                                    (((size_t)bi * (psect == 0 ? e.heads : e.kv_heads) + phead) * S + si) * HD + c * 8;
                        *(bf16x8 *)dst = *(const bf16x8 *)(ob + hs * kHeadBlock + qk_slot(r, c));
                    }
                } else {
                    const int d = pw >> 3, c = pw & 7;
                    const bf16x8 v = *(const bf16x8 *)(ob + hs * kHeadBlock + v_slot(d, c));
                    if (v_fast) {
                        *(bf16x8 *)((bf16 *)e.vt + (((size_t)b0 * e.kv_heads + phead) * HD + d) * e.seq_pad + s0 + c * 8) = v;
                    } else {
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const int row = rbase + c * 8 + u;
                            if (row < M) {
                                int bi, si;
                                tok(c * 8 + u, bi, si);
                                ((bf16 *)e.vt)[(((size_t)bi * e.kv_heads + phead) * HD + d) * e.seq_pad + si] = v[u];
                            }
                        }
                    }
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Split QKV (bf16, 4-wave tile): the GEMM epilogue only rounds and scatters,
// q and k to [B, H, S, hd] and v to v^T [B, Hk, hd, seq_pad]; qk_norm_rope_kernel
// then applies the qk-norm and RoPE to the q and k rows in place.  Each wave's
// 128 columns hold 128 / hd whole heads; a lane stores rows 4 lq + e of column
// l16 of each 16 x 16 block, from a wave-uniform base plus lane offsets: q / k
// with one 2-byte store per value (row pairs share one conversion), v^T with
// one 8-byte store of four consecutive tokens.
// ---------------------------------------------------------------------------
template <int HD>
struct EpiQkvRaw {
    static constexpr bool kDequant = false;
    QkvEpiArgs e;
    // int8 operands: row and W-row scales of the int32 sums (Tile4wQ)
    const float *a_scale = nullptr, *w_scale = nullptr;
    template <class T> static constexpr int lds_bytes() { return 0; }
    // Taken only when every 16-row block lies in one sequence and below M (a
    // single sequence, or a sequence length that is a multiple of 16, and M a
    // multiple of 16); a block's first position is then a multiple of 4, so
    // v^T's 4-token groups are 8-byte aligned.
    template <class T>
    __device__ __forceinline__ void apply(floatx4 (&acc)[T::TM][T::TN], int row0, int tn, int wn, int lane, int M,
                                          uint8_t *) const {
        static_assert(T::kAgpr && T::TN == 8 && T::kWaveN % HD == 0, "the 4-wave tile, whole heads per wave");
        const int l16 = lane & 15, lq = lane >> 4;
        const int S = e.seq, spad = e.seq_pad;
        const int qcols = e.heads * HD, kcols = e.kv_heads * HD;
        // per column block: section (0 q, 1 k, 2 v) and the byte address of its
        // first column at sequence 0, position 0 (wave-uniform)
        int sect[T::TN];
        uint8_t *cbase[T::TN];
        // int8 operands: C[m, n] = sum * (a_scale[m] w_scale[n]), converted and
        // scaled where each sum is read (the same products as the 8-wave kernel)
        constexpr bool kQ = T::ES == 1;
        float sw[kQ ? T::TN : 1];
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int c0 = tn * T::BN + wn * T::kWaveN + j * 16;
            if constexpr (kQ) sw[j] = w_scale[c0 + l16];
            sect[j] = c0 < qcols ? 0 : (c0 < qcols + kcols ? 1 : 2);
            const int cs = c0 - (sect[j] == 0 ? 0 : (sect[j] == 1 ? qcols : qcols + kcols));
            const int head = cs / HD, d0 = cs - head * HD;
            cbase[j] = sect[j] == 2 ? (uint8_t *)((bf16 *)e.vt + ((size_t)head * HD + d0) * spad)
                                    : (uint8_t *)((bf16 *)(sect[j] == 0 ? e.q : e.k) + ((size_t)head * S * HD + d0));
        }
        // lane byte offsets: q / k rows 4 lq + e are HD apart; a v^T row holds
        // one column's tokens, the lane's four adjacent
        uint32_t qo[4];
#pragma unroll
        for (int e_ = 0; e_ < 4; ++e_) qo[e_] = (uint32_t)((lq * 4 + e_) * HD + l16) * 2u;
        const uint32_t vo = ((uint32_t)l16 * (uint32_t)spad + (uint32_t)lq * 4u) * 2u;
        auto row_scales = [&](int i, float (&sa)[4]) {
            if constexpr (kQ) {
#pragma unroll
                for (int e_ = 0; e_ < 4; ++e_) sa[e_] = a_scale[min(row0 + acc_row(i, e_, lq), M - 1)];
            }
        };
        auto val = [&](int i, int j, int e_, const float (&sa)[4]) -> float {
            if constexpr (kQ)
                return (float)__builtin_bit_cast(int, acc_get<T>(acc[i][j], e_)) * (sa[e_] * sw[j]);
            else
                return acc_get<T>(acc[i][j], e_);
        };
        // SEC: the section of every block of the wave (0 q, 1 k, 2 v), or -1 for a
        // wave whose columns cross a section boundary (hd 64 only).  Stores are
        // ordered so that each 128-byte line is written by consecutive stores
        // (whole lines reach L2 together, no partial-line write-backs): a q / k
        // row's column blocks back to back, a v^T row's 16-token pieces back to
        // back (the row blocks innermost).
        auto offsets = [&](int i, size_t &oq, size_t &ok, size_t &ov) {
            const int t0 = row0 + i * 16;
            const int b0 = t0 / S, s0 = t0 - b0 * S;
            oq = ((size_t)b0 * e.heads * S + s0) * HD * 2;
            ok = ((size_t)b0 * e.kv_heads * S + s0) * HD * 2;
            ov = ((size_t)b0 * e.kv_heads * HD * spad + s0) * 2;
        };
        auto store = [&](auto sec_c) {
            constexpr int SEC = decltype(sec_c)::value;
            if constexpr (SEC == 2) {
                size_t ov[T::TM];
                float sa[T::TM][4];
#pragma unroll
                for (int i = 0; i < T::TM; ++i) {
                    size_t oq_, ok_;
                    offsets(min(i, (M - 1 - row0) / 16), oq_, ok_, ov[i]);   // (rows past M: not stored)
                    row_scales(i, sa[i]);
                }
#pragma unroll
                for (int j = 0; j < T::TN; ++j) {
#pragma unroll
                    for (int i = 0; i < T::TM; ++i) {
                        if (row0 + i * 16 < M) {
                            uint32_t p0, p1;
                            asm("v_cvt_pk_bf16_f32 %0, %1, %2"
                                : "=v"(p0) : "v"(val(i, j, 0, sa[i])), "v"(val(i, j, 1, sa[i])));
                            asm("v_cvt_pk_bf16_f32 %0, %1, %2"
                                : "=v"(p1) : "v"(val(i, j, 2, sa[i])), "v"(val(i, j, 3, sa[i])));
                            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                            *(u32x2 *)(cbase[j] + ov[i] + vo) = u32x2{p0, p1};
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
#pragma unroll
                for (int i = 0; i < T::TM; ++i) {
                    if (row0 + i * 16 < M) {
                        size_t oq, ok, ov;
                        offsets(i, oq, ok, ov);
                        float sa[4];
                        row_scales(i, sa);
                        if constexpr (SEC >= 0) {
                            // rows 4 lq + e (pairs share a conversion), each row's
                            // column blocks stored back to back
                            uint32_t pk[T::TN][2];
#pragma unroll
                            for (int j = 0; j < T::TN; ++j)
#pragma unroll
                                for (int h = 0; h < 2; ++h)
                                    asm("v_cvt_pk_bf16_f32 %0, %1, %2"
                                        : "=v"(pk[j][h])
                                        : "v"(val(i, j, 2 * h, sa)), "v"(val(i, j, 2 * h + 1, sa)));
#pragma unroll
                            for (int e_ = 0; e_ < 4; ++e_)
#pragma unroll
                                for (int j = 0; j < T::TN; ++j) {
                                    uint8_t *base = cbase[j] + (SEC == 0 ? oq : ok);
                                    const uint32_t w = pk[j][e_ >> 1];
                                    *(uint16_t *)(base + qo[e_]) = (uint16_t)((e_ & 1) ? (w >> 16) : w);
                                }
                        } else {
#pragma unroll
                            for (int j = 0; j < T::TN; ++j) {
                                float z[4];
#pragma unroll
                                for (int e_ = 0; e_ < 4; ++e_) z[e_] = val(i, j, e_, sa);
                                if (sect[j] < 2) {
                                    uint8_t *base = cbase[j] + (sect[j] == 0 ? oq : ok);
#pragma unroll
                                    for (int e_ = 0; e_ < 4; e_ += 2) {
                                        uint32_t pk;
                                        asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(pk) : "v"(z[e_]), "v"(z[e_ + 1]));
                                        *(uint16_t *)(base + qo[e_]) = (uint16_t)pk;
                                        *(uint16_t *)(base + qo[e_ + 1]) = (uint16_t)(pk >> 16);
                                    }
                                } else {
                                    uint32_t p0, p1;
                                    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(p0) : "v"(z[0]), "v"(z[1]));
                                    asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(p1) : "v"(z[2]), "v"(z[3]));
                                    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                                    *(u32x2 *)(cbase[j] + ov + vo) = u32x2{p0, p1};
                                }
                            }
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        if (sect[0] != sect[T::TN - 1]) store(std::integral_constant<int, -1>{});
        else if (sect[0] == 0) store(std::integral_constant<int, 0>{});
        else if (sect[0] == 1) store(std::integral_constant<int, 1>{});
        else store(std::integral_constant<int, 2>{});
    }
};

// In-place qk-norm and RoPE over the q and k rows of tokens [0, m_end) that the
// split QKV projection wrote (same arithmetic as the fused QKV epilogue, on the
// bf16-rounded projection).  A row of HD values is HD / 8 lanes of 8 values
// (one 16-byte chunk each); statistics by butterflies over those lanes.
// Interleaved RoPE pairs (2m, 2m + 1) lie in one lane; rotate-half pairs
// (m, m + HD / 2) in lanes HD / 16 apart.  A workgroup takes 256 / (HD / 8)
// consecutive tokens (one per lane group) and kGroup of the q and k heads
// (q heads first): a lane group loads its token's cos / sin and both norms'
// gamma / beta once, then its kGroup rows, all loads in flight together.
constexpr int kQkNormGroup = 8;
// v from lane (lane ^ 1), (lane ^ 2), the mirror in its 8 / 16 lanes, lane ^ 8 (DPP)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// sum over aligned groups of W = 8 or 16 lanes, the same value in every lane
template <int W>
__device__ __forceinline__ float dpp_group_sum(float v) {
    static_assert(W == 8 || W == 16, "lane group");
    v += dpp_f32<0xB1>(v);          // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);          // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);         // row_half_mirror: the other quad of the 8
    if constexpr (W == 16) v += dpp_f32<0x140>(v);   // row_mirror: the other 8 of the 16
    return v;
}
template <int HD, bool RMS, bool RF, bool RH>
__global__ __launch_bounds__(256)
void qk_norm_rope_kernel(QkvEpiArgs e, int m_end) {
    constexpr int LPR = HD / 8;                  // lanes per row
    constexpr int TPB = 256 / LPR;               // tokens per workgroup
    const int li = threadIdx.x % LPR;
    const int t = blockIdx.x * TPB + threadIdx.x / LPR;    // token, < m_end <= 2^31
    if (t >= m_end) return;                      // whole lane groups leave together
    const int S = e.seq;
    const int b = t / S, si = t - b * S;
    const int h0 = blockIdx.y * kQkNormGroup, nh = e.heads + e.kv_heads;
    bf16 *ptr[kQkNormGroup];
    bf16x8 raw[kQkNormGroup];
#pragma unroll
    for (int g = 0; g < kQkNormGroup; ++g) {
        const int hh = min(h0 + g, nh - 1);       // (a short last group repeats its last head, not stored twice)
        ptr[g] = hh < e.heads ? (bf16 *)e.q + (((size_t)b * e.heads + hh) * S + si) * HD + li * 8
                              : (bf16 *)e.k + (((size_t)b * e.kv_heads + (hh - e.heads)) * S + si) * HD + li * 8;
        raw[g] = *(const bf16x8 *)ptr[g];
    }
    // this lane's RoPE coefficients: 4 interleaved pairs or 8 rotate-half pairs
    const float *ct = e.cos_t + (size_t)si * (HD / 2), *st = e.sin_t + (size_t)si * (HD / 2);
    constexpr int H2 = LPR / 2;                  // lanes per half row (rotate-half)
    const bool lo = li < H2;
    const int m0 = RH ? (lo ? li : li - H2) * 8 : li * 4;
    const floatx4 c0 = *(const floatx4 *)(ct + m0);
    floatx4 s0 = *(const floatx4 *)(st + m0);
    floatx4 c1 = c0, s1 = s0;
    if constexpr (RH) {
        // rotate-half: the first half takes own cos - partner sin, the second
        // partner sin + own cos, i.e. own cos + partner (-+ sin)
        c1 = *(const floatx4 *)(ct + m0 + 4);
        s1 = *(const floatx4 *)(st + m0 + 4);
        if (lo) { s0 = -s0; s1 = -s1; }
    }
    // rows g0 .. g1 - 1 of the group, all q rows (Q = 1) or all k rows (Q = 0)
    auto rows = [&](int g0, int g1, auto q_c) {
        constexpr bool Q = decltype(q_c)::value;
        floatx4 ga = {}, gb = {}, ba = {}, bb = {};
        if (e.qk_norm) {
            const float *g = Q ? e.q_g : e.k_g, *be = Q ? e.q_b : e.k_b;
            ga = *(const floatx4 *)(g + li * 8), gb = *(const floatx4 *)(g + li * 8 + 4);
            ba = *(const floatx4 *)(be + li * 8), bb = *(const floatx4 *)(be + li * 8 + 4);
        }
#pragma unroll
        for (int g = 0; g < kQkNormGroup; ++g) {
            if (g < g0 || g >= g1) continue;
            float y[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) y[u] = (float)raw[g][u];
            auto rope = [&]() {
                if constexpr (!RH) {
#pragma unroll
                    for (int u = 0; u < 4; ++u) {
                        const float a0 = y[2 * u], a1 = y[2 * u + 1];
                        y[2 * u] = a0 * c0[u] - a1 * s0[u];
                        y[2 * u + 1] = a0 * s0[u] + a1 * c0[u];
                    }
                } else {
                    static_assert(H2 == 8, "rotate-half partner lane ^ 8");
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float other = dpp_f32<0x128>(y[u]);   // row_ror 8: lane ^ 8 of 16
                        const float cs = u < 4 ? c0[u] : c1[u - 4], sn = u < 4 ? s0[u] : s1[u - 4];
                        y[u] = y[u] * cs + other * sn;
                    }
                }
            };
            if (RF) rope();
            if (e.qk_norm) {
                float mean = 0.f;
                if constexpr (!RMS) {
                    float a = 0.f;
#pragma unroll
                    for (int u = 0; u < 8; ++u) a += y[u];
                    mean = dpp_group_sum<LPR>(a) * (1.0f / HD);
                }
                float v = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) v += (y[u] - mean) * (y[u] - mean);
                const float rstd = rsqrtf(dpp_group_sum<LPR>(v) * (1.0f / HD) + e.eps);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    y[u] = (y[u] - mean) * rstd * ga[u] + ba[u];
                    y[u + 4] = (y[u + 4] - mean) * rstd * gb[u] + bb[u];
                }
            }
            if (!RF) rope();
            bf16x8 o;
#pragma unroll
            for (int u = 0; u < 8; ++u) o[u] = f2bf(y[u]);
            *(bf16x8 *)ptr[g] = o;
        }
    };
    // q rows: heads h0 .. min(heads, h0 + group); k rows after them (group-uniform)
    const int nq = min(max(e.heads - h0, 0), kQkNormGroup), nall = min(nh - h0, kQkNormGroup);
    if (nq > 0) rows(0, nq, std::true_type{});
    if (nall > nq) rows(nq, nall, std::false_type{});
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// 8 waves (2 per SIMD, 128x64 each): two waves per SIMD let one wave's LDS
// waits overlap the other's MFMAs.
using Tile8w = Tile<256, 256, 2, 4>;
using Tile8wTall = Tile<320, 256, 2, 4>;   // 160 x 64 per wave: ragged row counts just above a multiple of 256
// 128-row tiles (8 waves of 64 x 64): ragged row tails, few-tile shapes; bf16
// over 3 LDS stages (144 KiB: with half the MFMA work of a 256-row tile per
// stage, loads two stages ahead are what keeps the MFMAs fed)
using Tile8wHalf = Tile<128, 256, 2, 4, 64, 3>;
// Narrow and quarter tiles for shapes with few 256 x 256 tiles, also 8 waves:
// 256 x 128 as 128 x 32 per wave over 3 LDS stages (144 KiB); 128 x 128 as
// 32 x 64 per wave, over 2 stages (64 KiB: two workgroups fit on a CU, which
// pays when the launch has more tiles than CUs) or over 3 stages (96 KiB: one
// workgroup per CU, so a launch of at most one tile per CU spreads over all of
// them instead of doubling up on some).
using Tile8wNarrow = Tile<256, 128, 2, 4, 64, 3>;
using Tile8wQuarter = Tile<128, 128, 4, 2>;
using Tile8wQuarter3 = Tile<128, 128, 4, 2, 64, 3>;
// the int8 and fp32 families keep 4-wave narrow and quarter tiles
using TileNarrow = Tile<256, 128, 2, 2>;
// the same tiles over int8 operands (128 int8 per 128-byte row)
using Tile8wQ = Tile<256, 256, 2, 4, 128, 2, 1>;
using Tile8wTallQ = Tile<320, 256, 2, 4, 128, 2, 1>;
using TileNarrowQ = Tile<256, 128, 2, 2, 128, 2, 1>;
using Tile8wHalfQ = Tile<128, 256, 2, 4, 128, 2, 1>;
using TileQuarterQ = Tile<128, 128, 2, 2, 128, 2, 1>;

// The tile family of an operand format: 0 bf16, 1 int8 (W8A8), 2 fp32 (the
// fp32 parity path: 32 floats of K per 128-byte LDS row, fp32 MFMA)
template <int FMT> struct TileSet;
// Quar1: the quarter tile for launches of at most one tile per CU.
template <> struct TileSet<0> {
    using S = Tile8w; using Tall = Tile8wTall; using Nar = Tile8wNarrow; using Half = Tile8wHalf;
    using Quar = Tile8wQuarter; using Quar1 = Tile8wQuarter3;
};
template <> struct TileSet<1> {
    using S = Tile8wQ; using Tall = Tile8wTallQ; using Nar = TileNarrowQ; using Half = Tile8wHalfQ;
    using Quar = TileQuarterQ; using Quar1 = TileQuarterQ;
};
template <> struct TileSet<2> {
    using S = Tile<256, 256, 2, 4, 32, 2, 4>; using Tall = Tile<320, 256, 2, 4, 32, 2, 4>;
    using Nar = Tile<256, 128, 2, 2, 32, 2, 4>; using Half = Tile<128, 256, 2, 4, 32, 2, 4>;
    using Quar = Tile<128, 128, 2, 2, 32, 2, 4>; using Quar1 = Quar;
};

// Tile choice for an M x N output.  Every tile of a launch costs about the
// same, so the time is the number of rounds of workgroups over the CUs times
// the cost of one tile: its area over its throughput relative to the 256 x 256
// tile, measured at shapes that fill the chip (320 x 256: 1.0; 128 x 256 and
// 256 x 128: 0.87 and 0.86 for the 3-stage bf16 tiles, 0.69 for the int8 /
// fp32 ones; 128 x 128: 0.775; N(0, 1) x N(0, 0.02)).  E.g.
// 4170 x 4096 takes the 320-row tile (224 tiles in one round instead of 272 in
// two), 4096 x 1024 the 128 x 128 tile (256 tiles instead of 64), 1024 x 6144
// the 256 x 128 tile (192 tiles in one round), 1024 x 8192 QKV the 128 x 256
// tile; the 256 x 256 tile wins ties.
enum TileKind { kTileS, kTileTall, kTileHalf, kTileNar, kTileQuar };
struct TileCand {
    TileKind kind;
    int bm, bn;
    double rate;
};
constexpr TileCand kTileCands[] = {{kTileS, 256, 256, 1.0},    {kTileTall, 320, 256, 1.0},
                                   {kTileHalf, 128, 256, 0.69}, {kTileNar, 256, 128, 0.69},
                                   {kTileQuar, 128, 128, 0.775}};

// mask: bit k allows TileKind k; fmt: the operand format (TileSet index)
static TileKind choose_tile(int64_t M, int N, unsigned mask, int fmt = 0, double *cost_out = nullptr) {
    const int64_t cus = device_cu_count();
    TileKind best = kTileS;
    double best_cost = 0.0;
    bool have = false;
    for (const TileCand &c : kTileCands) {
        if (!(mask >> c.kind & 1u) || N % c.bn) continue;
        const double rate = fmt != 0 ? c.rate : c.kind == kTileNar ? 0.86 : c.kind == kTileHalf ? 0.87 : c.rate;
        const int64_t tiles = (M + c.bm - 1) / c.bm * (N / c.bn);
        const double cost = (double)((tiles + cus - 1) / cus) * c.bm * c.bn / rate;
        if (!have || cost < best_cost) {
            best = c.kind;
            best_cost = cost;
            have = true;
        }
    }
    if (cost_out) *cost_out = best_cost;
    return best;
}
constexpr unsigned kAllTiles = 0x1f;

// at most one 128 x 128 tile per CU: the quarter tile variant that keeps one
// workgroup per CU
static bool quarter_one_round(int64_t M, int N) {
    return (M + 127) / 128 * (N / 128) <= (int64_t)device_cu_count();
}

// int8 operands carry their row scales (Scales), bf16 (NoScales) and fp32
// (F32Ops) operands none
struct NoScales {
    static constexpr bool kQ8 = false;
    static constexpr int kFmt = 0;
    const float *a = nullptr, *w = nullptr;
};
struct Scales {
    static constexpr bool kQ8 = true;
    static constexpr int kFmt = 1;
    const float *a, *w;
};
struct F32Ops {
    static constexpr bool kQ8 = false;
    static constexpr int kFmt = 2;
    const float *a = nullptr, *w = nullptr;
};

// rows [m_base, M) in tiles of T::BM
template <class T, class RowMap, class Epi>
static hipError_t run(const void *a, const void *w, int64_t M, int N_tile_cols, int K, RowMap rm, Epi epi,
                      hipStream_t s, const float *a_scale = nullptr, const float *w_scale = nullptr,
                      int64_t m_base = 0) {
    const int tiles_m = (int)((M - m_base + T::BM - 1) / T::BM);
    const int tiles_n = N_tile_cols / T::BN;
    const int grid = tiles_m * tiles_n;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel<T, RowMap, Epi>), dim3(grid), dim3(T::kThreads), 0, s, a, w, (int)M, K,
                       N_tile_cols, tiles_m, tiles_n, rm, epi, a_scale, w_scale, (int)m_base);
    return hipGetLastError();
}

template <class T, class RowMap, class Epi>
static hipError_t run4(const void *a, const void *w, int64_t M, int N_tile_cols, int K, RowMap rm, Epi epi,
                       hipStream_t s, int64_t m_base = 0) {
    const int tiles_m = (int)((M - m_base + T::BM - 1) / T::BM);
    const int tiles_n = N_tile_cols / T::BN;
    const int ntiles = tiles_m * tiles_n;
    if (ntiles == 0) return hipSuccess;
    // persistent workgroups, one per CU (a multiple of 8, one per XCD in turn)
    int grid = (int)std::min<int64_t>(ntiles, device_cu_count());
    if (grid < ntiles && grid >= 8) grid -= grid % 8;
    hipLaunchKernelGGL((gemm4_kernel<T, RowMap, Epi>), dim3(grid), dim3(T::kThreads), 0, s, a, w, (int)M, K,
                       N_tile_cols, tiles_m, tiles_n, rm, epi, (int)m_base);
    return hipGetLastError();
}

// Ragged row count (e.g. 4096 image + 74 text tokens): the last, partial row
// of 256-row tiles costs a whole extra round of workgroups when the full rows
// already fill whole rounds.  Then the full rows run as usual and the tail
// rows in a second launch of 128-row tiles (TH, same columns and wave layout)
// at about half the cost per tile.  Used for the QKV GEMM (4170 x 12288:
// 405 instead of 427 us).
static bool split_tail_rows(int64_t M, int N_tile_cols) {
    if (M % 256 == 0 || M % 256 > 128 || M < 256) return false;
    const int64_t cus = device_cu_count(), tn = N_tile_cols / 256;
    const int64_t full = M / 256 * tn, tail = tn;
    const double plain = (double)((full + tail + cus - 1) / cus);
    const double split = (double)((full + cus - 1) / cus) + 0.55 * (double)((tail + cus - 1) / cus);
    return split < plain;
}

template <class T, class TH, class RowMap, class Epi>
static hipError_t run_tail_split(const void *a, const void *w, int64_t M, int N_tile_cols, int K, RowMap rm,
                                 Epi epi, hipStream_t s, const float *a_scale = nullptr,
                                 const float *w_scale = nullptr) {
    static_assert(T::BM == 256 && TH::BM == 128 && T::BN == TH::BN, "full and tail tiles");
    constexpr int kFmt = T::ES == 2 ? 0 : (T::ES == 1 ? 1 : 2);
    // few row tiles (e.g. 1024 x 8192): every row in 128-row tiles
    if (choose_tile(M, N_tile_cols, 1u << kTileS | 1u << kTileHalf, kFmt) == kTileHalf)
        return run<TH>(a, w, M, N_tile_cols, K, rm, epi, s, a_scale, w_scale);
    if (!split_tail_rows(M, N_tile_cols)) return run<T>(a, w, M, N_tile_cols, K, rm, epi, s, a_scale, w_scale);
    const int64_t m_full = M / 256 * 256;
    hipError_t e = run<T>(a, w, m_full, N_tile_cols, K, rm, epi, s, a_scale, w_scale);
    if (e != hipSuccess) return e;
    return run<TH>(a, w, M, N_tile_cols, K, rm, epi, s, a_scale, w_scale, m_full);
}

// Column split of a bf16 residual launch whose 256 x 256 tiles fill whole
// rounds only over part of the columns (e.g. 4096 x 6144: 384 tiles = 1.5
// rounds): the first n0 columns in 256 x 256 tiles (whole rounds), the rest
// by its own tile choice, as two launches over offset W rows and output
// columns (same row stride).  4096 x 6144: one round of 256 x 256 plus one of
// 128 x 256 instead of three rounds of 128 x 256.  Returns n0, or 0 when a
// single launch models as fast (within 5 %).
static int residual_column_split(int64_t M, int N) {
    const int64_t cus = device_cu_count(), tm = (M + 255) / 256;
    if (N % 256 || tm > cus || cus % tm) return 0;
    const int64_t per_round = cus / tm, ct = N / 256;   // 256-column tiles per round, in all
    const int64_t n0 = ct / per_round * per_round * 256;
    if (n0 == 0 || n0 == N) return 0;
    double whole = 0.0, rest = 0.0;
    choose_tile(M, N, kAllTiles, 0, &whole);
    choose_tile(M, (int)(N - n0), kAllTiles, 0, &rest);
    const double split = (double)(n0 / 256 / per_round) * 65536.0 + rest;
    return split < 0.95 * whole ? (int)n0 : 0;
}

template <typename TR, typename TO, class SC>
static hipError_t residual_typed(const void *a, const void *w, int64_t M, int N, int K, const void *resid,
                                 const float *gate, int gate_fn, const float *bias, void *out, SC sc,
                                 hipStream_t s, int n0 = 0, int n_cols = 0) {
    using TSet = TileSet<SC::kFmt>;
    if (n_cols == 0) {   // the whole output, or its column split
        n_cols = N;
        if constexpr (SC::kFmt == 0) {
            const int c0 = residual_column_split(M, N);
            if (c0) {
                const hipError_t e = residual_typed<TR, TO>(a, w, M, N, K, resid, gate, gate_fn, bias, out, sc, s,
                                                            0, c0);
                if (e != hipSuccess) return e;
                return residual_typed<TR, TO>(a, w, M, N, K, resid, gate, gate_fn, bias, out, sc, s, c0, N - c0);
            }
        }
    }
    // columns [n0, n0 + n_cols) of the [M, N] output: W rows, output, residual,
    // gate and bias offset by n0, the row stride stays N
    if (n0) {
        w = (const uint8_t *)w + (size_t)n0 * K * TSet::S::ES;
        resid = resid ? (const void *)((const TR *)resid + n0) : nullptr;
        out = (TO *)out + n0;
        gate = gate ? gate + n0 : nullptr;
        bias = bias ? bias + n0 : nullptr;
    }
    EpiResidual<TR, TO, SC::kQ8> epi{(const TR *)resid, gate, bias, (TO *)out, N, gate_fn, sc.a, sc.w};
    const int Nc = n_cols;
    switch (choose_tile(M, Nc, kAllTiles, SC::kFmt)) {
        case kTileTall: return run<typename TSet::Tall>(a, w, M, Nc, K, RowsIdentity<256>{}, epi, s, sc.a, sc.w);
        case kTileHalf: return run<typename TSet::Half>(a, w, M, Nc, K, RowsIdentity<256>{}, epi, s, sc.a, sc.w);
        case kTileNar: return run<typename TSet::Nar>(a, w, M, Nc, K, RowsIdentity<128>{}, epi, s, sc.a, sc.w);
        case kTileQuar:
            if (quarter_one_round(M, Nc))
                return run<typename TSet::Quar1>(a, w, M, Nc, K, RowsIdentity<128>{}, epi, s, sc.a, sc.w);
            return run<typename TSet::Quar>(a, w, M, Nc, K, RowsIdentity<128>{}, epi, s, sc.a, sc.w);
        default:
            if constexpr (SC::kFmt == 0) return run4<Tile4w>(a, w, M, Nc, K, RowsIdentity<256>{}, epi, s);
            if constexpr (SC::kFmt == 1) return run4<Tile4wQ>(a, w, M, Nc, K, RowsIdentity<256>{}, epi, s);
            return run<typename TSet::S>(a, w, M, Nc, K, RowsIdentity<256>{}, epi, s, sc.a, sc.w);
    }
}

template <class SC>
static hipError_t residual_any(const void *a, const void *w, int64_t M, int N, int K, const void *resid,
                               int resid_f32, const float *gate, int gate_fn, const float *bias, void *out,
                               int out_f32, SC sc, hipStream_t s) {
    if constexpr (SC::kFmt == 2) {   // fp32 path: fp32 residual stream only
        if (!out_f32 || (resid && !resid_f32)) return hipErrorInvalidValue;
        return residual_typed<float, float>(a, w, M, N, K, resid, gate, gate_fn, bias, out, sc, s);
    } else {
        if (resid_f32) {
            return out_f32 ? residual_typed<float, float>(a, w, M, N, K, resid, gate, gate_fn, bias, out, sc, s)
                           : residual_typed<float, bf16>(a, w, M, N, K, resid, gate, gate_fn, bias, out, sc, s);
        }
        return out_f32 ? residual_typed<bf16, float>(a, w, M, N, K, resid, gate, gate_fn, bias, out, sc, s)
                       : residual_typed<bf16, bf16>(a, w, M, N, K, resid, gate, gate_fn, bias, out, sc, s);
    }
}

hipError_t launch_gemm_residual(const bf16 *a, const bf16 *w, int64_t M, int N, int K, const void *resid,
                                int resid_f32, const float *gate, int gate_fn, const float *bias, void *out,
                                int out_f32, hipStream_t s) {
    TraceScope trace_(s, "gemm_gated_residual");
    if (trace_.on()) trace_.args("M=%lld N=%d K=%d", (long long)M, N, K);
    return residual_any(a, w, M, N, K, resid, resid_f32, gate, gate_fn, bias, out, out_f32, NoScales{}, s);
}

hipError_t launch_gemm_residual_f32(const float *a, const float *w, int64_t M, int N, int K, const float *resid,
                                    const float *gate, int gate_fn, const float *bias, float *out, hipStream_t s) {
    TraceScope trace_(s, "gemm_gated_residual_f32");
    if (trace_.on()) trace_.args("M=%lld N=%d K=%d", (long long)M, N, K);
    return residual_any(a, w, M, N, K, resid, 1, gate, gate_fn, bias, out, 1, F32Ops{}, s);
}

hipError_t launch_gemm_residual_q8(const int8_t *a, const float *a_scale, const int8_t *w, const float *w_scale,
                                   int64_t M, int N, int K, const void *resid, int resid_f32, const float *gate,
                                   int gate_fn, const float *bias, void *out, int out_f32, hipStream_t s) {
    TraceScope trace_(s, "gemm_gated_residual_w8a8");
    if (trace_.on()) trace_.args("M=%lld N=%d K=%d", (long long)M, N, K);
    return residual_any(a, w, M, N, K, resid, resid_f32, gate, gate_fn, bias, out, out_f32,
                        Scales{a_scale, w_scale}, s);
}

template <class SC, typename TU>
static hipError_t swiglu_any(const void *a, const void *w, int64_t M, int F, int K, int act, TU *u, SC sc,
                             hipStream_t s) {
    using TSet = TileSet<SC::kFmt>;
    auto go = [&](auto tile, auto epi) {
        using T = decltype(tile);
        return run<T>(a, w, M, 2 * F, K, RowsSwiglu<T::BN, T::kWaveN>{F}, epi, s, sc.a, sc.w);
    };
    auto with_act = [&](auto tile) {
        return act == 1 ? go(tile, EpiSwiglu<1, TU>{u, F}) : go(tile, EpiSwiglu<0, TU>{u, F});
    };
    switch (choose_tile(M, 2 * F, kAllTiles, SC::kFmt)) {
        case kTileTall: return with_act(typename TSet::Tall{});
        case kTileHalf: return with_act(typename TSet::Half{});
        case kTileNar: return with_act(typename TSet::Nar{});
        case kTileQuar:
            if (quarter_one_round(M, 2 * F)) return with_act(typename TSet::Quar1{});
            return with_act(typename TSet::Quar{});
        default:
            if constexpr (SC::kFmt != 2) {
                // bf16 and int8: the 4-wave tile; a ragged tail that would cost a
                // whole round of 256-row tiles runs as a second launch of 128 x 256
                // tiles (4170 x 24576: 7 rounds of 256-row tiles become 6 plus a
                // short one)
                using T4 = std::conditional_t<SC::kFmt == 0, Tile4w, Tile4wQ>;
                using TH = typename TSet::Half;
                const bool split = split_tail_rows(M, 2 * F);
                const int64_t m_full = split ? M / 256 * 256 : M;
                auto launch = [&](auto epi) {
                    const hipError_t e =
                        run4<T4>(a, w, m_full, 2 * F, K, RowsSwiglu<T4::BN, T4::kWaveN>{F}, epi, s);
                    if (e != hipSuccess || !split) return e;
                    return run<TH>(a, w, M, 2 * F, K, RowsSwiglu<TH::BN, TH::kWaveN>{F}, epi, s, sc.a, sc.w, m_full);
                };
                return act == 1 ? launch(EpiSwiglu<1, TU>{u, F, sc.a, sc.w})
                                : launch(EpiSwiglu<0, TU>{u, F, sc.a, sc.w});
            }
            return with_act(typename TSet::S{});
    }
}

hipError_t launch_gemm_swiglu(const bf16 *a, const bf16 *w, int64_t M, int F, int K, int act, bf16 *u,
                              hipStream_t s) {
    TraceScope trace_(s, "gemm_swiglu");
    if (trace_.on()) trace_.args("M=%lld F=%d K=%d", (long long)M, F, K);
    return swiglu_any(a, w, M, F, K, act, u, NoScales{}, s);
}

hipError_t launch_gemm_swiglu_f32(const float *a, const float *w, int64_t M, int F, int K, int act, float *u,
                                  hipStream_t s) {
    TraceScope trace_(s, "gemm_swiglu_f32");
    if (trace_.on()) trace_.args("M=%lld F=%d K=%d", (long long)M, F, K);
    return swiglu_any(a, w, M, F, K, act, u, F32Ops{}, s);
}

hipError_t launch_gemm_swiglu_q8(const int8_t *a, const float *a_scale, const int8_t *w, const float *w_scale,
                                 int64_t M, int F, int K, int act, bf16 *u, hipStream_t s) {
    TraceScope trace_(s, "gemm_swiglu_w8a8");
    if (trace_.on()) trace_.args("M=%lld F=%d K=%d", (long long)M, F, K);
    return swiglu_any(a, w, M, F, K, act, u, Scales{a_scale, w_scale}, s);
}

// Rows of a bf16 or int8 (fmt 0 / 1) QKV projection that take the split form:
// those the tile choice puts in 256 x 256 tiles (all rows, or the full row tiles when a short
// tail runs in 128-row tiles).  0 (the fused epilogue throughout) when it picks
// 128-row tiles, for 64-wide heads (measured slower split: their norm pass
// moves the same bytes for half the GEMM work), and unless every 16-row block
// of the split rows lies in one sequence and below the row count (the split
// epilogue's condition): a row count that is a multiple of 16 and one
// sequence or a sequence length that is a multiple of 16.
static int64_t qkv_split_rows(int64_t M, int N, int batch, int seq, int head_dim, int fmt) {
    if (head_dim != 128 || choose_tile(M, N, 1u << kTileS | 1u << kTileHalf, fmt) == kTileHalf) return 0;
    const int64_t m4 = split_tail_rows(M, N) ? M / 256 * 256 : M;
    if (m4 % 16 || (batch > 1 && seq % 16)) return 0;
    return m4;
}

static hipError_t launch_qk_norm_rope(const QkvEpiArgs &e, int64_t m_end, hipStream_t s) {
    if (m_end <= 0) return hipSuccess;
    if (m_end >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const int tpb = 256 / (e.head_dim / 8);
    const dim3 grid((unsigned)((m_end + tpb - 1) / tpb), (unsigned)((e.heads + e.kv_heads + kQkNormGroup - 1) / kQkNormGroup));
#define DIT_QNR(HD_, RMS_, RF_, RH_) \
    hipLaunchKernelGGL((qk_norm_rope_kernel<HD_, RMS_, RF_, RH_>), grid, dim3(256), 0, s, e, (int)m_end)
#define DIT_QNR2(HD_, RMS_, RF_) \
    do { if (e.rope_half) DIT_QNR(HD_, RMS_, RF_, true); else DIT_QNR(HD_, RMS_, RF_, false); } while (0)
#define DIT_QNR3(HD_) \
    do { \
        if (e.rms) { if (e.rope_first) DIT_QNR2(HD_, true, true); else DIT_QNR2(HD_, true, false); } \
        else { if (e.rope_first) DIT_QNR2(HD_, false, true); else DIT_QNR2(HD_, false, false); } \
    } while (0)
    DIT_QNR3(128);
#undef DIT_QNR3
#undef DIT_QNR2
#undef DIT_QNR
    return hipGetLastError();
}

template <class SC>
static hipError_t qkv_any(const void *h, const void *w, int64_t M, int N, int K, const QkvEpiArgs &e, SC sc,
                          hipStream_t s) {
    using T = typename TileSet<SC::kFmt>::S;
    using TH = typename TileSet<SC::kFmt>::Half;
    using TQ = typename std::conditional<SC::kFmt == 2, float, bf16>::type;
    if constexpr (SC::kFmt != 2) {
        // bf16 and int8 rows in 256 x 256 tiles: the split form (persistent
        // 4-wave GEMM with a plain epilogue, then the in-place qk-norm + RoPE
        // pass); a 128-row tail keeps the fused 8-wave epilogue, whose rows the
        // pass skips
        using T4 = std::conditional_t<SC::kFmt == 0, Tile4w, Tile4wQ>;
        const int64_t m4 = qkv_split_rows(M, N, e.batch, e.seq, e.head_dim, SC::kFmt);
        if (m4 > 0) {
            hipError_t err = run4<T4>(h, w, m4, N, K, RowsIdentity<256>{}, EpiQkvRaw<128>{e, sc.a, sc.w}, s);
            if (err != hipSuccess) return err;
            if (m4 < M) {
#define DIT_QKV_TAIL(HD_, RMS_, RF_, RH_) \
    run<TH>(h, w, M, N, K, RowsIdentity<TH::BN>{}, EpiQkv<HD_, RMS_, RF_, RH_, TQ>{e}, s, sc.a, sc.w, m4)
#define DIT_QKV_TAIL2(HD_, RMS_, RF_) (e.rope_half ? DIT_QKV_TAIL(HD_, RMS_, RF_, true) : DIT_QKV_TAIL(HD_, RMS_, RF_, false))
                err = e.rms ? (e.rope_first ? DIT_QKV_TAIL2(128, true, true) : DIT_QKV_TAIL2(128, true, false))
                            : (e.rope_first ? DIT_QKV_TAIL2(128, false, true) : DIT_QKV_TAIL2(128, false, false));
#undef DIT_QKV_TAIL2
#undef DIT_QKV_TAIL
                if (err != hipSuccess) return err;
            }
            return launch_qk_norm_rope(e, m4, s);
        }
    }
#define DIT_QKV_RH(HD_, RMS_, RF_, RH_) \
    run_tail_split<T, TH>(h, w, M, N, K, RowsIdentity<T::BN>{}, EpiQkv<HD_, RMS_, RF_, RH_, TQ>{e}, s, sc.a, sc.w)
#define DIT_QKV(HD_, RMS_, RF_) \
    (e.rope_half ? DIT_QKV_RH(HD_, RMS_, RF_, true) : DIT_QKV_RH(HD_, RMS_, RF_, false))
    if (e.head_dim == 128) {
        if (e.rms) return e.rope_first ? DIT_QKV(128, true, true) : DIT_QKV(128, true, false);
        return e.rope_first ? DIT_QKV(128, false, true) : DIT_QKV(128, false, false);
    }
    if (e.rms) return e.rope_first ? DIT_QKV(64, true, true) : DIT_QKV(64, true, false);
    return e.rope_first ? DIT_QKV(64, false, true) : DIT_QKV(64, false, false);
#undef DIT_QKV
#undef DIT_QKV_RH
}

hipError_t launch_gemm_qkv(const bf16 *h, const bf16 *w, int64_t M, int N, int K, const QkvEpiArgs &e,
                           hipStream_t s) {
    TraceScope trace_(s, "gemm_qkv");
    if (trace_.on()) trace_.args("M=%lld N=%d K=%d", (long long)M, N, K);
    return qkv_any(h, w, M, N, K, e, NoScales{}, s);
}

hipError_t launch_gemm_qkv_f32(const float *h, const float *w, int64_t M, int N, int K, const QkvEpiArgs &e,
                               hipStream_t s) {
    TraceScope trace_(s, "gemm_qkv_f32");
    if (trace_.on()) trace_.args("M=%lld N=%d K=%d", (long long)M, N, K);
    return qkv_any(h, w, M, N, K, e, F32Ops{}, s);
}

hipError_t launch_gemm_qkv_q8(const int8_t *h, const float *h_scale, const int8_t *w, const float *w_scale,
                              int64_t M, int N, int K, const QkvEpiArgs &e, hipStream_t s) {
    TraceScope trace_(s, "gemm_qkv_w8a8");
    if (trace_.on()) trace_.args("M=%lld N=%d K=%d", (long long)M, N, K);
    return qkv_any(h, w, M, N, K, e, Scales{h_scale, w_scale}, s);
}

}  // namespace dit
