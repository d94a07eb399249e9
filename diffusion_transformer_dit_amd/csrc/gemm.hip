// bf16 MFMA GEMM for gfx950 with the block's fused epilogues.
//
// C[m, n] = sum_k A[m, k] * W[n, k]: A is [M, K] row-major (activations), W is
// [N, K] row-major (weights as [out, in]), both K-contiguous, so both operand
// tiles are copied to LDS row by row and read back as MFMA fragments without a
// transpose.  One workgroup computes a BM x BN tile with WM x WN waves; each
// wave owns a (BM/WM) x (BN/WN) sub-tile built from 32x32 MFMA blocks
// (v_mfma_f32_32x32x16_bf16, fp32 accumulators).  K advances in steps of 64
// through two LDS stages: while one stage feeds the MFMAs, the next tile is
// already in flight from global memory into registers.
//
// Epilogues (run on the fp32 accumulators, no extra pass over memory):
//   * residual : out = resid + gate[n] * acc + bias[n]   (gated residual, ERNIE
//                page §VII Decision 1; out-projection / down-projection)
//   * swiglu   : u = SiLU(acc_gate) * acc_up             (the tile's W rows
//                interleave gate rows and the matching up rows)
//   * qkv      : per-(token, head) LayerNorm over head_dim with gamma/beta,
//                RoPE rotation from cos/sin tables, scatter to head-major
//                q/k and transposed v (zml-flow-rs page §VI, "QKV + norm + RoPE")
#include "common.h"

namespace dit {

constexpr int kBK = 64;   // K step per LDS stage (one 128-byte row segment)

template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int kThreads = WM * WN * kWave;
    static constexpr int kWaveM = BM / WM, kWaveN = BN / WN;
    static constexpr int TM = kWaveM / 32, TN = kWaveN / 32;
    static constexpr int kAChunks = BM * 8 / kThreads;   // 16-byte chunks per thread per stage
    static constexpr int kBChunks = BN * 8 / kThreads;
    static constexpr int kStageBytes = (BM + BN) * 128;
    static_assert(BM * 8 % kThreads == 0 && BN * 8 % kThreads == 0, "tile/threads");
    static_assert(kWaveM % 32 == 0 && kWaveN % 32 == 0, "wave tile");
};

// Row-major LDS tile of 64 bf16 (128 B) per row, eight 16-byte chunks per row;
// chunk c of row r lives at chunk slot c ^ (r & 7) so that the 8 lanes of a
// ds_read_b128 phase (rows r..r+7, same logical chunk) hit 8 distinct slots.
__device__ __forceinline__ uint32_t lds_off(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

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

struct RowsIdentity {
    int bn;
    __device__ __forceinline__ int operator()(int tile_n, int t) const { return tile_n * bn + t; }
};

// SwiGLU tile rows: each wave's kWaveN columns are kWaveN/2 gate rows followed by
// the up rows (offset F) of the same features.
struct RowsSwiglu {
    int bn, wave_n, F;
    __device__ __forceinline__ int operator()(int tile_n, int t) const {
        const int half = wave_n >> 1;
        const int w = t / wave_n, within = t - w * wave_n;
        const int feat = tile_n * (bn >> 1) + w * half + (within % half);
        return within >= half ? feat + F : feat;
    }
};

template <class T, class RowMap, class Epi>
__global__ __launch_bounds__(T::kThreads, 1)
void gemm_kernel(const bf16 *__restrict__ A, const bf16 *__restrict__ W, int M, int K,
                 int tiles_m, int tiles_n, RowMap rowmap, Epi epi) {
    constexpr int kLds = Epi::template lds_bytes<T>() > 2 * T::kStageBytes ? Epi::template lds_bytes<T>()
                                                                              : 2 * T::kStageBytes;
    __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];

    int tm, tn;
    tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * T::BM;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / T::WN, wn = wave % T::WN;
    const int lrow = lane & 31, lhalf = lane >> 5;

    // global source offsets (elements) and LDS destinations of this thread's chunks
    uint32_t a_src[T::kAChunks], a_dst[T::kAChunks];
    uint32_t b_src[T::kBChunks], b_dst[T::kBChunks];
#pragma unroll
    for (int q = 0; q < T::kAChunks; ++q) {
        const int id = q * T::kThreads + tid, r = id >> 3, c = id & 7;
        const int grow = min(m0 + r, M - 1);              // ragged M: clamp reads, mask stores
        a_src[q] = (uint32_t)grow * (uint32_t)K + c * 8;
        a_dst[q] = lds_off(r, c);
    }
#pragma unroll
    for (int q = 0; q < T::kBChunks; ++q) {
        const int id = q * T::kThreads + tid, r = id >> 3, c = id & 7;
        b_src[q] = (uint32_t)rowmap(tn, r) * (uint32_t)K + c * 8;
        b_dst[q] = T::BM * 128 + lds_off(r, c);
    }

    uint4 ra[T::kAChunks], rb[T::kBChunks];
#define DIT_GEMM_GLOAD(k0)                                                                      \
    do {                                                                                        \
        _Pragma("unroll") for (int q = 0; q < T::kAChunks; ++q) ra[q] = *(const uint4 *)(A + a_src[q] + (k0)); \
        _Pragma("unroll") for (int q = 0; q < T::kBChunks; ++q) rb[q] = *(const uint4 *)(W + b_src[q] + (k0)); \
    } while (0)
#define DIT_GEMM_LSTORE(stage)                                                                  \
    do {                                                                                        \
        uint8_t *base_ = smem + (stage) * T::kStageBytes;                                       \
        _Pragma("unroll") for (int q = 0; q < T::kAChunks; ++q) *(uint4 *)(base_ + a_dst[q]) = ra[q]; \
        _Pragma("unroll") for (int q = 0; q < T::kBChunks; ++q) *(uint4 *)(base_ + b_dst[q]) = rb[q]; \
    } while (0)

    floatx16 acc[T::TM][T::TN];
#pragma unroll
    for (int i = 0; i < T::TM; ++i)
#pragma unroll
        for (int j = 0; j < T::TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int KT = K / kBK;
    DIT_GEMM_GLOAD(0);
    DIT_GEMM_LSTORE(0);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        // the last iteration re-reads the final K tile into the idle stage: no branch
        // around the prefetch, so the staging registers stay registers
        DIT_GEMM_GLOAD(min(kt + 1, KT - 1) * kBK);
        const uint8_t *sa = smem + cur * T::kStageBytes;
        const uint8_t *sb = sa + T::BM * 128;
#pragma unroll
        for (int kk = 0; kk < kBK / 16; ++kk) {
            const int c = kk * 2 + lhalf;
            bf16x8 af[T::TM], bfr[T::TN];
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
                af[i] = *(const bf16x8 *)(sa + lds_off(wm * T::kWaveM + i * 32 + lrow, c));
#pragma unroll
            for (int j = 0; j < T::TN; ++j)
                bfr[j] = *(const bf16x8 *)(sb + lds_off(wn * T::kWaveN + j * 32 + lrow, c));
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        DIT_GEMM_LSTORE(cur ^ 1);   // stage cur^1 was released by the barrier of iteration kt-1
        __syncthreads();
    }
#undef DIT_GEMM_GLOAD
#undef DIT_GEMM_LSTORE

    epi.template apply<T>(acc, m0 + wm * T::kWaveM, tn, wn, lane, M, smem);
}

// Accumulator element (i, j, e) of a wave sits at wave-tile row
// i*32 + (e/4)*8 + (lane/32)*4 + e%4 and wave-tile column j*32 + lane%32.
__device__ __forceinline__ int acc_row(int i, int e, int lhalf) { return i * 32 + ((e >> 2) << 3) + (lhalf << 2) + (e & 3); }

// ---------------------------------------------------------------------------
// epilogue: out = resid + gate * acc + bias
// ---------------------------------------------------------------------------
template <typename TR, typename TO>
struct EpiResidual {
    const TR *resid;
    const float *gate, *bias;
    TO *out;
    int N;
    template <class T> static constexpr int lds_bytes() { return 0; }
    template <class T>
    __device__ __forceinline__ void apply(floatx16 (&acc)[T::TM][T::TN], int row0, int tn, int wn, int lane, int M,
                                          uint8_t *) const {
        const int lrow = lane & 31, lhalf = lane >> 5;
        const int col0 = tn * T::BN + wn * T::kWaveN;
#pragma unroll
        for (int j = 0; j < T::TN; ++j) {
            const int col = col0 + j * 32 + lrow;
            const float g = gate ? gate[col] : 1.0f;
            const float bb = bias ? bias[col] : 0.0f;
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = row0 + acc_row(i, e, lhalf);
                    if (row < M) {
                        const size_t o = (size_t)row * N + col;
                        float v = acc[i][j][e] * g + bb;
                        if (resid) v += to_f32<TR>(resid[o]);
                        out[o] = from_f32<TO>(v);
                    }
                }
        }
    }
};

// ---------------------------------------------------------------------------
// epilogue: u = SiLU(gate) * up
// ---------------------------------------------------------------------------
struct EpiSwiglu {
    bf16 *u;
    int F;
    template <class T> static constexpr int lds_bytes() { return 0; }
    template <class T>
    __device__ __forceinline__ void apply(floatx16 (&acc)[T::TM][T::TN], int row0, int tn, int wn, int lane, int M,
                                          uint8_t *) const {
        const int lrow = lane & 31, lhalf = lane >> 5;
        constexpr int HJ = T::TN / 2;
        const int f0 = tn * (T::BN / 2) + wn * (T::kWaveN / 2);
#pragma unroll
        for (int j = 0; j < HJ; ++j) {
            const int f = f0 + j * 32 + lrow;
#pragma unroll
            for (int i = 0; i < T::TM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = row0 + acc_row(i, e, lhalf);
                    if (row < M) u[(size_t)row * F + f] = f2bf(silu_f(acc[i][j][e]) * acc[i][j + HJ][e]);
                }
        }
    }
};

// ---------------------------------------------------------------------------
// epilogue: qk-LayerNorm + RoPE, scatter to q [B,H,S,hd], k [B,Hk,S,hd],
// vt [B,Hk,hd,Spad].  The accumulators go through LDS (free once the K loop
// has drained) in two passes of 64 rows per wave, so that afterwards one lane
// holds one token row of a head: the LayerNorm statistics and the RoPE pairs
// are then in-lane, q/k rows leave as 16-byte stores, and for v one lane
// holds one head-dim column and writes it contiguously along the tokens.
// ---------------------------------------------------------------------------
constexpr int kQkvStride = 132;   // floats per staged row: 128 + 4 (row-per-lane reads hit distinct banks)

template <int HD>
struct EpiQkv {
    QkvEpiArgs e;
    template <class T> static constexpr int lds_bytes() { return T::WM * T::WN * 64 * kQkvStride * 4; }

    template <class T>
    __device__ __forceinline__ void apply(floatx16 (&acc)[T::TM][T::TN], int row0, int tn, int wn, int lane, int M,
                                          uint8_t *smem) const {
        static_assert(T::kWaveN == 128 && T::kWaveM == 128, "staging assumes 128x128 wave tiles");
        constexpr int HPW = 128 / HD;                  // heads per wave
        const int lrow = lane & 31, lhalf = lane >> 5;
        const int wave = threadIdx.x >> 6;
        float *red = (float *)smem + wave * 64 * kQkvStride;
        const int col0 = tn * T::BN + wn * 128;
        const int qcols = e.heads * HD, kcols = e.kv_heads * HD;
        const int S = e.seq;
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            __syncthreads();   // previous users of the LDS (K loop or pass 0) are done
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
#pragma unroll
                for (int j = 0; j < T::TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        red[(ii * 32 + ((r >> 2) << 3) + (lhalf << 2) + (r & 3)) * kQkvStride + j * 32 + lrow] =
                            acc[pass * 2 + ii][j][r];
            __syncthreads();
            const int rbase = row0 + pass * 64;        // token of staged row 0
#pragma unroll
            for (int hw = 0; hw < HPW; ++hw) {
                const int hc0 = col0 + hw * HD;
                const int sect = hc0 < qcols ? 0 : (hc0 < qcols + kcols ? 1 : 2);
                const int head = sect == 0 ? hc0 / HD : (sect == 1 ? (hc0 - qcols) / HD : (hc0 - qcols - kcols) / HD);
                if (sect < 2) {
                    // one token row per lane
                    const int row = rbase + lane;
                    float y[HD];
                    const float *src = red + lane * kQkvStride + hw * HD;
#pragma unroll
                    for (int c = 0; c < HD; c += 4) {
                        const floatx4 v = *(const floatx4 *)(src + c);
                        y[c] = v[0]; y[c + 1] = v[1]; y[c + 2] = v[2]; y[c + 3] = v[3];
                    }
                    if (e.qk_norm) {
                        const float *g = sect == 0 ? e.q_g : e.k_g;
                        const float *bb = sect == 0 ? e.q_b : e.k_b;
                        float sum = 0.f;
#pragma unroll
                        for (int c = 0; c < HD; ++c) sum += y[c];
                        const float mean = sum * (1.0f / HD);
                        float ss = 0.f;
#pragma unroll
                        for (int c = 0; c < HD; ++c) { y[c] -= mean; ss += y[c] * y[c]; }
                        const float rstd = rsqrtf(ss * (1.0f / HD) + e.eps);
#pragma unroll
                        for (int c = 0; c < HD; ++c) y[c] = y[c] * rstd * g[c] + bb[c];
                    }
                    const int trow = min(row, M - 1);
                    const int bidx = trow / S, sp = trow - bidx * S;
                    const float *ct = e.cos_t + (size_t)sp * (HD / 2);
                    const float *st = e.sin_t + (size_t)sp * (HD / 2);
                    // rotate in place, 4 pair slots (one float4 of each table) at a time
#pragma unroll
                    for (int m4 = 0; m4 < HD / 2; m4 += 4) {
                        const floatx4 c4 = *(const floatx4 *)(ct + m4), s4 = *(const floatx4 *)(st + m4);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const int m = m4 + u;
                            const int ia = e.rope_half ? m : 2 * m;
                            const int ib = e.rope_half ? m + HD / 2 : 2 * m + 1;
                            const float a = y[ia], bq = y[ib];
                            y[ia] = a * c4[u] - bq * s4[u];
                            y[ib] = a * s4[u] + bq * c4[u];
                        }
                    }
                    if (row < M) {
                        bf16 *dst = (sect == 0 ? e.q : e.k) +
                                    (((size_t)bidx * (sect == 0 ? e.heads : e.kv_heads) + head) * S + sp) * HD;
#pragma unroll
                        for (int c = 0; c < HD; c += 8) {
                            bf16x8 v;
#pragma unroll
                            for (int u = 0; u < 8; ++u) v[u] = f2bf(y[c + u]);
                            *(bf16x8 *)(dst + c) = v;
                        }
                    }
                } else {
                    // v: one head-dim column per lane, 64 tokens along the row of vt
                    const int b0 = min(rbase, M - 1) / S;
                    const int s0 = rbase - b0 * S;
                    const bool fast = (rbase + 63 < M) && (s0 + 63 < S) && ((s0 & 7) == 0);
#pragma unroll
                    for (int dc = 0; dc < HD; dc += 64) {
                        const int d = dc + lane;
                        const float *src = red + hw * HD + d;
                        if (fast) {
                            bf16 *dst = e.vt + (((size_t)b0 * e.kv_heads + head) * HD + d) * e.seq_pad + s0;
#pragma unroll
                            for (int r8 = 0; r8 < 64; r8 += 8) {
                                bf16x8 v;
#pragma unroll
                                for (int u = 0; u < 8; ++u) v[u] = f2bf(src[(r8 + u) * kQkvStride]);
                                *(bf16x8 *)(dst + r8) = v;
                            }
                        } else {
                            for (int r = 0; r < 64; ++r) {
                                const int row = rbase + r;
                                if (row >= M) break;
                                const int bidx = row / S, sp = row - bidx * S;
                                e.vt[(((size_t)bidx * e.kv_heads + head) * HD + d) * e.seq_pad + sp] =
                                    f2bf(src[r * kQkvStride]);
                            }
                        }
                    }
                }
            }
        }
    }
};

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
using TileBig = Tile<256, 256, 2, 2>;    // 128x128 per wave
using TileNarrow = Tile<256, 128, 2, 2>; // 128x64 per wave (N = 128 outputs)

template <class T, class RowMap, class Epi>
static hipError_t run(const bf16 *a, const bf16 *w, int64_t M, int N_tile_cols, int K, RowMap rm, Epi epi,
                      hipStream_t s) {
    const int tiles_m = (int)((M + T::BM - 1) / T::BM);
    const int tiles_n = N_tile_cols / T::BN;
    const int grid = tiles_m * tiles_n;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel<T, RowMap, Epi>), dim3(grid), dim3(T::kThreads), 0, s, a, w, (int)M, K,
                       tiles_m, tiles_n, rm, epi);
    return hipGetLastError();
}

template <typename TR, typename TO>
static hipError_t residual_typed(const bf16 *a, const bf16 *w, int64_t M, int N, int K, const void *resid,
                                 const float *gate, const float *bias, void *out, hipStream_t s) {
    EpiResidual<TR, TO> epi{(const TR *)resid, gate, bias, (TO *)out, N};
    if (N % 256 == 0) return run<TileBig>(a, w, M, N, K, RowsIdentity{256}, epi, s);
    return run<TileNarrow>(a, w, M, N, K, RowsIdentity{128}, epi, s);
}

hipError_t launch_gemm_residual(const bf16 *a, const bf16 *w, int64_t M, int N, int K, const void *resid,
                                int resid_f32, const float *gate, const float *bias, void *out, int out_f32,
                                hipStream_t s) {
    if (resid_f32) {
        return out_f32 ? residual_typed<float, float>(a, w, M, N, K, resid, gate, bias, out, s)
                       : residual_typed<float, bf16>(a, w, M, N, K, resid, gate, bias, out, s);
    }
    return out_f32 ? residual_typed<bf16, float>(a, w, M, N, K, resid, gate, bias, out, s)
                   : residual_typed<bf16, bf16>(a, w, M, N, K, resid, gate, bias, out, s);
}

hipError_t launch_gemm_swiglu(const bf16 *a, const bf16 *w, int64_t M, int F, int K, bf16 *u, hipStream_t s) {
    using T = TileBig;
    return run<T>(a, w, M, 2 * F, K, RowsSwiglu{T::BN, T::kWaveN, F}, EpiSwiglu{u, F}, s);
}

hipError_t launch_gemm_qkv(const bf16 *h, const bf16 *w, int64_t M, int N, int K, const QkvEpiArgs &e,
                           hipStream_t s) {
    using T = TileBig;
    if (e.head_dim == 128) return run<T>(h, w, M, N, K, RowsIdentity{T::BN}, EpiQkv<128>{e}, s);
    return run<T>(h, w, M, N, K, RowsIdentity{T::BN}, EpiQkv<64>{e}, s);
}

}  // namespace dit
