// The W8A8 H256 format of the zml-flow-rs page (§VII "Precision Formats
// Derived, Not Picked"): int8 codes per row with a 256-point Hadamard rotation
// on both operands of a projection, legal because (x H)(W H)^T = x W^T for an
// orthogonal H.
//
//   quantize_h256    q, s = I8(rows of x blockdiag(H256))
//                    (the weights once, when they are prepared; the attention
//                    output and the GLU output before their projections)
//   ln_modulate_q8   q, s = I8(rows of (norm(x) mul + add) blockdiag(H256))
//                    (the block's two pre-norms feed their GEMMs in int8)
//
// I8 of a row v: amax = max |v|, s = amax / 127, q = v * (127 / amax) rounded
// half to even, in [-127, 127] (a zero row: codes 0, s = 0).  H256 is the
// Sylvester-Hadamard matrix scaled by 1/16, entry (a, b) = (-1)^popcount(a & b)
// / 16, applied to every run of 256 consecutive elements of a row.
//
// Register layout: a row is walked in rounds of 1024 elements; in round r lane
// l holds the 16 consecutive elements [1024 r + 16 l, +16).  Rotation block
// 4 r + l / 16 then lies in one 16-lane DPP row with element index
// e = 16 (l % 16) + j: the four low bits of e are butterflies inside a lane,
// the four high bits butterflies between lanes l and l ^ 1, 2, 4, 8, which DPP
// moves reach without LDS.  A row length that is not a multiple of 1024 leaves
// whole 16-lane groups idle (holding zeros) in its last round.
#include "common.h"
#include "trace.h"

namespace dit {

// v of lane (lane ^ M) inside each row of 16 lanes (every source lane exists,
// so no lane keeps an old value and the move can fold into its user)
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    const int i = __float_as_int(v);
    int r;
    if constexpr (M == 1) {
        r = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, true);     // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        r = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, true);     // quad_perm [2,3,0,1]
    } else if constexpr (M == 4) {
        // row_half_mirror (lane 7 - i of 8, i.e. i ^ 7), then quad_perm [3,2,1,0] (i ^ 3)
        const int t = __builtin_amdgcn_mov_dpp(i, 0x141, 0xF, 0xF, true);
        r = __builtin_amdgcn_mov_dpp(t, 0x1B, 0xF, 0xF, true);
    } else {
        static_assert(M == 8, "lane_xor: 1, 2, 4 or 8");
        r = __builtin_amdgcn_mov_dpp(i, 0x128, 0xF, 0xF, true);    // row_ror 8: i ^ 8 of 16
    }
    return __int_as_float(r);
}

// v <- v H256 for the block held by the 16 lanes of a DPP row.  Must run with
// every lane of the wave active (the DPP moves read the partner lanes).
__device__ __forceinline__ void hadamard256(float (&v)[16], int lane) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int j = 0; j < 16; ++j)
            if (!(j & h)) {
                const float a = v[j], b = v[j | h];
                v[j] = a + b;
                v[j | h] = a - b;
            }
    // lanes l and l ^ m: the pair (a, b) becomes (a + b, a - b).  Each lane computes
    // own + sg * partner (sg = -1 on the lane with bit m set), one fused
    // v_fmac with the partner's value read through DPP; the upper lane so holds
    // b - a = -(a - b).  Partners carry the same sign from the earlier stages
    // (their lane numbers differ only in bit m), so after the four stages lane l
    // holds (-1)^popcount(l & 15) times its result, undone with the 1/16 scale.
#define DIT_HSTAGE(M)                                                                                 \
    {                                                                                                 \
        const float sg = (lane & (M)) ? -1.0f : 1.0f;                                                 \
        _Pragma("unroll") for (int j = 0; j < 16; ++j) v[j] = fmaf(lane_xor<M>(v[j]), sg, v[j]);     \
    }
    DIT_HSTAGE(1)
    DIT_HSTAGE(2)
    DIT_HSTAGE(4)
    DIT_HSTAGE(8)
#undef DIT_HSTAGE
    const float fix = (__popc(lane & 15) & 1) ? -0.0625f : 0.0625f;
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] *= fix;
}

// 16 codes rne(v * inv) clamped to +-127, packed little-endian into 16 bytes
__device__ __forceinline__ intx4 codes16(const float (&v)[16], float inv) {
    intx4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t p = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float c = fminf(fmaxf(rintf(v[w * 4 + b] * inv), -127.0f), 127.0f);
            p |= ((uint32_t)(int)c & 255u) << (8 * b);
        }
        o[w] = (int)p;
    }
    return o;
}

template <typename TX>
__device__ __forceinline__ void load16(const TX *p, float (&v)[16]) {
    if constexpr (sizeof(TX) == 4) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const floatx4 t = *(const floatx4 *)(p + c * 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) v[c * 4 + u] = t[u];
        }
    } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const bf16x8 t = *(const bf16x8 *)(p + c * 8);
#pragma unroll
            for (int u = 0; u < 8; ++u) v[c * 8 + u] = (float)t[u];
        }
    }
}

__device__ __forceinline__ void load16f(const float *p, float (&v)[16]) { load16<float>(p, v); }

// ---------------------------------------------------------------------------
// quantize_h256: NWR waves per row (rounds part, part + NWR, ...), RW rounds per
// wave; the row max of NWR > 1 waves meets in LDS.
// ---------------------------------------------------------------------------
template <typename TX, int RW, int NWR>
__global__ __launch_bounds__(256)
void quantize_h256_kernel(const TX *__restrict__ x, int64_t rows, int cols, int8_t *__restrict__ q,
                          float *__restrict__ scale) {
    constexpr int RPB = 4 / NWR;   // rows per workgroup of 4 waves
    __shared__ float wmax[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int part = wave % NWR;
    const int64_t row = (int64_t)blockIdx.x * RPB + wave / NWR;
    const bool live = row < rows;   // uniform over a row's waves (so over the workgroup when NWR = 4)
    const int64_t rr = live ? row : rows - 1;
    const TX *xr = x + rr * cols;
    float v[RW][16];
#pragma unroll
    for (int k = 0; k < RW; ++k) {
        const int start = (part + k * NWR) * 1024 + lane * 16;
        load16<TX>(xr + (start < cols ? start : 0), v[k]);
        if (start >= cols) {
#pragma unroll
            for (int j = 0; j < 16; ++j) v[k][j] = 0.0f;
        }
    }
    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < RW; ++k) {
        hadamard256(v[k], lane);
#pragma unroll
        for (int j = 0; j < 16; ++j) am = fmaxf(am, fabsf(v[k][j]));
    }
    am = group_max<64>(am);
    if constexpr (NWR > 1) {
        if (lane == 0) wmax[wave] = am;
        __syncthreads();
        const int g0 = (wave / NWR) * NWR;
        am = wmax[g0];
#pragma unroll
        for (int w = 1; w < NWR; ++w) am = fmaxf(am, wmax[g0 + w]);
    }
    if (!live) return;
    const float inv = am > 0.0f ? 127.0f / am : 0.0f;
    int8_t *qr = q + rr * cols;
#pragma unroll
    for (int k = 0; k < RW; ++k) {
        const int start = (part + k * NWR) * 1024 + lane * 16;
        if (start < cols) *(intx4 *)(qr + start) = codes16(v[k], inv);
    }
    if (part == 0 && lane == 0) scale[row] = am / 127.0f;
}

template <typename TX>
static hipError_t quantize_typed(const TX *x, int64_t rows, int cols, int8_t *q, float *scale, hipStream_t s) {
    const int R = (cols + 1023) / 1024;
#define DIT_QH(RW_, NWR_)                                                                                    \
    hipLaunchKernelGGL((quantize_h256_kernel<TX, RW_, NWR_>), dim3((unsigned)((rows + 4 / NWR_ - 1) / (4 / NWR_))), \
                       dim3(256), 0, s, x, rows, cols, q, scale)
    if (R % 4 == 0) {
        switch (R / 4) {
            case 1: DIT_QH(1, 4); break;
            case 2: DIT_QH(2, 4); break;
            case 3: DIT_QH(3, 4); break;
            case 4: DIT_QH(4, 4); break;
            case 5: DIT_QH(5, 4); break;
            case 6: DIT_QH(6, 4); break;
            case 7: DIT_QH(7, 4); break;
            case 8: DIT_QH(8, 4); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (R) {
            case 1: DIT_QH(1, 1); break;
            case 2: DIT_QH(2, 1); break;
            case 3: DIT_QH(3, 1); break;
            case 5: DIT_QH(5, 1); break;
            case 6: DIT_QH(6, 1); break;
            case 7: DIT_QH(7, 1); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef DIT_QH
    return hipGetLastError();
}

bool quantize_h256_supported(int cols) {
    if (cols <= 0 || cols % 256) return false;
    const int R = (cols + 1023) / 1024;
    return R % 4 == 0 ? R / 4 <= 8 : R <= 7;
}

hipError_t launch_quantize_h256(const void *x, int x_f32, int64_t rows, int cols, int8_t *q, float *scale,
                                hipStream_t s) {
    TraceScope trace_(s, "quantize_h256");
    if (trace_.on()) trace_.args("rows=%lld cols=%d", (long long)rows, cols);
    if (rows <= 0) return hipSuccess;
    return x_f32 ? quantize_typed((const float *)x, rows, cols, q, scale, s)
                 : quantize_typed((const bf16 *)x, rows, cols, q, scale, s);
}

// ---------------------------------------------------------------------------
// ln_modulate_q8: the row norm and modulation of ln_modulate, then the rotation
// and the codes, one wave per row (R rounds, dim <= 8192), h never leaves
// registers.  mode 0: mul = 1 + scale; mode 1: mul = scale (NULL = 1); add =
// shift (NULL = 0).
// ---------------------------------------------------------------------------
template <typename TX, int R, bool RMS>
__global__ __launch_bounds__(256)
void ln_modulate_q8_kernel(const TX *__restrict__ x, int64_t rows, int dim, const float *__restrict__ shift,
                           const float *__restrict__ scale, int mode, float eps, int8_t *__restrict__ q,
                           float *__restrict__ qscale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;   // whole wave: no barrier below
    const TX *xr = x + row * dim;
    float v[R][16];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int start = k * 1024 + lane * 16;
        load16<TX>(xr + (start < dim ? start : 0), v[k]);
        if (start >= dim) {
#pragma unroll
            for (int j = 0; j < 16; ++j) v[k][j] = 0.0f;
        }
    }
    float mean = 0.0f;
    if (!RMS) {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < R; ++k)
#pragma unroll
            for (int j = 0; j < 16; ++j) s += v[k][j];
        mean = group_sum<64>(s) * (1.0f / dim);
    }
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const bool act = k * 1024 + lane * 16 < dim;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float d = act ? v[k][j] - mean : 0.0f;
            v[k][j] = d;
            ss += d * d;
        }
    }
    const float rstd = rsqrtf(group_sum<64>(ss) * (1.0f / dim) + eps);
    const float one = mode == 0 ? 1.0f : 0.0f;
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int start = k * 1024 + lane * 16;
        const int st = start < dim ? start : 0;
        float mul[16], add[16];
        if (scale) {
            load16f(scale + st, mul);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) mul[j] = 1.0f - one;   // mode 1 with no scale: mul = 1
        }
        if (shift) {
            load16f(shift + st, add);
        } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) add[j] = 0.0f;
        }
        const bool act = start < dim;
#pragma unroll
        for (int j = 0; j < 16; ++j) v[k][j] = act ? v[k][j] * rstd * (mul[j] + one) + add[j] : 0.0f;
    }
    float am = 0.0f;
#pragma unroll
    for (int k = 0; k < R; ++k) {
        hadamard256(v[k], lane);
#pragma unroll
        for (int j = 0; j < 16; ++j) am = fmaxf(am, fabsf(v[k][j]));
    }
    am = group_max<64>(am);
    const float inv = am > 0.0f ? 127.0f / am : 0.0f;
    int8_t *qr = q + row * dim;
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const int start = k * 1024 + lane * 16;
        if (start < dim) *(intx4 *)(qr + start) = codes16(v[k], inv);
    }
    if (lane == 0) qscale[row] = am / 127.0f;
}

template <typename TX, bool RMS>
static hipError_t ln_q8_typed(const TX *x, int64_t rows, int dim, const float *shift, const float *scale, int mode,
                              float eps, int8_t *q, float *qs, hipStream_t s) {
    const dim3 grid((unsigned)((rows + 3) / 4));
#define DIT_LQ(R_) \
    hipLaunchKernelGGL((ln_modulate_q8_kernel<TX, R_, RMS>), grid, dim3(256), 0, s, x, rows, dim, shift, scale, mode, eps, q, qs)
    switch ((dim + 1023) / 1024) {
        case 1: DIT_LQ(1); break;
        case 2: DIT_LQ(2); break;
        case 3: DIT_LQ(3); break;
        case 4: DIT_LQ(4); break;
        case 5: DIT_LQ(5); break;
        case 6: DIT_LQ(6); break;
        case 7: DIT_LQ(7); break;
        case 8: DIT_LQ(8); break;
        default: return hipErrorInvalidValue;
    }
#undef DIT_LQ
    return hipGetLastError();
}

hipError_t launch_ln_modulate_q8(const void *x, int x_f32, int64_t rows, int dim, int rms, const float *shift,
                                 const float *scale, int mode, float eps, int8_t *q, float *qscale, hipStream_t s) {
    TraceScope trace_(s, "ln_modulate_h256q");
    if (trace_.on()) trace_.args("rows=%lld dim=%d", (long long)rows, dim);
    if (rows <= 0) return hipSuccess;
    if (x_f32)
        return rms ? ln_q8_typed<float, true>((const float *)x, rows, dim, shift, scale, mode, eps, q, qscale, s)
                   : ln_q8_typed<float, false>((const float *)x, rows, dim, shift, scale, mode, eps, q, qscale, s);
    return rms ? ln_q8_typed<bf16, true>((const bf16 *)x, rows, dim, shift, scale, mode, eps, q, qscale, s)
               : ln_q8_typed<bf16, false>((const bf16 *)x, rows, dim, shift, scale, mode, eps, q, qscale, s);
}

}  // namespace dit
