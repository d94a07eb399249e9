// Memory-bound kernels of the block and the loop (gfx950):
//   adaln_gemv     m = W act(c) + b            (ERNIE page §IV: 6-way AdaLN modulation;
//                                               §V Bug 4: final modulation, no SiLU)
//   ln_modulate    h = LN(x) * mul + add       (ERNIE page §V Bug 4 modulation form;
//                                               makepad log: affine LN of the ViT)
//   euler          latent += dsigma * v        (zml-flow-rs page §IV "Euler sign +1")
//   timestep_emb   [cos(t w) | sin(t w)]       (zml-flow-rs page §IV flip_sin_to_cos)
//   f32_to_bf16, vt_pad_zero                   (layout helpers of the path)
#include <algorithm>

#include "common.h"
#include "trace.h"

namespace dit {

// ---------------------------------------------------------------------------
// AdaLN GEMV: one wave per 4 output rows; each lane streams 8-element chunks
// of the 4 weight rows (16 bytes of bf16, or 32 bytes of fp32 weights) against
// act(c) of the same 8 inputs, so a lane keeps 8 independent chunk loads in
// flight per unrolled step.
// ---------------------------------------------------------------------------
constexpr int kGemvRows = 4;

struct f32x8 {
    floatx4 lo, hi;
    __device__ __forceinline__ float operator[](int k) const { return k < 4 ? lo[k] : hi[k - 4]; }
};
__device__ __forceinline__ bf16x8 load8(const bf16 *p) { return *(const bf16x8 *)p; }
__device__ __forceinline__ f32x8 load8(const float *p) {
    return f32x8{*(const floatx4 *)p, *(const floatx4 *)(p + 4)};
}

template <typename TW>
__global__ __launch_bounds__(256)
void adaln_gemv_kernel(const TW *__restrict__ W, const float *__restrict__ b, const float *__restrict__ c,
                       int out_dim, int in_dim, int silu_input, float *__restrict__ m) {
    const int lane = threadIdx.x & 63;
    const int o0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kGemvRows;
    if (o0 >= out_dim) return;
    const int nch = in_dim >> 3;   // 8-element chunks per row
    float acc[kGemvRows] = {0.f, 0.f, 0.f, 0.f};
    const TW *wr[kGemvRows];
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) wr[r] = W + (size_t)min(o0 + r, out_dim - 1) * in_dim;

    for (int ch0 = lane; ch0 < nch; ch0 += 128) {
        decltype(load8(W)) wv[2][kGemvRows];
        floatx4 c0[2], c1[2];
        bool ok[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ch = ch0 + u * 64;
            ok[u] = ch < nch;
            const int chs = ok[u] ? ch : ch0;
#pragma unroll
            for (int r = 0; r < kGemvRows; ++r) wv[u][r] = load8(wr[r] + chs * 8);
            c0[u] = *(const floatx4 *)(c + chs * 8);
            c1[u] = *(const floatx4 *)(c + chs * 8 + 4);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (!ok[u]) continue;
            float a[8] = {c0[u][0], c0[u][1], c0[u][2], c0[u][3], c1[u][0], c1[u][1], c1[u][2], c1[u][3]};
            if (silu_input) {
#pragma unroll
                for (int k = 0; k < 8; ++k) a[k] = silu_f(a[k]);
            }
#pragma unroll
            for (int r = 0; r < kGemvRows; ++r)
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[r] += (float)wv[u][r][k] * a[k];
        }
    }
#pragma unroll
    for (int r = 0; r < kGemvRows; ++r) {
        const float s = group_sum<64>(acc[r]);
        if (lane == 0 && o0 + r < out_dim) m[o0 + r] = s + (b ? b[o0 + r] : 0.f);
    }
}

hipError_t launch_adaln_gemv(const void *w, int w_f32, const float *b, const float *c, int out_dim, int in_dim,
                             int silu_input, float *m, hipStream_t s) {
    TraceScope trace_(s, "adaln_gemv");
    if (trace_.on()) trace_.args("out=%d in=%d silu=%d", out_dim, in_dim, silu_input);
    const int waves = (out_dim + kGemvRows - 1) / kGemvRows;
    if (w_f32)
        hipLaunchKernelGGL(adaln_gemv_kernel<float>, dim3((waves + 3) / 4), dim3(256), 0, s, (const float *)w, b, c,
                           out_dim, in_dim, silu_input, m);
    else
        hipLaunchKernelGGL(adaln_gemv_kernel<bf16>, dim3((waves + 3) / 4), dim3(256), 0, s, (const bf16 *)w, b, c,
                           out_dim, in_dim, silu_input, m);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LayerNorm (or RMSNorm) + modulation, one wave per row, 8 rows per workgroup
// sharing one LDS copy of the modulation vectors.  The row stays in registers
// (IT = dim/256 float4 per lane) between the mean pass, the centred variance
// pass and the output pass, so x is read from HBM exactly once.  IT is a
// template parameter so that all IT loads of a lane are issued back to back
// (a runtime trip count puts each load behind its own branch and the wave
// then waits for every load before issuing the next).
//   mode 0: h = n * (1 + scale) + shift      mode 1: h = n * scale + shift
// n = (x - mean) / sqrt(var + eps) (LayerNorm) or x / sqrt(mean(x^2) + eps)
// (RMSNorm, RMS = true: no centring).  h is bf16, or fp32 (TH = float) on the
// fp32 path.
// ---------------------------------------------------------------------------
template <typename TH>
__device__ __forceinline__ void store4(TH *p, const floatx4 &v) {
    if constexpr (sizeof(TH) == 4) {
        *(floatx4 *)p = v;
    } else {
        bf16x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = f2bf(v[k]);
        *(bf16x4 *)p = o;
    }
}

// rows (one wave each) per workgroup: they share one LDS copy of the modulation
constexpr int kLnRows = 8;

template <typename TX, typename TH, int IT, bool RMS>
__global__ __launch_bounds__(kLnRows * 64)
void ln_modulate_kernel(const TX *__restrict__ x, int64_t rows, const float *__restrict__ shift,
                        const float *__restrict__ scale, int mode, float eps, TH *__restrict__ h) {
    constexpr int dim = IT * 256;
    // multiplier (1 + scale, or scale in mode 1, or 1 without scale) and addend
    // (shift, or 0), loaded once per workgroup instead of once per row
    __shared__ floatx4 s_mul[IT * 64], s_add[IT * 64];
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kLnRows + (threadIdx.x >> 6);
    const bool valid = row < rows;
    const TX *xr = x + (valid ? row : 0) * dim;
    // the row's loads go out first; the modulation fill below overlaps their latency
    floatx4 v[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int i = it * 256 + lane * 4;
        if constexpr (sizeof(TX) == 4) {
            v[it] = *(const floatx4 *)(xr + i);
        } else {
            const bf16x4 t = *(const bf16x4 *)(xr + i);
            v[it] = floatx4{(float)t[0], (float)t[1], (float)t[2], (float)t[3]};
        }
    }
    const float one = mode == 0 ? 1.0f : 0.0f;
    for (int i = threadIdx.x; i < IT * 64; i += kLnRows * 64) {
        floatx4 mul = {1.f, 1.f, 1.f, 1.f}, add = {0.f, 0.f, 0.f, 0.f};
        if (scale) mul = *(const floatx4 *)(scale + 4 * i) + one;
        if (shift) add = *(const floatx4 *)(shift + 4 * i);
        s_mul[i] = mul;
        s_add[i] = add;
    }
    __syncthreads();
    if (!valid) return;
    float mean = 0.f;
    if (!RMS) {
        float s = 0.f;
#pragma unroll
        for (int it = 0; it < IT; ++it) s += (v[it][0] + v[it][1]) + (v[it][2] + v[it][3]);
        mean = group_sum<64>(s) * (1.0f / dim);
    }
    float ss = 0.f;
#pragma unroll
    for (int it = 0; it < IT; ++it)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float d = v[it][k] - mean;
            v[it][k] = d;
            ss += d * d;
        }
    const float rstd = rsqrtf(group_sum<64>(ss) * (1.0f / dim) + eps);
    TH *hr = h + row * dim;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const floatx4 mul = s_mul[it * 64 + lane], add = s_add[it * 64 + lane];
        floatx4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = v[it][k] * rstd * mul[k] + add[k];
        store4(hr + it * 256 + lane * 4, o);
    }
}

template <typename TX, typename TH, bool RMS>
static hipError_t ln_modulate_typed(const TX *x, int64_t rows, int dim, const float *shift, const float *scale,
                                    int mode, float eps, TH *h, hipStream_t s) {
    const dim3 grid((unsigned)((rows + kLnRows - 1) / kLnRows));
    switch (dim >> 8) {
#define DIT_LN_CASE(n)                                                                                 \
    case n:                                                                                            \
        hipLaunchKernelGGL((ln_modulate_kernel<TX, TH, n, RMS>), grid, dim3(kLnRows * 64), 0, s, x, rows, shift, \
                           scale, mode, eps, h);                                                       \
        break;
        DIT_LN_CASE(1) DIT_LN_CASE(2) DIT_LN_CASE(3) DIT_LN_CASE(4) DIT_LN_CASE(5) DIT_LN_CASE(6)
        DIT_LN_CASE(7) DIT_LN_CASE(8) DIT_LN_CASE(9) DIT_LN_CASE(10) DIT_LN_CASE(11) DIT_LN_CASE(12)
        DIT_LN_CASE(13) DIT_LN_CASE(14) DIT_LN_CASE(15) DIT_LN_CASE(16) DIT_LN_CASE(17) DIT_LN_CASE(18)
        DIT_LN_CASE(19) DIT_LN_CASE(20) DIT_LN_CASE(21) DIT_LN_CASE(22) DIT_LN_CASE(23) DIT_LN_CASE(24)
        DIT_LN_CASE(25) DIT_LN_CASE(26) DIT_LN_CASE(27) DIT_LN_CASE(28) DIT_LN_CASE(29) DIT_LN_CASE(30)
        DIT_LN_CASE(31) DIT_LN_CASE(32)
#undef DIT_LN_CASE
        default:
            return hipErrorInvalidValue;   // dim must be a multiple of 256 in [256, 8192]
    }
    return hipGetLastError();
}

hipError_t launch_ln_modulate(const void *x, int x_f32, int64_t rows, int dim, int rms, const float *shift,
                              const float *scale, int mode, float eps, bf16 *h, hipStream_t s) {
    TraceScope trace_(s, "ln_modulate");
    if (trace_.on()) trace_.args("rows=%lld dim=%d x_f32=%d", (long long)rows, dim, x_f32);
    if (dim % 256 != 0) return hipErrorInvalidValue;
    if (x_f32)
        return rms ? ln_modulate_typed<float, bf16, true>((const float *)x, rows, dim, shift, scale, mode, eps, h, s)
                   : ln_modulate_typed<float, bf16, false>((const float *)x, rows, dim, shift, scale, mode, eps, h, s);
    return rms ? ln_modulate_typed<bf16, bf16, true>((const bf16 *)x, rows, dim, shift, scale, mode, eps, h, s)
               : ln_modulate_typed<bf16, bf16, false>((const bf16 *)x, rows, dim, shift, scale, mode, eps, h, s);
}

hipError_t launch_ln_modulate_f32(const float *x, int64_t rows, int dim, int rms, const float *shift,
                                  const float *scale, int mode, float eps, float *h, hipStream_t s) {
    TraceScope trace_(s, "ln_modulate_f32");
    if (trace_.on()) trace_.args("rows=%lld dim=%d", (long long)rows, dim);
    if (dim % 256 != 0) return hipErrorInvalidValue;
    return rms ? ln_modulate_typed<float, float, true>(x, rows, dim, shift, scale, mode, eps, h, s)
               : ln_modulate_typed<float, float, false>(x, rows, dim, shift, scale, mode, eps, h, s);
}

// ---------------------------------------------------------------------------
// Euler step: latent += dsigma * v  (float4 body, scalar tail)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256)
void euler_kernel(float *__restrict__ lat, const float *__restrict__ v, int64_t n, float dsigma) {
    const int64_t n4 = n >> 2;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) {
        floatx4 a = ((floatx4 *)lat)[i];
        const floatx4 b = ((const floatx4 *)v)[i];
        a += dsigma * b;
        ((floatx4 *)lat)[i] = a;
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
        const int64_t i = n4 * 4 + threadIdx.x;
        lat[i] += dsigma * v[i];
    }
}

hipError_t launch_euler(float *latent, const float *v, int64_t n, float dsigma, hipStream_t s) {
    TraceScope trace_(s, "euler_update");
    if (trace_.on()) trace_.args("n=%lld", (long long)n);
    const int64_t n4 = (n >> 2) + 1;
    const int blocks = (int)std::min<int64_t>((n4 + 255) / 256, 4096);
    hipLaunchKernelGGL(euler_kernel, dim3(blocks), dim3(256), 0, s, latent, v, n, dsigma);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// timestep embedding [cos(t w_j) | sin(t w_j)], w_j = exp(-ln(1e4) j / half)
// ---------------------------------------------------------------------------
__global__ void timestep_embedding_kernel(float t, int half, float *__restrict__ out) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= half) return;
    const float w = expf(-9.210340371976184f * (float)j / (float)half);   // ln(10000)
    const float a = t * w;
    out[j] = cosf(a);
    out[half + j] = sinf(a);
}

hipError_t launch_timestep_embedding(float t, int dim, float *out, hipStream_t s) {
    TraceScope trace_(s, "timestep_embedding");
    if (trace_.on()) trace_.args("dim=%d", dim);
    const int half = dim / 2;
    hipLaunchKernelGGL(timestep_embedding_kernel, dim3((half + 255) / 256), dim3(256), 0, s, t, half, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 -> bf16 (round to nearest even)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256)
void f32_to_bf16_kernel(const float *__restrict__ x, bf16 *__restrict__ y, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) y[i] = f2bf(x[i]);
}

hipError_t launch_f32_to_bf16(const float *x, bf16 *y, int64_t n, hipStream_t s) {
    TraceScope trace_(s, "f32_to_bf16");
    if (trace_.on()) trace_.args("n=%lld", (long long)n);
    const int blocks = (int)std::min<int64_t>((n + 255) / 256, 8192);
    hipLaunchKernelGGL(f32_to_bf16_kernel, dim3(blocks), dim3(256), 0, s, x, y, n);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// zero the padded key positions [seq, seq_pad) of every row of transposed V
// ---------------------------------------------------------------------------
template <typename TV>
__global__ __launch_bounds__(256)
void vt_pad_zero_kernel(TV *__restrict__ vt, int rows, int seq, int seq_pad) {
    const int pad = seq_pad - seq;
    const int64_t n = (int64_t)rows * pad;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
        const int64_t r = i / pad;
        const int c = (int)(i - r * pad);
        vt[r * seq_pad + seq + c] = TV(0.f);
    }
}

hipError_t launch_vt_pad_zero(void *vt, int vt_f32, int rows, int seq, int seq_pad, hipStream_t s) {
    const int64_t n = (int64_t)rows * (seq_pad - seq);
    if (n <= 0) return hipSuccess;   // nothing to zero: no launch, and no trace record
    TraceScope trace_(s, "vt_pad_zero");
    if (trace_.on()) trace_.args("rows=%d seq=%d pad=%d", rows, seq, seq_pad);
    const int blocks = (int)std::min<int64_t>((n + 255) / 256, 4096);
    if (vt_f32)
        hipLaunchKernelGGL(vt_pad_zero_kernel<float>, dim3(blocks), dim3(256), 0, s, (float *)vt, rows, seq, seq_pad);
    else
        hipLaunchKernelGGL(vt_pad_zero_kernel<bf16>, dim3(blocks), dim3(256), 0, s, (bf16 *)vt, rows, seq, seq_pad);
    return hipGetLastError();
}

}  // namespace dit
