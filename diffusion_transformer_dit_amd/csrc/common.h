// Shared device types and helpers of the gfx950 kernels (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef int intx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16 v) { return (float)v; }
__device__ __forceinline__ bf16 f2bf(float v) { return (bf16)v; }   // v_cvt_pk_bf16_f32, round-to-nearest-even

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// butterfly sum over groups of `W` consecutive lanes (W a power of two <= 64)
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = 1; m < W; m <<= 1) v += __shfl_xor(v, m, 64);
    return v;
}

template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int m = 1; m < W; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

// Register-free global -> LDS loads (buffer_load_dwordx4 ... lds): one
// instruction moves 64 lanes x 16 bytes into 1 KiB of LDS at the wave-uniform
// LDS address (lane l at +16 l).
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14], expcnt
// [6:4], lgkmcnt [11:8]); LGKM = 0 also drains this wave's LDS reads.
template <int N, int LGKM = 15>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// would wait for every outstanding buffer->LDS load, including the stages
// still meant to be in flight.  Ordering is provided by the explicit waits.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Reciprocals in the GLU activations use v_rcp_f32 (1 ulp) instead of the
// IEEE division sequence (about ten instructions): these run once per output
// element in the GEMM epilogue, where the division was a third of the
// epilogue's instructions, and 1 ulp sits far below the bf16 output rounding.
__device__ __forceinline__ float rcp_f(float x) { return __builtin_amdgcn_rcpf(x); }

// clamped GELU in its tanh approximation: 0.5 z (1 + tanh(a)), a = sqrt(2/pi)(z + 0.044715 z^3)
// clamped to [-20, 20], result clamped to +-65504 (ERNIE page §V Bug 1).  tanh(a) is
// 1 - 2 / (e^{2a} + 1), finite for |a| <= 20.
__device__ __forceinline__ float gelu_tanh_f(float z) {
    float a = 0.7978845608028654f * (z + 0.044715f * z * z * z);
    a = fminf(fmaxf(a, -20.0f), 20.0f);   // an overflowing z^3 gives +-inf: clamped like any large value
    const float t = 1.0f - 2.0f * rcp_f(__expf(2.0f * a) + 1.0f);
    return fminf(fmaxf(0.5f * z * (1.0f + t), -65504.0f), 65504.0f);
}

// gate function before the gated residual: 0 identity, 1 tanh, 2 sigmoid
__device__ __forceinline__ float gate_f(float g, int fn) {
    if (fn == 1) return tanhf(g);
    if (fn == 2) return 1.0f / (1.0f + expf(-g));
    return g;
}

__device__ __forceinline__ float silu_f(float z) {
    // z * sigmoid(z); expf of a large positive -z gives inf, rcp(inf) = 0 and z * 0 -> -0
    return z * rcp_f(1.0f + __expf(-z));
}

}  // namespace dit

// ---------------------------------------------------------------------------
// launchers (host side), implemented in the .hip files of this directory
// ---------------------------------------------------------------------------
namespace dit {

struct QkvEpiArgs {
    int batch, seq, seq_pad, heads, kv_heads, head_dim;
    int qk_norm, rope_half;
    int rms;          // qk-norm kind: 0 LayerNorm, 1 RMSNorm
    int rope_first;   // 0: qk-norm then RoPE, 1: RoPE then qk-norm
    float eps;
    const float *q_g, *q_b, *k_g, *k_b;
    const float *cos_t, *sin_t;
    void *q, *k, *vt;    // bf16, or fp32 on the fp32 parity path
};

// gate_fn: 0 identity, 1 tanh, 2 sigmoid (applied to gate[n]); act: 0 SiLU, 1 clamped GELU-tanh
hipError_t launch_gemm_residual(const bf16 *a, const bf16 *w, int64_t M, int N, int K,
                                const void *resid, int resid_f32, const float *gate, int gate_fn,
                                const float *bias, void *out, int out_f32, hipStream_t s);
hipError_t launch_gemm_swiglu(const bf16 *a, const bf16 *w, int64_t M, int F, int K, int act,
                              bf16 *u, hipStream_t s);
hipError_t launch_gemm_qkv(const bf16 *h, const bf16 *w, int64_t M, int N, int K,
                           const QkvEpiArgs &e, hipStream_t s);

// W8A8 H256 projections: a / w int8 codes [M, K] / [rows, K] with fp32 row scales
// a_scale [M] and w_scale [rows of w]; the products are dequantized before the
// same epilogues
hipError_t launch_gemm_residual_q8(const int8_t *a, const float *a_scale, const int8_t *w, const float *w_scale,
                                   int64_t M, int N, int K, const void *resid, int resid_f32, const float *gate,
                                   int gate_fn, const float *bias, void *out, int out_f32, hipStream_t s);
hipError_t launch_gemm_swiglu_q8(const int8_t *a, const float *a_scale, const int8_t *w, const float *w_scale,
                                 int64_t M, int F, int K, int act, bf16 *u, hipStream_t s);
hipError_t launch_gemm_qkv_q8(const int8_t *h, const float *h_scale, const int8_t *w, const float *w_scale,
                              int64_t M, int N, int K, const QkvEpiArgs &e, hipStream_t s);
// the fp32 parity path: fp32 operands, fp32 outputs (q, k, vt and u fp32)
hipError_t launch_gemm_residual_f32(const float *a, const float *w, int64_t M, int N, int K, const float *resid,
                                    const float *gate, int gate_fn, const float *bias, float *out, hipStream_t s);
hipError_t launch_gemm_swiglu_f32(const float *a, const float *w, int64_t M, int F, int K, int act, float *u,
                                  hipStream_t s);
hipError_t launch_gemm_qkv_f32(const float *h, const float *w, int64_t M, int N, int K, const QkvEpiArgs &e,
                               hipStream_t s);
bool quantize_h256_supported(int cols);
hipError_t launch_quantize_h256(const void *x, int x_f32, int64_t rows, int cols, int8_t *q, float *scale,
                                hipStream_t s);
hipError_t launch_ln_modulate_q8(const void *x, int x_f32, int64_t rows, int dim, int rms, const float *shift,
                                 const float *scale, int mode, float eps, int8_t *q, float *qscale, hipStream_t s);

// nsplit > 1 with part != NULL (attention_split_bytes(batch, heads, head_dim,
// nsplit) bytes): the partial last q tile is split over nsplit key chunks
hipError_t launch_flash_attention(const bf16 *q, const bf16 *k, const bf16 *vt, bf16 *out,
                                  int batch, int seq, int seq_pad, int heads, int kv_heads,
                                  int head_dim, int nsplit, void *part, hipStream_t s);
// fp32 operands (the fp32 parity path); no split
hipError_t launch_flash_attention_f32(const float *q, const float *k, const float *vt, float *out, int batch,
                                      int seq, int seq_pad, int heads, int kv_heads, int head_dim, hipStream_t s);
int attention_split_count(int batch, int seq, int heads, int cus);
size_t attention_split_bytes(int batch, int heads, int head_dim, int nsplit);
int device_cu_count();

hipError_t launch_adaln_gemv(const void *w, int w_f32, const float *b, const float *c, int out_dim,
                             int in_dim, int silu_input, float *m, hipStream_t s);
hipError_t launch_ln_modulate(const void *x, int x_f32, int64_t rows, int dim, int rms,
                              const float *shift, const float *scale, int mode, float eps,
                              bf16 *h, hipStream_t s);
hipError_t launch_ln_modulate_f32(const float *x, int64_t rows, int dim, int rms, const float *shift,
                                  const float *scale, int mode, float eps, float *h, hipStream_t s);
hipError_t launch_euler(float *latent, const float *v, int64_t n, float dsigma, hipStream_t s);
hipError_t launch_timestep_embedding(float t, int dim, float *out, hipStream_t s);
hipError_t launch_f32_to_bf16(const float *x, bf16 *y, int64_t n, hipStream_t s);
hipError_t launch_vt_pad_zero(void *vt, int vt_f32, int rows, int seq, int seq_pad, hipStream_t s);

}  // namespace dit
