// Mask-free flash attention forward for gfx950 (bf16 MFMA, fp32 online softmax).
//
// O_h = softmax(Q_h K_g^T / sqrt(hd)) V_g per sequence and query head h, with
// KV head g = h / (H / Hkv) (ERNIE page §VII Decision 2 and §IX "Flash SDPA";
// grouped KV heads as in the zml-flow-rs page §VI attention signature).
//
// Work split: one workgroup = 4 waves = 256 queries of one (batch, head); each
// wave owns 64 queries.  Keys stream through LDS in tiles of 64 (K tile and
// the transposed V tile, double-buffered, next tile prefetched into registers
// while the current one is consumed).
//
// The scores are computed transposed, S^T = K Q^T (MFMA A = K rows, B = Q rows),
// so an accumulator lane owns one query column and 16 keys: the running row
// max and row sum are in-lane reductions plus one exchange with lane ^ 32.
// P^T is then already in the B-operand layout of O^T += V^T P^T, up to a fixed
// permutation of the 16 keys of each MFMA k-step, which the V^T fragment reads
// apply as well (two 8-byte LDS reads per fragment).
#include "common.h"

namespace dit {

template <int HD>
__global__ __launch_bounds__(256, 1)
void flash_attn_kernel(const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ Vt,
                       bf16 *__restrict__ O, int S, int S_pad, int H, int Hkv, float scale_log2) {
    constexpr int QW = 64;                   // queries per wave
    constexpr int BQ = 4 * QW;               // queries per workgroup
    constexpr int BKV = 64;                  // keys per tile
    constexpr int KCH = HD / 8;              // 16-byte chunks per K row
    constexpr int KT_BYTES = BKV * HD * 2;   // K tile  [64 keys][HD]
    constexpr int VT_BYTES = HD * BKV * 2;   // V^T tile [HD][64 keys]
    constexpr int STAGE = KT_BYTES + VT_BYTES;
    constexpr int KLD = BKV * KCH / 256;     // K chunks per thread
    constexpr int VLD = HD * 8 / 256;        // V^T chunks per thread
    constexpr int KK = HD / 16;              // MFMA k-steps over head_dim
    constexpr int DS = HD / 32;              // 32-row blocks of O^T
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    const int h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / Hkv);
    const bf16 *Qh = Q + (size_t)(b * H + h) * S * HD;
    const bf16 *Kh = K + (size_t)(b * Hkv + g) * S * HD;
    const bf16 *Vh = Vt + (size_t)(b * Hkv + g) * HD * S_pad;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int q_base = blockIdx.x * BQ + wave * QW;

    // Q as the B operand: lane -> query q_base + qs*32 + lrow, dims kk*16 + lhalf*8 .. +8
    bf16x8 qf[2][KK];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        const int qr = min(q_base + qs * 32 + lrow, S - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[qs][kk] = *(const bf16x8 *)(Qh + (size_t)qr * HD + kk * 16 + lhalf * 8);
    }

    uint4 rk[KLD], rv[VLD];
    auto gload = [&](int kv0) {
#pragma unroll
        for (int q = 0; q < KLD; ++q) {
            const int id = q * 256 + tid, r = id / KCH, c = id % KCH;
            const int key = min(kv0 + r, S - 1);              // tail keys: any valid row, masked below
            rk[q] = *(const uint4 *)(Kh + (size_t)key * HD + c * 8);
        }
#pragma unroll
        for (int q = 0; q < VLD; ++q) {
            const int id = q * 256 + tid, d = id >> 3, c = id & 7;
            rv[q] = *(const uint4 *)(Vh + (size_t)d * S_pad + kv0 + c * 8);   // [S, S_pad) is zero
        }
    };
    // K tile: row r (key) of HD*2 bytes, 16-byte chunk c at slot c ^ (r & 7).
    // V^T tile: row d of 128 bytes = 16 slots of 8 bytes (4 keys); slot s at s ^ (d & 15).
    auto lstore = [&](int st) {
        uint8_t *base = smem + st * STAGE;
#pragma unroll
        for (int q = 0; q < KLD; ++q) {
            const int id = q * 256 + tid, r = id / KCH, c = id % KCH;
            *(uint4 *)(base + r * (HD * 2) + ((c ^ (r & 7)) << 4)) = rk[q];
        }
#pragma unroll
        for (int q = 0; q < VLD; ++q) {
            const int id = q * 256 + tid, d = id >> 3, c = id & 7;
            uint8_t *row = base + KT_BYTES + d * 128;
            *(uint2 *)(row + (((2 * c) ^ (d & 15)) << 3)) = make_uint2(rv[q].x, rv[q].y);
            *(uint2 *)(row + (((2 * c + 1) ^ (d & 15)) << 3)) = make_uint2(rv[q].z, rv[q].w);
        }
    };

    floatx16 oacc[DS][2];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[ds][qs][e] = 0.f;
    float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.f, 0.f};

    const int ntiles = (S + BKV - 1) / BKV;
    gload(0);
    lstore(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        const int kv0 = t * BKV;
        if (t + 1 < ntiles) gload(kv0 + BKV);
        const uint8_t *sk = smem + cur * STAGE;
        const uint8_t *sv = sk + KT_BYTES;

        // S^T[key, q] for 64 keys x 64 queries
        floatx16 sacc[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int qs = 0; qs < 2; ++qs)
#pragma unroll
                for (int e = 0; e < 16; ++e) sacc[ks][qs][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int c = kk * 2 + lhalf;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 kf = *(const bf16x8 *)(sk + (ks * 32 + lrow) * (HD * 2) + ((c ^ (lrow & 7)) << 4));
#pragma unroll
                for (int qs = 0; qs < 2; ++qs)
                    sacc[ks][qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qs][kk], sacc[ks][qs], 0, 0, 0);
            }
        }

        // online softmax (log2 domain); keys >= S are masked in the last tile
        const bool tail = kv0 + BKV > S;
        bf16x8 pf[4][2];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
            float mx = -INFINITY;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float v = sacc[ks][qs][e] * scale_log2;
                    if (tail) {
                        const int key = kv0 + ks * 32 + ((e >> 2) << 3) + (lhalf << 2) + (e & 3);
                        if (key >= S) v = -INFINITY;
                    }
                    sacc[ks][qs][e] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mnew = fmaxf(mrun[qs], mx);
            const float alpha = __builtin_amdgcn_exp2f(mrun[qs] - mnew);
            mrun[qs] = mnew;
            float rs = 0.f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float p = __builtin_amdgcn_exp2f(sacc[ks][qs][e] - mnew);
                    rs += p;
                    pf[ks * 2 + (e >> 3)][qs][e & 7] = f2bf(p);
                }
            lrun[qs] = lrun[qs] * alpha + rs;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[ds][qs][e] *= alpha;
        }

        // O^T[d, q] += V^T[d, keys] P^T[keys, q]
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
            const int slot = k2 * 4 + lhalf;   // keys k2*16 + lhalf*4 .. +3 ; second half at slot + 2
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const int d = ds * 32 + lrow;
                const uint8_t *row = sv + d * 128;
                const uint2 lo = *(const uint2 *)(row + ((slot ^ (d & 15)) << 3));
                const uint2 hi = *(const uint2 *)(row + (((slot + 2) ^ (d & 15)) << 3));
                const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
                for (int qs = 0; qs < 2; ++qs)
                    oacc[ds][qs] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[k2][qs], oacc[ds][qs], 0, 0, 0);
            }
        }

        if (t + 1 < ntiles) lstore(cur ^ 1);
        __syncthreads();
    }

    // normalise and store O[b*S + q, h*HD + d] (4 consecutive d per 8-byte store)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
        const float l = lrun[qs] + __shfl_xor(lrun[qs], 32, 64);
        const float inv = 1.0f / l;
        const int q = q_base + qs * 32 + lrow;
        if (q < S) {
            bf16 *orow = O + ((size_t)b * S + q) * (size_t)(H * HD) + (size_t)h * HD;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    bf16x4 v;
#pragma unroll
                    for (int u = 0; u < 4; ++u) v[u] = f2bf(oacc[ds][qs][e4 * 4 + u] * inv);
                    *(bf16x4 *)(orow + ds * 32 + e4 * 8 + lhalf * 4) = v;
                }
        }
    }
}

hipError_t launch_flash_attention(const bf16 *q, const bf16 *k, const bf16 *vt, bf16 *out, int batch, int seq,
                                  int seq_pad, int heads, int kv_heads, int head_dim, hipStream_t s) {
    const dim3 grid((seq + 255) / 256, heads, batch);
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)head_dim);
    if (head_dim == 128)
        hipLaunchKernelGGL(flash_attn_kernel<128>, grid, dim3(256), 0, s, q, k, vt, out, seq, seq_pad, heads,
                           kv_heads, scale_log2);
    else
        hipLaunchKernelGGL(flash_attn_kernel<64>, grid, dim3(256), 0, s, q, k, vt, out, seq, seq_pad, heads,
                           kv_heads, scale_log2);
    return hipGetLastError();
}

}  // namespace dit
