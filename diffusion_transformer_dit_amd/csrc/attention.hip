// Mask-free flash attention forward for gfx950 (bf16 MFMA, fp32 online softmax).
//
// O_h = softmax(Q_h K_g^T / sqrt(hd)) V_g per sequence and query head h, with
// KV head g = h / (H / Hkv) (ERNIE page §VII Decision 2 and §IX "Flash SDPA";
// grouped KV heads as in the zml-flow-rs page §VI attention signature).
//
// Work split: one workgroup = 8 waves = 256 queries of one (batch, head); each
// wave owns 32 queries, two waves share a SIMD so that one wave's softmax
// (VALU, transcendental exp2) overlaps the other wave's MFMAs.  Keys stream
// through LDS in tiles of 64 (the K tile and the transposed V tile,
// double-buffered; the next tile is prefetched into registers while the
// current one is consumed).
//
// The scores are computed transposed, S^T = K Q^T (MFMA A = K rows, B = Q rows),
// so an accumulator lane owns one query column and 16 keys: the running row
// max and row sum are in-lane reductions plus one exchange with lane ^ 32.
// P^T is then already in the B-operand layout of O^T += V^T P^T, up to a fixed
// permutation of the 16 keys of each MFMA k-step ({0-3, 8-11} in lanes 0-31,
// {4-7, 12-15} in lanes 32-63); the V^T tile is stored in LDS with its keys in
// that order, so every V^T fragment is one 16-byte read.
#include "common.h"

namespace dit {

template <int HD>
__global__ __launch_bounds__(512, 1)
void flash_attn_kernel(const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ Vt,
                       bf16 *__restrict__ O, int S, int S_pad, int H, int Hkv, float scale_log2) {
    constexpr int NW = 8;                    // waves per workgroup
    constexpr int QW = 32;                   // queries per wave
    constexpr int BQ = NW * QW;              // queries per workgroup
    constexpr int BKV = 64;                  // keys per tile
    constexpr int NT = NW * kWave;           // threads
    constexpr int KCH = HD / 8;              // 16-byte chunks per K row
    constexpr int KT_BYTES = BKV * HD * 2;   // K tile  [64 keys][HD]
    constexpr int VT_BYTES = HD * BKV * 2;   // V^T tile [HD][64 keys]
    constexpr int STAGE = KT_BYTES + VT_BYTES;
    constexpr int KLD = BKV * KCH / NT;      // K chunks per thread
    constexpr int VLD = HD * 8 / NT;         // V^T chunks per thread
    constexpr int KK = HD / 16;              // MFMA k-steps over head_dim
    constexpr int DS = HD / 32;              // 32-row blocks of O^T
    static_assert(KLD >= 1 && VLD >= 1, "tile vs threads");
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

    // LDS layouts (gfx950: 64 banks, 256 B per cycle; a ds_read_b128 serves 16
    // lanes per cycle, a ds_write_b64 32 lanes).
    // K tile: row r (key) of HD*2 bytes; 16-byte chunk c at slot c ^ kswz(r):
    //   HD = 128: 256-byte rows, kswz = r & 15 (16 rows hit 16 distinct slots);
    //   HD = 64: 128-byte rows, two per bank line, kswz = (r >> 1) & 7.
    // V^T tile: row d of 128 bytes.  Keys 4q..4q+3 of 16-key group g sit in
    //   8-byte slot 4g + perm(q), perm = {0, 2, 1, 3}, so 16-byte slot 2g+h
    //   holds exactly the 8 keys lane half h feeds to the MFMA; 16-byte slot s
    //   is stored at s ^ ((d >> 1) & 7).
    auto kswz = [](int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); };
    auto vslot = [](int d, int s16) { return (s16 ^ ((d >> 1) & 7)) << 4; };

    const int h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / Hkv);
    const bf16 *Qh = Q + (size_t)(b * H + h) * S * HD;
    const bf16 *Kh = K + (size_t)(b * Hkv + g) * S * HD;
    const bf16 *Vh = Vt + (size_t)(b * Hkv + g) * HD * S_pad;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int q_base = blockIdx.x * BQ + wave * QW;

    // Q as the B operand: lane -> query q_base + lrow, dims kk*16 + lhalf*8 .. +8
    bf16x8 qf[KK];
    {
        const int qr = min(q_base + lrow, S - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const bf16x8 *)(Qh + (size_t)qr * HD + kk * 16 + lhalf * 8);
    }

    uint4 rk[KLD], rv[VLD];
#define DIT_ATT_GLOAD(kv0)                                                                          \
    do {                                                                                            \
        _Pragma("unroll") for (int q = 0; q < KLD; ++q) {                                          \
            const int id = q * NT + tid, r = id / KCH, c = id % KCH;                                \
            const int key = min((kv0) + r, S - 1);   /* tail keys: any valid row, masked below */   \
            rk[q] = *(const uint4 *)(Kh + (size_t)key * HD + c * 8);                                \
        }                                                                                           \
        _Pragma("unroll") for (int q = 0; q < VLD; ++q) {                                          \
            const int id = q * NT + tid, d = id >> 3, c = id & 7;                                   \
            rv[q] = *(const uint4 *)(Vh + (size_t)d * S_pad + (kv0) + c * 8); /* [S,S_pad) zero */  \
        }                                                                                           \
    } while (0)
#define DIT_ATT_LSTORE(st)                                                                          \
    do {                                                                                            \
        uint8_t *base_ = smem + (st) * STAGE;                                                       \
        _Pragma("unroll") for (int q = 0; q < KLD; ++q) {                                          \
            const int id = q * NT + tid, r = id / KCH, c = id % KCH;                                \
            *(uint4 *)(base_ + r * (HD * 2) + ((c ^ kswz(r)) << 4)) = rk[q];                        \
        }                                                                                           \
        _Pragma("unroll") for (int q = 0; q < VLD; ++q) {                                          \
            const int id = q * NT + tid, d = id >> 3, c = id & 7;                                   \
            /* keys 8c..8c+3 -> 8-byte slot 4(c/2) + (c&1); keys 8c+4.. -> 4(c/2) + 2 + (c&1) */    \
            const int lo = ((c >> 1) << 2) + (c & 1), hi = lo + 2;                                  \
            uint8_t *row = base_ + KT_BYTES + d * 128;                                              \
            *(uint2 *)(row + vslot(d, lo >> 1) + ((lo & 1) << 3)) = make_uint2(rv[q].x, rv[q].y);  \
            *(uint2 *)(row + vslot(d, hi >> 1) + ((hi & 1) << 3)) = make_uint2(rv[q].z, rv[q].w);  \
        }                                                                                           \
    } while (0)

    floatx16 oacc[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[ds][e] = 0.f;
    float mraw = -INFINITY;     // running max of the raw (unscaled) scores of this lane's query
    float lsum = 0.f;           // this lane's partial row sum (the other 16 keys live in lane ^ 32)

    const int ntiles = (S + BKV - 1) / BKV;
    DIT_ATT_GLOAD(0);
    DIT_ATT_LSTORE(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int cur = t & 1;
        const int kv0 = t * BKV;
        if (t + 1 < ntiles) DIT_ATT_GLOAD(kv0 + BKV);
        const uint8_t *sk = smem + cur * STAGE;
        const uint8_t *sv = sk + KT_BYTES;

        // S^T[key, q] for 64 keys x 32 queries
        floatx16 sacc[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[ks][e] = 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const int c = kk * 2 + lhalf;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 kf = *(const bf16x8 *)(sk + (ks * 32 + lrow) * (HD * 2) + ((c ^ kswz(lrow)) << 4));
                sacc[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], sacc[ks], 0, 0, 0);
            }
        }

        // online softmax on raw scores (scale > 0 commutes with max); keys >= S
        // are masked in the last tile
        if (kv0 + BKV > S) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = kv0 + ks * 32 + ((e >> 2) << 3) + (lhalf << 2) + (e & 3);
                    if (key >= S) sacc[ks][e] = -INFINITY;
                }
        }
        float mx = sacc[0][0];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[ks][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // rescale only when some lane's running max grew (wave-uniform branch;
        // lanes whose max did not move get factor 1)
        if (__any(mx > mraw)) {
            const float mnew = fmaxf(mraw, mx);
            const float alpha = __builtin_amdgcn_exp2f((mraw - mnew) * scale_log2);
            mraw = mnew;
            lsum *= alpha;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[ds][e] *= alpha;
        }
        const float neg = -mraw * scale_log2;
        bf16x8 pf[4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[ks][e], scale_log2, neg));
                lsum += p;
                pf[ks * 2 + (e >> 3)][e & 7] = f2bf(p);
            }

        // O^T[d, q] += V^T[d, keys] P^T[keys, q]
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2) {
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const int d = ds * 32 + lrow;
                const bf16x8 vf = *(const bf16x8 *)(sv + d * 128 + vslot(d, k2 * 2 + lhalf));
                oacc[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[k2], oacc[ds], 0, 0, 0);
            }
        }

        // stage cur ^ 1 (tile t - 1) was released by the barrier closing iteration t - 1
        if (t + 1 < ntiles) DIT_ATT_LSTORE(cur ^ 1);
        __syncthreads();
    }
#undef DIT_ATT_GLOAD
#undef DIT_ATT_LSTORE

    // normalise and store O[b*S + q, h*HD + d] (4 consecutive d per 8-byte store)
    const float l = lsum + __shfl_xor(lsum, 32, 64);
    const float inv = 1.0f / l;
    const int q = q_base + lrow;
    if (q < S) {
        bf16 *orow = O + ((size_t)b * S + q) * (size_t)(H * HD) + (size_t)h * HD;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                bf16x4 v;
#pragma unroll
                for (int u = 0; u < 4; ++u) v[u] = f2bf(oacc[ds][e4 * 4 + u] * inv);
                *(bf16x4 *)(orow + ds * 32 + e4 * 8 + lhalf * 4) = v;
            }
    }
}

hipError_t launch_flash_attention(const bf16 *q, const bf16 *k, const bf16 *vt, bf16 *out, int batch, int seq,
                                  int seq_pad, int heads, int kv_heads, int head_dim, hipStream_t s) {
    const dim3 grid((seq + 255) / 256, heads, batch);
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)head_dim);
    if (head_dim == 128)
        hipLaunchKernelGGL(flash_attn_kernel<128>, grid, dim3(512), 0, s, q, k, vt, out, seq, seq_pad, heads,
                           kv_heads, scale_log2);
    else
        hipLaunchKernelGGL(flash_attn_kernel<64>, grid, dim3(512), 0, s, q, k, vt, out, seq, seq_pad, heads,
                           kv_heads, scale_log2);
    return hipGetLastError();
}

}  // namespace dit
