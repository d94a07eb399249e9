// Mask-free flash attention forward for gfx950 (bf16 MFMA, fp32 online softmax).
//
// O_h = softmax(Q_h K_g^T / sqrt(hd)) V_g per sequence and query head h, with
// KV head g = h / (H / Hkv) (ERNIE page §VII Decision 2 and §IX "Flash SDPA";
// grouped KV heads as in the zml-flow-rs page §VI attention signature).
//
// Work split: one workgroup = 8 waves = 256 queries of one (batch, head); each
// wave owns 32 queries, two waves share a SIMD.  Keys stream through LDS in
// tiles of 64, the K tile and the transposed V tile each over a ring of 4
// slots, filled by register-free buffer->LDS loads three steps ahead of use.
//
// The scores are computed transposed, S^T = K Q^T (MFMA A = K rows, B = Q rows),
// so an accumulator lane owns one query column and 16 keys: row maxima and
// row sums are in-lane reductions plus one exchange with lane ^ 32.
// P^T is then already the B operand of O^T += V^T P^T provided the 16 keys a
// lane holds per MFMA k-step are the 8 consecutive keys its half of the wave
// feeds to that k-step.  The accumulator puts rows {0-3, 8-11} of each
// 16-row group in lanes 0-31 and {4-7, 12-15} in lanes 32-63, so the K tile is
// loaded with rows 4-7 and 8-11 of every 16-row group swapped: LDS row r holds
// key r with bits 2 and 3 exchanged.  V^T then stays in natural key order and
// every V^T fragment is one 16-byte LDS read.
//
// Three-stage software pipeline per wave: step t runs the QK^T MFMAs of key
// tile t + 2, the PV MFMAs of tile t and the exponentials of tile t + 1, none
// of which waits for another, so the matrix pipe and the VALU of the two waves
// on a SIMD always have independent work; one barrier per step releases the
// ring slots.  Every fragment read is a per-lane base register plus a
// constant offset (the step loop is unrolled over the 4 ring slots), and the
// K loads are bounded by their buffer resource, so a step spends no VALU on
// addresses.
//
// Softmax in log2 units: q is multiplied by log2(e) / sqrt(hd) once, when it
// is loaded, and the QK^T MFMAs of a tile start from the accumulator
// -reference (the query's softmax reference), so they deliver the exponent
// itself and every probability is one v_exp_f32 of an accumulator.  Row sums
// are taken over the bf16 probabilities the PV MFMAs use, by v_dot2 with
// (1, 1); there is no per-tile row max (the reference moves only when a
// tile's probabilities sum past a bound).
//
// Ragged tail (seq not a multiple of 256, e.g. 4096 image + 74 text tokens):
// the last, partial q tile of every (batch, head) would otherwise be a whole
// extra round of workgroups.  With nsplit > 1 that tile's keys are cut into
// nsplit chunks of whole 64-key tiles, one workgroup each; a chunk writes its
// unnormalised O, its softmax reference max and its row sum (fp32) and
// attn_combine merges the chunks: O = sum_c 2^((m_c - M) s) O_c /
// sum_c 2^((m_c - M) s) l_c with M = max_c m_c (the split-KV form of the same
// online softmax).
#include "common.h"

#include <type_traits>
#include "trace.h"

namespace dit {
template <int N> using IC = std::integral_constant<int, N>;

// Tasks [0, n_full) are (q tile, batch * head) pairs over all keys; with
// nsplit > 1 the tasks after them are (chunk, batch * head) pairs of the last
// q tile (index n_full_qt), chunk c covering key tiles [c ct, (c + 1) ct).
template <int HD>
__global__ __launch_bounds__(512, 1)
void flash_attn_kernel(const bf16 *__restrict__ Q, const bf16 *__restrict__ K, const bf16 *__restrict__ Vt,
                       bf16 *__restrict__ O, int S, int S_pad, int H, int Hkv, int n_full_qt, int n_full,
                       float scale_log2, int nsplit, int ct, float *__restrict__ part_o,
                       floatx2 *__restrict__ part_ml) {
#if defined(__HIP_DEVICE_COMPILE__)   // buffer resources exist only in the device pass
    constexpr int NW = 8;                    // waves per workgroup
    constexpr int QW = 32;                   // queries per wave
    constexpr int BQ = NW * QW;              // queries per workgroup
    constexpr int BKV = 64;                  // keys per tile
    constexpr int NS = 4;                    // slots of the K ring and of the V^T ring
    constexpr int KROW = HD * 2;             // bytes per K row
    constexpr int KT_BYTES = BKV * KROW;     // K tile  [64 keys][HD]
    constexpr int VT_BYTES = HD * BKV * 2;   // V^T tile [HD][64 keys]
    constexpr int V_BASE = NS * KT_BYTES;    // the V^T ring follows the K ring
    constexpr int KL = KT_BYTES / (1024 * NW);   // 1 KiB K loads per wave per tile
    constexpr int VL = VT_BYTES / (1024 * NW);   // 1 KiB V^T loads per wave per tile
    constexpr int LOADS = KL + VL;
    constexpr int KK = HD / 16;              // MFMA k-steps over head_dim
    constexpr int DS = HD / 32;              // 32-row blocks of O^T
    static_assert(KL >= 1 && VL >= 1 && KT_BYTES % (1024 * NW) == 0, "tile vs waves");
    // every fragment read is a per-lane base register plus a constant that
    // fits the 16-bit LDS offset field
    static_assert((NS - 1) * KT_BYTES + 32 * KROW < 65536, "K offsets");
    static_assert((NS - 1) * VT_BYTES + (DS - 1) * 32 * 128 < 65536, "V offsets");
    __shared__ __attribute__((aligned(16))) uint8_t smem[NS * (KT_BYTES + VT_BYTES)];

    // LDS layouts (gfx950: 64 banks, 256 B per cycle; a ds_read_b128 serves 16
    // lanes per cycle).
    // K tile: row r of HD*2 bytes; 16-byte chunk c at slot c ^ kswz(r):
    //   HD = 128: 256-byte rows, kswz = r & 15 (16 rows hit 16 distinct slots);
    //   HD = 64: 128-byte rows, two per bank line, kswz = (r >> 1) & 7.
    // V^T tile: row d of 128 bytes (64 keys); chunk c at slot c ^ ((d >> 1) & 7).
    auto kswz = [](int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); };
    auto vswz = [](int d) { return (d >> 1) & 7; };

    // Task order: with a multiple of 8 workgroups, XCD x (workgroups x, x + 8,
    // ...) runs the contiguous task range [x n/8, (x+1) n/8), so the q tiles of
    // one head share that XCD's L2 for K and V.
    // With split chunks, XCD x runs full tasks [x F/8, (x+1) F/8) first, then its
    // eighth of the chunks (workgroups are dispatched in index order per XCD),
    // so every XCD gets the same mix instead of some only long, some only short
    // tasks.
    int task = blockIdx.x;
    const int G = gridDim.x;
    if (G > n_full && (n_full & 7) == 0 && ((G - n_full) & 7) == 0) {
        const int x = task & 7, l = task >> 3, fpx = n_full >> 3, tpx = (G - n_full) >> 3;
        task = l < fpx ? x * fpx + l : n_full + x * tpx + (l - fpx);
    } else if ((G & 7) == 0) {
        task = (task & 7) * (G >> 3) + (task >> 3);
    }
    int qt, bh, t0 = 0, t1 = (S + BKV - 1) / BKV, chunk = -1;   // key tiles [t0, t1)
    if (task < n_full) {
        qt = task % n_full_qt;
        bh = task / n_full_qt;
    } else {
        chunk = (task - n_full) % nsplit;
        bh = (task - n_full) / nsplit;
        qt = n_full_qt;
        t0 = chunk * ct;
        t1 = min(t1, t0 + ct);
    }
    const int h = bh % H, b = bh / H;
    const int g = h / (H / Hkv);
    const bf16 *Qh = Q + (size_t)(b * H + h) * S * HD;
    const bf16 *Kh = K + (size_t)(b * Hkv + g) * S * HD;
    const bf16 *Vh = Vt + (size_t)(b * Hkv + g) * HD * S_pad;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lrow = lane & 31, lhalf = lane >> 5;
    const int q_base = qt * BQ + wave * QW;

    // Q as the B operand: lane -> query q_base + lrow, dims kk*16 + lhalf*8 .. +8
    bf16x8 qf[KK];
    {
        const int qr = min(q_base + lrow, S - 1);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            // q pre-multiplied by log2(e) / sqrt(hd): the scores come out of the
            // MFMA in log2 units, so the exponent needs no multiply (one more
            // bf16 rounding of q, well inside the bf16 path's error)
            const bf16x8 raw = *(const bf16x8 *)(Qh + (size_t)qr * HD + kk * 16 + lhalf * 8);
#pragma unroll
            for (int u = 0; u < 8; ++u) qf[kk][u] = f2bf(bf2f(raw[u]) * scale_log2);
        }
    }

    // Load q of this wave fills 1 KiB at (q * NW + wave) KiB of a K (V^T) tile;
    // lane l lands at +16 l, i.e. in row lin / rowbytes, slot (lin % rowbytes) / 16.
    // K rows are read through a buffer resource based at the tile's first key
    // and bounded at S, so rows past the end read as zeros (their scores are
    // masked); V^T keys in [S, S_pad) are zero in memory.
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh, (uint32_t)HD * (uint32_t)S_pad * 2u);
    uint32_t k_off[KL];       // byte offset within the tile (key bits 2 and 3 swapped, swizzled chunk)
    uint32_t v_off[VL];
#pragma unroll
    for (int q = 0; q < KL; ++q) {
        const int lin = (q * NW + wave) * 1024 + lane * 16;
        const int r = lin / KROW, slot = (lin % KROW) >> 4;
        const int key = (r & ~15) | (((r >> 2) & 1) << 3) | (((r >> 3) & 1) << 2) | (r & 3);
        k_off[q] = (uint32_t)(key * KROW + ((slot ^ kswz(r)) << 4));
    }
#pragma unroll
    for (int q = 0; q < VL; ++q) {
        const int lin = (q * NW + wave) * 1024 + lane * 16;
        const int d = lin >> 7, slot = (lin & 127) >> 4;
        v_off[q] = (uint32_t)d * (uint32_t)S_pad * 2u + (uint32_t)((slot ^ vswz(d)) << 4);
    }
    auto issue_k = [&](int tile, auto SLOT) __attribute__((always_inline)) {
        const int kv0 = tile * BKV;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)kv0 * HD, (uint32_t)(S - kv0) * (uint32_t)KROW);
#pragma unroll
        for (int q = 0; q < KL; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (lds_void *)(smem + decltype(SLOT)::value * KT_BYTES + (q * NW + wave) * 1024), 16, k_off[q], 0,
                0, 0);
    };
    auto issue_v = [&](int tile, auto SLOT) __attribute__((always_inline)) {
        const int kv0 = tile * BKV;
#pragma unroll
        for (int q = 0; q < VL; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (lds_void *)(smem + V_BASE + decltype(SLOT)::value * VT_BYTES + (q * NW + wave) * 1024), 16,
                v_off[q], (uint32_t)kv0 * 2u, 0, 0);
    };

    // per-lane fragment bases: K chunk of k-step kk in row lrow; V^T chunk of
    // key group k2 in row lrow of the V ring
    int kb[KK], vb[4];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) kb[kk] = lrow * KROW + (((kk * 2 + lhalf) ^ kswz(lrow)) << 4);
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) vb[k2] = V_BASE + lrow * 128 + (((k2 * 2 + lhalf) ^ vswz(lrow)) << 4);
    // opaque to the compiler, so the V_BASE part stays in the register and the
    // constant part of every read (slot, row block) goes to the offset field
#pragma unroll
    for (int k2 = 0; k2 < 4; ++k2) asm volatile("" : "+v"(vb[k2]));

    floatx16 zero16;
#pragma unroll
    for (int e = 0; e < 16; ++e) zero16[e] = 0.f;
    floatx16 oacc[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) oacc[ds] = zero16;
    floatx16 sc[2][2];   // S^T of two key tiles (64 keys x 32 queries each), log2 units
    bf16x8 pf[2][4];     // P^T of two key tiles, bf16, as B operands of the PV MFMAs

    // S^T[key, q] = K Q^T of the tile in K slot SLOT, plus the start value c0
    // (in every element of a lane's column the same: minus the query's softmax
    // reference, or zero)
    auto qk = [&](floatx16(&acc)[2], auto SLOT, const floatx16 &c0) __attribute__((always_inline)) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8 kf =
                    *(const bf16x8 *)(smem + kb[kk] + (decltype(SLOT)::value * KT_BYTES + ks * 32 * KROW));
                acc[ks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], kk == 0 ? c0 : acc[ks], 0, 0, 0);
            }
    };
    // O^T[d, q] += V^T[d, keys] P^T[keys, q] of the tile in V slot SLOT
    auto pv = [&](const bf16x8(&p)[4], auto SLOT) __attribute__((always_inline)) {
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2)
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                const bf16x8 vf =
                    *(const bf16x8 *)(smem + vb[k2] + (decltype(SLOT)::value * VT_BYTES + ds * 32 * 128));
                oacc[ds] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p[k2], oacc[ds], 0, 0, 0);
            }
    };
    // keys >= S (the last, partial tile) -> -inf; element e of acc[ks] in lane
    // half h is key kv0 + 32 ks + 16 (e / 8) + 8 h + e % 8
    auto mask = [&](floatx16(&acc)[2], int kv0) __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = kv0 + ks * 32 + ((e >> 3) << 4) + (lhalf << 3) + (e & 7);
                if (key >= S) acc[ks][e] = -INFINITY;
            }
    };

    // Softmax reference of this lane's query, in log2 units: the exponentials,
    // O and l are taken against it; the QK^T MFMAs start from negm = -mref, so
    // they deliver the exponent itself.  It starts at the first tile's max and
    // moves only when a tile's probabilities against it sum to more than
    // 2^kLazy in some lane of the wave (which every probability above 2^kLazy,
    // an overflow included, implies): then it moves up to that tile's max, O
    // and l are rescaled and the tile's probabilities recomputed.  So every
    // probability that reaches O and l is <= 2^kLazy (exact in fp32 and bf16
    // range), with no per-tile max, and O / l is the same softmax for any
    // reference.
    constexpr float kLazyMax = 256.0f;   // 2^kLazy, kLazy = 8
    float mref;
    floatx16 negm;
    // P = 2^S in bf16 (S already relative to the reference); returns this lane's sum of the bf16 values (the
    // very numbers the PV MFMAs multiply), by dot products with (1, 1)
    auto expo = [&](const floatx16(&s)[2], bf16x8(&p)[4]) __attribute__((always_inline)) -> float {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                p[ks * 2 + (e >> 3)][e & 7] = f2bf(__builtin_amdgcn_exp2f(s[ks][e]));
        const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
        float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k2 = 0; k2 < 4; ++k2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bf16x2 pr = {p[k2][2 * i], p[k2][2 * i + 1]};
                a[i] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, a[i], false);
            }
        return (a[0] + a[1]) + (a[2] + a[3]);
    };
    auto tile_max = [&](const floatx16(&s)[2]) __attribute__((always_inline)) {
        float mx = s[0][0];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[ks][e]);
        return fmaxf(mx, __shfl_xor(mx, 32, 64));
    };

    // Pipeline: key tile j has its K in K slot (j - t0) % NS and its V^T in V
    // slot (j - t0) % NS; S^T and P^T of tile j live in buffer (j - t0) % 2.
    // Step t runs, with no dependence among the three, the QK^T MFMAs of tile
    // t + 2, the PV MFMAs of tile t and the exponentials of tile t + 1; it
    // issues the loads of K(t + 5) and V(t + 3) (three steps ahead of use) and
    // ends with tiles K(t + 3), V(t + 1) landed and a barrier.
    // prologue: K(t0 .. t0+2), V(t0) in one group, then K(t0+3), V(t0+1)
    issue_k(t0, IC<0>{});
    issue_k(min(t0 + 1, t1 - 1), IC<1>{});
    issue_k(min(t0 + 2, t1 - 1), IC<2>{});
    issue_v(t0, IC<0>{});
    issue_k(min(t0 + 3, t1 - 1), IC<3>{});
    issue_v(min(t0 + 1, t1 - 1), IC<1>{});
    wait_vmcnt<LOADS>();
    barrier_only();
    qk(sc[0], IC<0>{}, zero16);
    qk(sc[1], IC<1>{}, zero16);
    if ((t0 + 1) * BKV > S) mask(sc[0], t0 * BKV);
    mref = tile_max(sc[0]);
#pragma unroll
    for (int e = 0; e < 16; ++e) negm[e] = -mref;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        sc[0][ks] += negm;
        sc[1][ks] += negm;
    }
    float lsum = expo(sc[0], pf[0]);   // this lane's partial row sum (the other 32 keys live in lane ^ 32)
    barrier_only();                    // K slot 0 (tile t0) is read by every wave before K(t0 + 4) replaces it
    issue_k(min(t0 + 4, t1 - 1), IC<0>{});
    issue_v(min(t0 + 2, t1 - 1), IC<2>{});

    auto step = [&](int t, auto R_) __attribute__((always_inline)) {
        constexpr int R = decltype(R_)::value;   // (t - t0) % NS
        constexpr int CUR = R % 2, NXT = (R + 1) % 2;
        issue_k(min(t + 5, t1 - 1), IC<(R + 1) % NS>{});
        issue_v(min(t + 3, t1 - 1), IC<(R + 3) % NS>{});
        if (t + 1 < t1 && (t + 2) * BKV > S) mask(sc[NXT], (t + 1) * BKV);
        // tiles past t1 - 1 are computed on a repeated tile and never used
        qk(sc[CUR], IC<(R + 2) % NS>{}, negm);
        pv(pf[CUR], IC<R % NS>{});
        float psum = expo(sc[NXT], pf[NXT]);
        // interleave: per MFMA one fragment read and three VALU instructions
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < 4 * KK - 2; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if (t + 1 < t1) {
            if (__any(psum > kLazyMax)) {
                // rare: move the reference up to this tile's max; the scores of
                // this tile and of tile t + 2 were taken against the old one
                const float dcur = fmaxf(tile_max(sc[NXT]), 0.f);
                const float alpha = __builtin_amdgcn_exp2f(-dcur);
#pragma unroll
                for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[ds][e] *= alpha;
                lsum *= alpha;
                mref += dcur;
#pragma unroll
                for (int e = 0; e < 16; ++e) negm[e] = -mref;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        sc[NXT][ks][e] -= dcur;
                        sc[CUR][ks][e] -= dcur;
                    }
                psum = expo(sc[NXT], pf[NXT]);
            }
            lsum += psum;
        }
        // K(t + 3) and V(t + 1) landed (the loads of the last two steps may be in flight)
        wait_vmcnt<2 * LOADS, 0>();
        barrier_only();
    };
    for (int t = t0;;) {
        step(t, IC<0>{});
        if (++t >= t1) break;
        step(t, IC<1>{});
        if (++t >= t1) break;
        step(t, IC<2>{});
        if (++t >= t1) break;
        step(t, IC<3>{});
        if (++t >= t1) break;
    }
    wait_vmcnt<0>();      // retire the trailing (never read) loads before the workgroup's LDS is released

    const float l = lsum + __shfl_xor(lsum, 32, 64);
    const int q = q_base + lrow;
    if (chunk >= 0) {
        // a key chunk of the tail q tile: unnormalised O, reference max and row sum
        if (q < S) {
            const int slot = (bh * nsplit + chunk) * BQ + (q - qt * BQ);
            float *po = part_o + (size_t)slot * HD;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4)
                    *(floatx4 *)(po + ds * 32 + e4 * 8 + lhalf * 4) =
                        floatx4{oacc[ds][e4 * 4], oacc[ds][e4 * 4 + 1], oacc[ds][e4 * 4 + 2], oacc[ds][e4 * 4 + 3]};
            if (lhalf == 0) part_ml[slot] = floatx2{mref, l};
        }
    } else if (q < S) {
        // normalise and store O[b*S + q, h*HD + d] (4 consecutive d per 8-byte store)
        const float inv = 1.0f / l;
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
#endif
}

// Merge the key chunks of the tail q tile: one wave per (batch * head, tail
// query), lane l owning dims l, l + 64 (HD 128) or l (HD 64).
template <int HD>
__global__ __launch_bounds__(256)
void attn_combine_kernel(const float *__restrict__ part_o, const floatx2 *__restrict__ part_ml, bf16 *__restrict__ O,
                         int S, int H, int q0, int n_tail, int n_rows, int nsplit, float scale_log2) {
    constexpr int BQ = 256, PER = HD / 64;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // bh * n_tail + tail query
    if (row >= n_rows) return;
    const int bh = row / n_tail, ql = row - bh * n_tail;
    const int h = bh % H, b = bh / H;
    float M = -INFINITY;
    for (int c = 0; c < nsplit; ++c) M = fmaxf(M, part_ml[(bh * nsplit + c) * BQ + ql][0]);
    float num[PER], den = 0.0f;
#pragma unroll
    for (int u = 0; u < PER; ++u) num[u] = 0.0f;
    for (int c = 0; c < nsplit; ++c) {
        const int slot = (bh * nsplit + c) * BQ + ql;
        const floatx2 ml = part_ml[slot];
        const float w = __builtin_amdgcn_exp2f((ml[0] - M) * scale_log2);
        den += w * ml[1];
#pragma unroll
        for (int u = 0; u < PER; ++u) num[u] += w * part_o[(size_t)slot * HD + u * 64 + lane];
    }
    const float inv = 1.0f / den;
    bf16 *orow = O + ((size_t)b * S + q0 + ql) * (size_t)(H * HD) + (size_t)h * HD;
#pragma unroll
    for (int u = 0; u < PER; ++u) orow[u * 64 + lane] = f2bf(num[u] * inv);
}

// Compute units of the current device (cached; 256 when it cannot be read).
int device_cu_count() {
    static int n = 0;
    if (n == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            n = v;
        else
            n = 256;
    }
    return n;
}

int attention_split_count(int batch, int seq, int heads, int cus) {
    // a tail exists and its (batch, head) tasks leave most CUs idle: spread
    // them over the CUs, at least 2 key tiles per chunk, at most 16 chunks
    if (seq % 256 == 0) return 1;
    const int nt = (seq + 63) / 64, tails = batch * heads;
    int n = cus / tails;
    n = n < 16 ? n : 16;
    n = n < nt / 2 ? n : nt / 2;
    return n > 1 ? n : 1;
}

size_t attention_split_bytes(int batch, int heads, int head_dim, int nsplit) {
    if (nsplit <= 1) return 0;
    const size_t slots = (size_t)batch * heads * nsplit * 256;
    return slots * head_dim * 4 + slots * 8;
}

hipError_t launch_flash_attention(const bf16 *q, const bf16 *k, const bf16 *vt, bf16 *out, int batch, int seq,
                                  int seq_pad, int heads, int kv_heads, int head_dim, int nsplit, void *part,
                                  hipStream_t s) {
    TraceScope trace_(s, "flash_attention");
    if (trace_.on()) trace_.args("B=%d S=%d H=%d Hkv=%d hd=%d nsplit=%d", batch, seq, heads, kv_heads, head_dim, nsplit);
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)head_dim);
    const int nt = (seq + 63) / 64;
    int n_full_qt = (seq + 255) / 256, ct = nt;
    float *part_o = nullptr;
    floatx2 *part_ml = nullptr;
    if (nsplit > 1 && seq % 256 != 0 && part != nullptr) {
        n_full_qt = seq / 256;
        ct = (nt + nsplit - 1) / nsplit;
        nsplit = (nt + ct - 1) / ct;   // every chunk non-empty
        part_o = (float *)part;
        part_ml = (floatx2 *)(part_o + (size_t)batch * heads * nsplit * 256 * head_dim);
    } else {
        nsplit = 1;
    }
    const int n_full = n_full_qt * heads * batch;
    const int tail_tasks = part_o ? nsplit * heads * batch : 0;
    const dim3 grid((unsigned)(n_full + tail_tasks));
#define DIT_ATT_LAUNCH(HD_)                                                                                   \
    hipLaunchKernelGGL(flash_attn_kernel<HD_>, grid, dim3(512), 0, s, q, k, vt, out, seq, seq_pad, heads,     \
                       kv_heads, n_full_qt, n_full, scale_log2, nsplit, ct, part_o, part_ml)
    if (head_dim == 128)
        DIT_ATT_LAUNCH(128);
    else
        DIT_ATT_LAUNCH(64);
#undef DIT_ATT_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !part_o) return e;
    const int q0 = n_full_qt * 256, n_tail = seq - q0, n_rows = batch * heads * n_tail;
    const dim3 cgrid((unsigned)((n_rows + 3) / 4));
    if (head_dim == 128)
        hipLaunchKernelGGL(attn_combine_kernel<128>, cgrid, dim3(256), 0, s, part_o, part_ml, out, seq, heads, q0,
                           n_tail, n_rows, nsplit, 1.0f);
    else
        hipLaunchKernelGGL(attn_combine_kernel<64>, cgrid, dim3(256), 0, s, part_o, part_ml, out, seq, heads, q0,
                           n_tail, n_rows, nsplit, 1.0f);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 attention (the fp32 parity path): the same softmax(Q K^T / sqrt(hd)) V
// with fp32 operands on the vector ALUs.  One workgroup = 64 queries of one
// (batch, head); 4 lanes per query, each holding HD/4 consecutive dims of q
// (pre-scaled by log2(e) / sqrt(hd)) and of the output.  A 64-key tile of K
// and of V (read from V^T and transposed on the way into LDS) is staged per
// step; the scores of the tile are partial dots reduced over the 4 lanes of a
// query, followed by one online-softmax update of (m, l, o).
// ---------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256)
void attn_f32_kernel(const float *__restrict__ Q, const float *__restrict__ K, const float *__restrict__ Vt,
                     float *__restrict__ O, int S, int S_pad, int H, int Hkv, float scale_log2) {
    constexpr int BKV = 64, DL = HD / 4, LD = HD + 4;
    __shared__ float Ks[BKV * LD];
    __shared__ float Vs[BKV * LD];
    const int qt = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (H / Hkv);
    const int tid = threadIdx.x, ql = tid >> 2, sub = tid & 3;
    const int q = qt * 64 + ql;
    const float *Qh = Q + (size_t)(b * H + h) * S * HD;
    const float *Kh = K + (size_t)(b * Hkv + g) * S * HD;
    const float *Vh = Vt + (size_t)(b * Hkv + g) * HD * S_pad;
    float qr[DL], o[DL];
    {
        const float *qp = Qh + (size_t)min(q, S - 1) * HD + sub * DL;
#pragma unroll
        for (int i = 0; i < DL; i += 4) {
            const floatx4 v = *(const floatx4 *)(qp + i);
#pragma unroll
            for (int u = 0; u < 4; ++u) { qr[i + u] = v[u] * scale_log2; o[i + u] = 0.f; }
        }
    }
    float m = -INFINITY, l = 0.f;
    const int nt = (S + BKV - 1) / BKV;
    for (int t = 0; t < nt; ++t) {
        const int k0 = t * BKV;
        __syncthreads();   // the previous tile's reads are done
        // K rows k0 .. k0 + 63 (rows past S clamped; their scores are masked)
#pragma unroll
        for (int it = 0; it < HD / 16; ++it) {
            const int c = it * 256 + tid, r = c / (HD / 4), d4 = c - r * (HD / 4);
            const floatx4 v = *(const floatx4 *)(Kh + (size_t)min(k0 + r, S - 1) * HD + d4 * 4);
            *(floatx4 *)(Ks + r * LD + d4 * 4) = v;
        }
        // V^T columns k0 .. k0 + 63 (inside the padded row: S_pad is a multiple of 64)
#pragma unroll
        for (int it = 0; it < HD / 16; ++it) {
            const int c = it * 256 + tid, d = c / 16, j4 = c - d * 16;
            const floatx4 v = *(const floatx4 *)(Vh + (size_t)d * S_pad + k0 + j4 * 4);
#pragma unroll
            for (int u = 0; u < 4; ++u) Vs[(j4 * 4 + u) * LD + d] = v[u];
        }
        __syncthreads();
        float sc[BKV];
        float mt = m;
#pragma unroll
        for (int j = 0; j < BKV; ++j) {
            const float *kr = Ks + j * LD + sub * DL;
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < DL; i += 4) {
                const floatx4 kv = *(const floatx4 *)(kr + i);
#pragma unroll
                for (int u = 0; u < 4; ++u) acc += qr[i + u] * kv[u];
            }
            acc += __shfl_xor(acc, 1, 64);
            acc += __shfl_xor(acc, 2, 64);
            sc[j] = k0 + j < S ? acc : -INFINITY;
            mt = fmaxf(mt, sc[j]);
        }
        const float alpha = exp2f(m - mt);
        m = mt;
        l *= alpha;
#pragma unroll
        for (int i = 0; i < DL; ++i) o[i] *= alpha;
#pragma unroll
        for (int j = 0; j < BKV; ++j) {
            const float p = exp2f(sc[j] - mt);
            l += p;
            const float *vr = Vs + j * LD + sub * DL;
#pragma unroll
            for (int i = 0; i < DL; i += 4) {
                const floatx4 vv = *(const floatx4 *)(vr + i);
#pragma unroll
                for (int u = 0; u < 4; ++u) o[i + u] += p * vv[u];
            }
        }
    }
    if (q < S) {
        const float inv = 1.0f / l;
        float *orow = O + ((size_t)b * S + q) * (size_t)(H * HD) + (size_t)h * HD + sub * DL;
#pragma unroll
        for (int i = 0; i < DL; i += 4)
            *(floatx4 *)(orow + i) = floatx4{o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv};
    }
}

hipError_t launch_flash_attention_f32(const float *q, const float *k, const float *vt, float *out, int batch,
                                      int seq, int seq_pad, int heads, int kv_heads, int head_dim, hipStream_t s) {
    TraceScope trace_(s, "attn_f32");
    if (trace_.on()) trace_.args("B=%d S=%d H=%d Hkv=%d hd=%d", batch, seq, heads, kv_heads, head_dim);
    if (seq_pad % 64 || seq_pad < seq) return hipErrorInvalidValue;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)head_dim);
    const dim3 grid((unsigned)((seq + 63) / 64), (unsigned)heads, (unsigned)batch);
    if (head_dim == 128)
        hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(256), 0, s, q, k, vt, out, seq, seq_pad, heads, kv_heads,
                           scale_log2);
    else if (head_dim == 64)
        hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(256), 0, s, q, k, vt, out, seq, seq_pad, heads, kv_heads,
                           scale_log2);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace dit
