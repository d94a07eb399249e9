// C ABI of libdit.so: argument validation, workspace layout and the
// composition of the block / stack / loop entry points out of the kernels.
#include "dit.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "common.h"

using namespace dit;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return DIT_OK;
}

#define DIT_TRY_HIP(expr)                                                                  \
    do {                                                                                   \
        hipError_t e_ = (expr);                                                            \
        if (e_ != hipSuccess) return fail(DIT_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

#define DIT_TRY(expr)             \
    do {                          \
        int rc_ = (expr);         \
        if (rc_ != DIT_OK) return rc_; \
    } while (0)

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3) == 0; }

int device_check() {
    static int status = 1;
    static std::once_flag once;
    std::call_once(once, [] {
        int n = 0;
        status = (hipGetDeviceCount(&n) == hipSuccess && n > 0) ? DIT_OK : DIT_ERR_NO_DEVICE;
    });
    if (status != DIT_OK) return fail(DIT_ERR_NO_DEVICE, "no HIP device is visible to this process");
    return DIT_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int32_t seq_pad_of(int32_t s) { return (s + 63) / 64 * 64; }

// Workspace of one block evaluation.  On the fp32 path (fp32 weights) the
// intermediates h, q, k, vt, att and u are fp32.  In the W8A8 format h holds the int8
// codes of the normed rows (hs their scales), and the attention output and the
// GLU output get int8 copies (aq/as, uq/us) for the projections that read them.
// With a ragged sequence (seq % 256 != 0) it also holds the attention's
// split-KV partials of the last q tile (up to 16 key chunks).
struct BlockWs {
    size_t m, h, q, k, vt, att, x1, u, hs, aq, as, uq, us, part, total;
};

constexpr int kMaxAttnSplit = 16;

BlockWs block_ws(const dit_block_desc &d) {
    const size_t N = (size_t)d.batch * d.seq, D = d.hidden, B = d.batch;
    const size_t hd = d.head_dim, H = d.heads, Hk = d.kv_heads, F = d.ffn;
    const size_t es = d.w_dtype == DIT_F32 ? 4 : 2;   // bytes per intermediate element
    BlockWs L{};
    size_t off = 0;
    L.m = off;   off += align256(6 * D * 4);
    L.h = off;   off += align256(N * D * es);
    L.q = off;   off += align256(B * H * d.seq * hd * es);
    L.k = off;   off += align256(B * Hk * d.seq * hd * es);
    L.vt = off;  off += align256(B * Hk * hd * (size_t)seq_pad_of(d.seq) * es);
    L.att = off; off += align256(N * H * hd * es);
    L.x1 = off;  off += align256(N * D * 4);
    L.u = off;   off += align256(N * F * es);
    if (d.seq % 256 && d.w_dtype != DIT_F32) {
        L.part = off; off += align256(attention_split_bytes(d.batch, d.heads, d.head_dim, kMaxAttnSplit));
    }
    if (d.fmt == DIT_FMT_W8A8_H256) {
        L.hs = off; off += align256(N * 4);
        L.aq = off; off += align256(N * H * hd);
        L.as = off; off += align256(N * 4);
        L.uq = off; off += align256(N * F);
        L.us = off; off += align256(N * 4);
    }
    L.total = off;
    return L;
}

int check_desc(const dit_block_desc *d) {
    if (!d) return fail(DIT_ERR_INVALID_ARG, "desc is NULL");
    if (d->batch <= 0 || d->seq <= 0 || d->hidden <= 0 || d->heads <= 0 || d->kv_heads <= 0 ||
        d->head_dim <= 0 || d->ffn <= 0 || d->cond_dim < 0)
        return fail(DIT_ERR_INVALID_ARG, "dimensions must be positive (cond_dim >= 0)");
    // products in 64 bits: any of the fields may be near INT32_MAX here
    if ((int64_t)d->heads * d->head_dim != d->hidden)
        return fail(DIT_ERR_INVALID_ARG, "heads * head_dim (%lld) != hidden (%d)",
                    (long long)d->heads * d->head_dim, d->hidden);
    if (d->heads % d->kv_heads != 0)
        return fail(DIT_ERR_INVALID_ARG, "heads (%d) not a multiple of kv_heads (%d)", d->heads, d->kv_heads);
    if (!(d->eps > 0.f) || !isfinite(d->eps)) return fail(DIT_ERR_INVALID_ARG, "eps must be positive and finite");
    if (d->x_dtype != DIT_F32 && d->x_dtype != DIT_BF16) return fail(DIT_ERR_INVALID_ARG, "bad x_dtype");
    if (d->rope != DIT_ROPE_INTERLEAVED && d->rope != DIT_ROPE_HALF) return fail(DIT_ERR_INVALID_ARG, "bad rope layout");
    if (d->norm != DIT_LAYERNORM && d->norm != DIT_RMSNORM) return fail(DIT_ERR_INVALID_ARG, "bad norm kind");
    if (d->act != DIT_ACT_SILU && d->act != DIT_ACT_GELU_TANH) return fail(DIT_ERR_INVALID_ARG, "bad act");
    if (d->gate < DIT_GATE_IDENTITY || d->gate > DIT_GATE_SIGMOID) return fail(DIT_ERR_INVALID_ARG, "bad gate function");
    if (d->mod != DIT_MOD_SHIFT_SCALE_GATE && d->mod != DIT_MOD_SCALE_GATE) return fail(DIT_ERR_INVALID_ARG, "bad mod");
    if (d->qk_order != DIT_QK_NORM_ROPE && d->qk_order != DIT_QK_ROPE_NORM) return fail(DIT_ERR_INVALID_ARG, "bad qk_order");
    if (d->fmt != DIT_FMT_BF16 && d->fmt != DIT_FMT_W8A8_H256) return fail(DIT_ERR_INVALID_ARG, "bad fmt");
    if (d->w_dtype != DIT_BF16 && d->w_dtype != DIT_F32) return fail(DIT_ERR_INVALID_ARG, "bad w_dtype");
    if (d->w_dtype == DIT_F32 && (d->x_dtype != DIT_F32 || d->fmt != DIT_FMT_BF16))
        return fail(DIT_ERR_UNSUPPORTED, "fp32 weights (the fp32 path) need x_dtype F32 and fmt BF16");
    if (d->head_dim != 64 && d->head_dim != 128) return fail(DIT_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    if (d->hidden % 256) return fail(DIT_ERR_UNSUPPORTED, "hidden must be a multiple of 256");
    if (d->hidden > 8192) return fail(DIT_ERR_UNSUPPORTED, "hidden must be <= 8192");
    if (d->ffn % 128) return fail(DIT_ERR_UNSUPPORTED, "ffn must be a multiple of 128");
    if ((((int64_t)d->heads + 2 * (int64_t)d->kv_heads) * d->head_dim) % 256)
        return fail(DIT_ERR_UNSUPPORTED, "(heads + 2 kv_heads) * head_dim must be a multiple of 256");
    if (d->cond_dim % 8) return fail(DIT_ERR_UNSUPPORTED, "cond_dim must be a multiple of 8");
    if (d->fmt == DIT_FMT_W8A8_H256 && (d->ffn % 256 || !quantize_h256_supported(d->ffn)))
        return fail(DIT_ERR_UNSUPPORTED, "W8A8 H256 needs ffn a multiple of 256 with ceil(ffn / 1024) <= 7 or a multiple of 4 up to 32");
    // The kernels address each operand through a buffer resource whose size
    // and offsets are 32-bit byte counts: every GEMM operand and intermediate
    // must stay below 2^32 bytes, i.e. 2^31 bf16 elements or 2^30 fp32 ones.
    const double n = (double)d->batch * d->seq;
    const double lim = d->w_dtype == DIT_F32 ? 1073741824.0 : 2147483648.0;
    const double qkv = (double)(d->heads + 2 * d->kv_heads) * d->head_dim;
    if (n * d->ffn >= lim || n * d->hidden >= lim || (double)d->ffn * 2 * d->hidden >= lim ||
        qkv * d->hidden >= lim || n * qkv >= lim)
        return fail(DIT_ERR_UNSUPPORTED, "a GEMM operand exceeds 2^32 bytes (2^31 bf16 or 2^30 fp32 elements)");
    return DIT_OK;
}

int check_weights(const dit_block_desc &d, const dit_block_weights *w) {
    if (!w) return fail(DIT_ERR_INVALID_ARG, "weights is NULL");
    if (!w->w_qkv || !w->w_o || !w->w_gate_up || !w->w_down)
        return fail(DIT_ERR_INVALID_ARG, "w_qkv, w_o, w_gate_up and w_down are required");
    if (!aligned16(w->w_qkv) || !aligned16(w->w_o) || !aligned16(w->w_gate_up) || !aligned16(w->w_down))
        return fail(DIT_ERR_ALIGNMENT, "weight matrices must be 16-byte aligned");
    if (d.cond_dim > 0) {
        if (!w->w_ada || !w->b_ada) return fail(DIT_ERR_INVALID_ARG, "AdaLN mode needs w_ada and b_ada");
        if (!aligned16(w->w_ada) || !aligned16(w->b_ada)) return fail(DIT_ERR_ALIGNMENT, "w_ada/b_ada must be 16-byte aligned");
        if (w->ln1_g || w->ln1_b || w->ln2_g || w->ln2_b)
            return fail(DIT_ERR_UNSUPPORTED, "LayerNorm affine is not used in AdaLN mode; pass NULL");
    } else {
        const float *v[4] = {w->ln1_g, w->ln1_b, w->ln2_g, w->ln2_b};
        for (const float *p : v)
            if (p && !aligned16(p)) return fail(DIT_ERR_ALIGNMENT, "LayerNorm gamma/beta must be 16-byte aligned");
    }
    if (d.fmt == DIT_FMT_W8A8_H256) {
        if (!w->s_qkv || !w->s_o || !w->s_gate_up || !w->s_down)
            return fail(DIT_ERR_INVALID_ARG, "the W8A8 format needs the weight scales s_qkv, s_o, s_gate_up, s_down");
        if (!aligned16(w->s_qkv) || !aligned16(w->s_o) || !aligned16(w->s_gate_up) || !aligned16(w->s_down))
            return fail(DIT_ERR_ALIGNMENT, "weight scales must be 16-byte aligned");
    }
    if (d.qk_norm) {
        if (!w->q_g || !w->q_b || !w->k_g || !w->k_b) return fail(DIT_ERR_INVALID_ARG, "qk_norm needs q_g, q_b, k_g, k_b");
        if (!aligned4(w->q_g) || !aligned4(w->q_b) || !aligned4(w->k_g) || !aligned4(w->k_b))
            return fail(DIT_ERR_ALIGNMENT, "qk-norm vectors must be 4-byte aligned");
    }
    return DIT_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

hipStream_t as_stream(void *s) { return (hipStream_t)s; }

// Rows of the AdaLN linear: 6 or 4 chunks of hidden.
int ada_rows(const dit_block_desc &d) { return (d.mod == DIT_MOD_SCALE_GATE ? 4 : 6) * d.hidden; }

// The block body after the modulation vector m (or NULL without AdaLN) is ready.
int block_body(const dit_block_desc &d, const dit_block_weights &w, const void *x, int x_f32, const float *m,
               const float *cosT, const float *sinT, void *out, int out_f32, uint8_t *ws, const BlockWs &L,
               hipStream_t s) {
    const int64_t N = (int64_t)d.batch * d.seq;
    const int D = d.hidden, hd = d.head_dim, F = d.ffn;
    const int qkv_dim = (d.heads + 2 * d.kv_heads) * hd;
    const int spad = seq_pad_of(d.seq);
    bf16 *h = (bf16 *)(ws + L.h);
    bf16 *q = (bf16 *)(ws + L.q), *k = (bf16 *)(ws + L.k), *vt = (bf16 *)(ws + L.vt);
    bf16 *att = (bf16 *)(ws + L.att);
    float *x1 = (float *)(ws + L.x1);
    bf16 *u = (bf16 *)(ws + L.u);
    const int mode = m ? 0 : 1;
    const int rms = d.norm == DIT_RMSNORM;
    // split-KV for the partial last q tile when the sequence is ragged
    void *part = d.seq % 256 ? (void *)(ws + L.part) : nullptr;
    int nsplit = attention_split_count(d.batch, d.seq, d.heads, device_cu_count());
    nsplit = nsplit < kMaxAttnSplit ? nsplit : kMaxAttnSplit;
    // modulation chunks: (shift1, scale1, gate1, shift2, scale2, gate2) or, without
    // shift, (scale1, gate1, scale2, gate2); without AdaLN the affine LN parameters
    const float *shift1, *scale1, *gate1, *shift2, *scale2, *gate2;
    if (!m) {
        shift1 = w.ln1_b; scale1 = w.ln1_g; shift2 = w.ln2_b; scale2 = w.ln2_g; gate1 = gate2 = nullptr;
    } else if (d.mod == DIT_MOD_SCALE_GATE) {
        shift1 = shift2 = nullptr; scale1 = m; gate1 = m + D; scale2 = m + 2 * D; gate2 = m + 3 * D;
    } else {
        shift1 = m; scale1 = m + D; gate1 = m + 2 * D; shift2 = m + 3 * D; scale2 = m + 4 * D; gate2 = m + 5 * D;
    }

    QkvEpiArgs e{d.batch, d.seq, spad, d.heads, d.kv_heads, hd, d.qk_norm, d.rope == DIT_ROPE_HALF, rms,
                 d.qk_order == DIT_QK_ROPE_NORM, d.eps, w.q_g, w.q_b, w.k_g, w.k_b, cosT, sinT, q, k, vt};
    if (d.w_dtype == DIT_F32) {
        // the fp32 path: every operand and intermediate fp32 (fp32 MFMA GEMMs,
        // fp32 attention); x and out are the fp32 residual stream
        float *hf = (float *)(ws + L.h), *uf = (float *)(ws + L.u), *af = (float *)(ws + L.att);
        float *qf = (float *)(ws + L.q), *kf = (float *)(ws + L.k), *vf = (float *)(ws + L.vt);
        DIT_TRY_HIP(launch_ln_modulate_f32((const float *)x, N, D, rms, shift1, scale1, mode, d.eps, hf, s));
        DIT_TRY_HIP(launch_vt_pad_zero(vf, 1, d.batch * d.kv_heads * hd, d.seq, spad, s));
        DIT_TRY_HIP(launch_gemm_qkv_f32(hf, (const float *)w.w_qkv, N, qkv_dim, D, e, s));
        DIT_TRY_HIP(launch_flash_attention_f32(qf, kf, vf, af, d.batch, d.seq, spad, d.heads, d.kv_heads, hd, s));
        DIT_TRY_HIP(launch_gemm_residual_f32(af, (const float *)w.w_o, N, D, d.heads * hd, (const float *)x, gate1,
                                             d.gate, nullptr, x1, s));
        DIT_TRY_HIP(launch_ln_modulate_f32(x1, N, D, rms, shift2, scale2, mode, d.eps, hf, s));
        DIT_TRY_HIP(launch_gemm_swiglu_f32(hf, (const float *)w.w_gate_up, N, F, D, d.act, uf, s));
        DIT_TRY_HIP(launch_gemm_residual_f32(uf, (const float *)w.w_down, N, D, F, x1, gate2, d.gate, nullptr,
                                             (float *)out, s));
        return DIT_OK;
    }
    if (d.fmt == DIT_FMT_W8A8_H256) {
        // the four projections in int8 (zml-flow-rs page §VII W8A8 with H256 on
        // both sides); norms, attention and the residual stream as in bf16
        int8_t *hq = (int8_t *)(ws + L.h), *aq = (int8_t *)(ws + L.aq), *uq = (int8_t *)(ws + L.uq);
        float *hs = (float *)(ws + L.hs), *as = (float *)(ws + L.as), *us = (float *)(ws + L.us);
        DIT_TRY_HIP(launch_ln_modulate_q8(x, x_f32, N, D, rms, shift1, scale1, mode, d.eps, hq, hs, s));
        DIT_TRY_HIP(launch_vt_pad_zero(vt, 0, d.batch * d.kv_heads * hd, d.seq, spad, s));
        DIT_TRY_HIP(launch_gemm_qkv_q8(hq, hs, (const int8_t *)w.w_qkv, w.s_qkv, N, qkv_dim, D, e, s));
        DIT_TRY_HIP(launch_flash_attention(q, k, vt, att, d.batch, d.seq, spad, d.heads, d.kv_heads, hd, nsplit,
                                           part, s));
        DIT_TRY_HIP(launch_quantize_h256(att, 0, N, d.heads * hd, aq, as, s));
        DIT_TRY_HIP(launch_gemm_residual_q8(aq, as, (const int8_t *)w.w_o, w.s_o, N, D, d.heads * hd, x, x_f32, gate1,
                                            d.gate, nullptr, x1, 1, s));
        DIT_TRY_HIP(launch_ln_modulate_q8(x1, 1, N, D, rms, shift2, scale2, mode, d.eps, hq, hs, s));
        DIT_TRY_HIP(launch_gemm_swiglu_q8(hq, hs, (const int8_t *)w.w_gate_up, w.s_gate_up, N, F, D, d.act, u, s));
        DIT_TRY_HIP(launch_quantize_h256(u, 0, N, F, uq, us, s));
        DIT_TRY_HIP(launch_gemm_residual_q8(uq, us, (const int8_t *)w.w_down, w.s_down, N, D, F, x1, 1, gate2, d.gate,
                                            nullptr, out, out_f32, s));
        return DIT_OK;
    }
    DIT_TRY_HIP(launch_ln_modulate(x, x_f32, N, D, rms, shift1, scale1, mode, d.eps, h, s));
    DIT_TRY_HIP(launch_vt_pad_zero(vt, 0, d.batch * d.kv_heads * hd, d.seq, spad, s));
    DIT_TRY_HIP(launch_gemm_qkv(h, (const bf16 *)w.w_qkv, N, qkv_dim, D, e, s));
    DIT_TRY_HIP(launch_flash_attention(q, k, vt, att, d.batch, d.seq, spad, d.heads, d.kv_heads, hd, nsplit, part,
                                       s));
    DIT_TRY_HIP(launch_gemm_residual(att, (const bf16 *)w.w_o, N, D, d.heads * hd, x, x_f32, gate1, d.gate,
                                     nullptr, x1, 1, s));
    DIT_TRY_HIP(launch_ln_modulate(x1, 1, N, D, rms, shift2, scale2, mode, d.eps, h, s));
    DIT_TRY_HIP(launch_gemm_swiglu(h, (const bf16 *)w.w_gate_up, N, F, D, d.act, u, s));
    DIT_TRY_HIP(launch_gemm_residual(u, (const bf16 *)w.w_down, N, D, F, x1, 1, gate2, d.gate, nullptr,
                                     out, out_f32, s));
    return DIT_OK;
}

// Stack workspace: the block workspace followed by the fp32 residual stream,
// the final modulation and the bf16 copy of the latent.
struct StackWs {
    BlockWs blk;
    size_t x, fm, lat, total;
};

StackWs stack_ws(const dit_model &mdl) {
    StackWs L{};
    L.blk = block_ws(mdl.blk);
    const size_t N = (size_t)mdl.blk.batch * mdl.blk.seq, D = mdl.blk.hidden;
    size_t off = L.blk.total;
    L.x = off;   off += align256(N * D * 4);
    L.fm = off;  off += align256(2 * D * 4);
    L.lat = off; off += align256(N * (size_t)mdl.latent_dim * 2);
    L.total = off;
    return L;
}

int check_model(const dit_model *mdl) {
    if (!mdl) return fail(DIT_ERR_INVALID_ARG, "model is NULL");
    DIT_TRY(check_desc(&mdl->blk));
    if (mdl->layers <= 0 || !mdl->blocks) return fail(DIT_ERR_INVALID_ARG, "layers must be > 0 and blocks non-NULL");
    if (mdl->blk.cond_dim <= 0) return fail(DIT_ERR_INVALID_ARG, "the stack needs a conditioning vector (cond_dim > 0)");
    if (mdl->blk.x_dtype != DIT_F32) return fail(DIT_ERR_UNSUPPORTED, "the stack keeps an fp32 residual stream (x_dtype F32)");
    if (mdl->latent_dim <= 0 || mdl->latent_dim % 128) return fail(DIT_ERR_UNSUPPORTED, "latent_dim must be a multiple of 128");
    if (!mdl->w_in || !mdl->b_in || !mdl->w_fmod || !mdl->b_fmod || !mdl->w_out || !mdl->b_out)
        return fail(DIT_ERR_INVALID_ARG, "stack edge weights are required");
    if (!aligned16(mdl->w_in) || !aligned16(mdl->w_fmod) || !aligned16(mdl->w_out) || !aligned16(mdl->b_in) ||
        !aligned16(mdl->b_fmod) || !aligned16(mdl->b_out))
        return fail(DIT_ERR_ALIGNMENT, "stack edge weights must be 16-byte aligned");
    for (int l = 0; l < mdl->layers; ++l) DIT_TRY(check_weights(mdl->blk, &mdl->blocks[l]));
    return DIT_OK;
}

}  // namespace

extern "C" {

const char *dit_version(void) { return "dit-gfx950 0.1"; }

const char *dit_last_error(void) { return g_err.c_str(); }

const char *dit_status_string(int st) {
    switch (st) {
        case DIT_OK: return "ok";
        case DIT_ERR_INVALID_ARG: return "invalid argument";
        case DIT_ERR_UNSUPPORTED: return "unsupported shape or option";
        case DIT_ERR_WORKSPACE: return "workspace too small";
        case DIT_ERR_ALIGNMENT: return "misaligned pointer";
        case DIT_ERR_NO_DEVICE: return "no HIP device";
        case DIT_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int32_t dit_seq_pad(int32_t seq) { return seq_pad_of(seq); }

int dit_block_workspace_size(const dit_block_desc *desc, size_t *bytes) {
    DIT_TRY(check_desc(desc));
    if (!bytes) return fail(DIT_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = block_ws(*desc).total;
    return ok();
}

}  // extern "C"

namespace {

// Validation shared by the block entry points (everything but the workspace).
int check_block_call(const dit_block_desc *desc, const dit_block_weights *w, const void *x, const float *cond,
                     const float *rope_cos, const float *rope_sin, const void *out) {
    DIT_TRY(check_desc(desc));
    const dit_block_desc &d = *desc;
    DIT_TRY(check_weights(d, w));
    if (!x || !out || !rope_cos || !rope_sin) return fail(DIT_ERR_INVALID_ARG, "x, out and rope tables are required");
    if ((d.cond_dim > 0) != (cond != nullptr)) return fail(DIT_ERR_INVALID_ARG, "cond must be given iff cond_dim > 0");
    if (!aligned16(x) || !aligned16(out) || !aligned4(rope_cos) || !aligned4(rope_sin) || (cond && !aligned16(cond)))
        return fail(DIT_ERR_ALIGNMENT, "x, out, cond must be 16-byte aligned (rope tables 4-byte)");
    const size_t xbytes = (size_t)d.batch * d.seq * d.hidden * (d.x_dtype == DIT_F32 ? 4 : 2);
    if (out != x && overlaps(out, xbytes, x, xbytes)) return fail(DIT_ERR_INVALID_ARG, "out overlaps x without being equal to it");
    return DIT_OK;
}

int check_ws_apart(const dit_block_desc &d, const void *ws, const void *x, const void *out) {
    const size_t total = block_ws(d).total;
    const size_t xbytes = (size_t)d.batch * d.seq * d.hidden * (d.x_dtype == DIT_F32 ? 4 : 2);
    if (overlaps(ws, total, x, xbytes) || overlaps(ws, total, out, xbytes))
        return fail(DIT_ERR_INVALID_ARG, "workspace overlaps x or out");
    return DIT_OK;
}

// The block on a validated call with a workspace of at least block_ws(d).total bytes.
int run_block(const dit_block_desc &d, const dit_block_weights *w, const void *x, const float *cond,
              const float *rope_cos, const float *rope_sin, void *out, void *ws, hipStream_t s) {
    const BlockWs L = block_ws(d);
    uint8_t *wsb = (uint8_t *)ws;
    float *m = nullptr;
    if (d.cond_dim > 0) {
        m = (float *)(wsb + L.m);
        DIT_TRY_HIP(launch_adaln_gemv(w->w_ada, d.w_dtype == DIT_F32, w->b_ada, cond, ada_rows(d), d.cond_dim, 1, m,
                                      s));
    }
    const int xf = d.x_dtype == DIT_F32;
    DIT_TRY(block_body(d, *w, x, xf, m, rope_cos, rope_sin, out, xf, wsb, L, s));
    return ok();
}

// Scratch of the allocation-free block entry point: the block workspace in a
// device array of the library, one copy per GPU (from the library's load on
// that GPU until the process ends).  In host code `scratch` names a host-side
// stand-in: its device address, per GPU, comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's scratch, looked up once per GPU.
int scratch_of_current_device(void **ptr) {
    int dev = -1;
    DIT_TRY_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(DIT_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        DIT_TRY_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        if (!p) return fail(DIT_ERR_HIP, "hipGetSymbolAddress returned NULL for the scratch array");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return DIT_OK;
}

}  // namespace

extern "C" {

int dit_block_forward(const dit_block_desc *desc, const dit_block_weights *w, const void *x, const float *cond,
                      const float *rope_cos, const float *rope_sin, void *out, void *ws, size_t ws_bytes,
                      void *stream) {
    DIT_TRY(check_block_call(desc, w, x, cond, rope_cos, rope_sin, out));
    if (!ws) return fail(DIT_ERR_INVALID_ARG, "ws is required");
    if (!aligned16(ws)) return fail(DIT_ERR_ALIGNMENT, "ws must be 16-byte aligned");
    const size_t need = block_ws(*desc).total;
    if (ws_bytes < need) return fail(DIT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, need);
    DIT_TRY(check_ws_apart(*desc, ws, x, out));
    DIT_TRY(device_check());
    return run_block(*desc, w, x, cond, rope_cos, rope_sin, out, ws, as_stream(stream));
}

size_t dit_block_forward_noalloc_max_bytes(void) { return kScratchBytes; }

int dit_block_forward_noalloc(const dit_block_desc *desc, const dit_block_weights *w, const void *x,
                              const float *cond, const float *rope_cos, const float *rope_sin, void *out,
                              void *stream) {
    DIT_TRY(check_block_call(desc, w, x, cond, rope_cos, rope_sin, out));
    const size_t need = block_ws(*desc).total;
    if (need > kScratchBytes)
        return fail(DIT_ERR_WORKSPACE, "this block needs %zu bytes of workspace; the allocation-free entry point "
                                       "holds %zu (use dit_block_forward with a caller workspace)", need, kScratchBytes);
    DIT_TRY(device_check());
    void *ws = nullptr;
    DIT_TRY(scratch_of_current_device(&ws));
    DIT_TRY(check_ws_apart(*desc, ws, x, out));
    return run_block(*desc, w, x, cond, rope_cos, rope_sin, out, ws, as_stream(stream));
}

// ---------------------------------------------------------------------------
// chain of blocks in place, with the next block's modulation GEMV pipelined
// ---------------------------------------------------------------------------
namespace {
size_t chain_ws_bytes(const dit_block_desc &d) {
    return block_ws(d).total + align256((size_t)ada_rows(d) * 4);
}

struct EventPair {
    hipEvent_t ready = nullptr, freed = nullptr;
    ~EventPair() {
        if (ready) (void)hipEventDestroy(ready);
        if (freed) (void)hipEventDestroy(freed);
    }
};
}  // namespace

int dit_block_chain_workspace_size(const dit_block_desc *desc, size_t *bytes) {
    DIT_TRY(check_desc(desc));
    if (!bytes) return fail(DIT_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = chain_ws_bytes(*desc);
    return ok();
}

int dit_block_chain_forward(const dit_block_desc *desc, const dit_block_weights *blocks, int32_t n_blocks, void *x,
                            const float *cond, const float *rope_cos, const float *rope_sin, void *ws,
                            size_t ws_bytes, void *stream, void *side_stream) {
    if (n_blocks < 1 || !blocks) return fail(DIT_ERR_INVALID_ARG, "n_blocks must be >= 1 and blocks non-NULL");
    for (int l = 0; l < n_blocks; ++l) DIT_TRY(check_block_call(desc, &blocks[l], x, cond, rope_cos, rope_sin, x));
    const dit_block_desc &d = *desc;
    if (!ws) return fail(DIT_ERR_INVALID_ARG, "ws is required");
    if (!aligned16(ws)) return fail(DIT_ERR_ALIGNMENT, "ws must be 16-byte aligned");
    const size_t need = chain_ws_bytes(d);
    if (ws_bytes < need) return fail(DIT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, need);
    const size_t xbytes = (size_t)d.batch * d.seq * d.hidden * (d.x_dtype == DIT_F32 ? 4 : 2);
    if (overlaps(ws, need, x, xbytes)) return fail(DIT_ERR_INVALID_ARG, "workspace overlaps x");
    DIT_TRY(device_check());
    hipStream_t s = as_stream(stream), side = as_stream(side_stream);
    const BlockWs L = block_ws(d);
    uint8_t *wsb = (uint8_t *)ws;
    const int xf = d.x_dtype == DIT_F32, wf = d.w_dtype == DIT_F32;
    if (d.cond_dim == 0) {
        for (int l = 0; l < n_blocks; ++l)
            DIT_TRY(block_body(d, blocks[l], x, xf, nullptr, rope_cos, rope_sin, x, xf, wsb, L, s));
        return ok();
    }
    // two modulation buffers: the block's own slot and one behind the block workspace
    float *mbuf[2] = {(float *)(wsb + L.m), (float *)(wsb + L.total)};
    bool shared = true;
    for (int l = 1; l < n_blocks; ++l)
        shared = shared && blocks[l].w_ada == blocks[0].w_ada && blocks[l].b_ada == blocks[0].b_ada;
    const int rows = ada_rows(d);
    DIT_TRY_HIP(launch_adaln_gemv(blocks[0].w_ada, wf, blocks[0].b_ada, cond, rows, d.cond_dim, 1, mbuf[0], s));
    if (shared || n_blocks == 1 || !side_stream || side == s) {
        for (int l = 0; l < n_blocks; ++l) {
            float *m = mbuf[0];
            if (l > 0 && !shared)
                DIT_TRY_HIP(launch_adaln_gemv(blocks[l].w_ada, wf, blocks[l].b_ada, cond, rows, d.cond_dim, 1, m, s));
            DIT_TRY(block_body(d, blocks[l], x, xf, m, rope_cos, rope_sin, x, xf, wsb, L, s));
        }
        return ok();
    }
    // Layer pipelining: the modulation GEMV of block l + 1 (HBM-bound) runs on
    // the side stream while block l's GEMMs (MFMA-bound) run on the main
    // stream.  `freed` marks the end of the block that last read a buffer,
    // `ready` the end of the GEMV that refills it.
    EventPair ev;
    DIT_TRY_HIP(hipEventCreateWithFlags(&ev.ready, hipEventDisableTiming));
    DIT_TRY_HIP(hipEventCreateWithFlags(&ev.freed, hipEventDisableTiming));
    DIT_TRY_HIP(hipEventRecord(ev.freed, s));   // cond and every earlier write on the main stream
    for (int l = 0; l < n_blocks; ++l) {
        if (l + 1 < n_blocks) {
            DIT_TRY_HIP(hipStreamWaitEvent(side, ev.freed, 0));
            DIT_TRY_HIP(launch_adaln_gemv(blocks[l + 1].w_ada, wf, blocks[l + 1].b_ada, cond, rows, d.cond_dim, 1,
                                          mbuf[(l + 1) & 1], side));
            DIT_TRY_HIP(hipEventRecord(ev.ready, side));
        }
        DIT_TRY(block_body(d, blocks[l], x, xf, mbuf[l & 1], rope_cos, rope_sin, x, xf, wsb, L, s));
        if (l + 1 < n_blocks) {
            DIT_TRY_HIP(hipEventRecord(ev.freed, s));
            DIT_TRY_HIP(hipStreamWaitEvent(s, ev.ready, 0));
        }
    }
    return ok();
}

int dit_stack_workspace_size(const dit_model *model, size_t *bytes) {
    DIT_TRY(check_model(model));
    if (!bytes) return fail(DIT_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = stack_ws(*model).total;
    return ok();
}

int dit_stack_step(const dit_model *model, const float *latent, const float *cond, const float *rope_cos,
                   const float *rope_sin, float *velocity, void *ws, size_t ws_bytes, void *stream) {
    DIT_TRY(check_model(model));
    const dit_model &M = *model;
    const dit_block_desc &d = M.blk;
    if (!latent || !cond || !rope_cos || !rope_sin || !velocity || !ws)
        return fail(DIT_ERR_INVALID_ARG, "latent, cond, rope tables, velocity and ws are required");
    if (!aligned16(latent) || !aligned16(cond) || !aligned16(velocity) || !aligned16(ws) || !aligned4(rope_cos) ||
        !aligned4(rope_sin))
        return fail(DIT_ERR_ALIGNMENT, "latent, cond, velocity, ws must be 16-byte aligned");
    const StackWs L = stack_ws(M);
    if (ws_bytes < L.total) return fail(DIT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, L.total);
    const int64_t N = (int64_t)d.batch * d.seq;
    const size_t lbytes = (size_t)N * M.latent_dim * 4;
    if (overlaps(ws, L.total, latent, lbytes) || overlaps(ws, L.total, velocity, lbytes))
        return fail(DIT_ERR_INVALID_ARG, "workspace overlaps latent or velocity");
    DIT_TRY(device_check());
    hipStream_t s = as_stream(stream);
    uint8_t *wsb = (uint8_t *)ws;
    float *x = (float *)(wsb + L.x);
    float *fm = (float *)(wsb + L.fm);
    bf16 *lat = (bf16 *)(wsb + L.lat);
    float *m = (float *)(wsb + L.blk.m);
    const int D = d.hidden;

    const bool f32 = d.w_dtype == DIT_F32;
    // patch embedding: x = bf16(latent) W_in^T + b_in (fp32 residual stream);
    // the fp32 path takes the fp32 latent as it is
    if (f32) {
        DIT_TRY_HIP(launch_gemm_residual_f32(latent, (const float *)M.w_in, N, D, M.latent_dim, nullptr, nullptr, 0,
                                             M.b_in, x, s));
    } else {
        DIT_TRY_HIP(launch_f32_to_bf16(latent, lat, N * M.latent_dim, s));
        DIT_TRY_HIP(launch_gemm_residual(lat, (const bf16 *)M.w_in, N, D, M.latent_dim, nullptr, 1, nullptr, 0, M.b_in,
                                         x, 1, s));
    }

    bool shared = true;
    for (int l = 1; l < M.layers; ++l)
        shared = shared && M.blocks[l].w_ada == M.blocks[0].w_ada && M.blocks[l].b_ada == M.blocks[0].b_ada;
    for (int l = 0; l < M.layers; ++l) {
        const dit_block_weights &w = M.blocks[l];
        if (l == 0 || !shared)
            DIT_TRY_HIP(launch_adaln_gemv(w.w_ada, f32, w.b_ada, cond, ada_rows(d), d.cond_dim, 1, m, s));
        DIT_TRY(block_body(d, w, x, 1, m, rope_cos, rope_sin, x, 1, wsb, L.blk, s));
    }

    // final AdaLN-continuous norm: [scale | shift] = W_f c + b_f (no SiLU), then projection
    DIT_TRY_HIP(launch_adaln_gemv(M.w_fmod, f32, M.b_fmod, cond, 2 * D, d.cond_dim, 0, fm, s));
    if (f32) {
        float *hf = (float *)(wsb + L.blk.h);
        DIT_TRY_HIP(launch_ln_modulate_f32(x, N, D, d.norm == DIT_RMSNORM, fm + D, fm, 0, d.eps, hf, s));
        DIT_TRY_HIP(launch_gemm_residual_f32(hf, (const float *)M.w_out, N, M.latent_dim, D, nullptr, nullptr, 0,
                                             M.b_out, velocity, s));
        return ok();
    }
    bf16 *h = (bf16 *)(wsb + L.blk.h);
    DIT_TRY_HIP(launch_ln_modulate(x, 1, N, D, d.norm == DIT_RMSNORM, fm + D, fm, 0, d.eps, h, s));
    DIT_TRY_HIP(launch_gemm_residual(h, (const bf16 *)M.w_out, N, M.latent_dim, D, nullptr, 1, nullptr, 0, M.b_out,
                                     velocity, 1, s));
    return ok();
}

int euler_flowmatch_update(float *latent, const float *velocity, int64_t n, float sigma, float sigma_next,
                           void *stream) {
    if (!latent || !velocity) return fail(DIT_ERR_INVALID_ARG, "latent and velocity are required");
    if (n < 0) return fail(DIT_ERR_INVALID_ARG, "n must be >= 0");
    if (!aligned16(latent) || !aligned16(velocity)) return fail(DIT_ERR_ALIGNMENT, "latent/velocity must be 16-byte aligned");
    if (latent != velocity && overlaps(latent, n * 4, velocity, n * 4))
        return fail(DIT_ERR_INVALID_ARG, "latent and velocity overlap");
    if (!isfinite(sigma) || !isfinite(sigma_next)) return fail(DIT_ERR_INVALID_ARG, "sigmas must be finite");
    DIT_TRY(device_check());
    if (n == 0) return ok();
    DIT_TRY_HIP(launch_euler(latent, velocity, n, sigma_next - sigma, as_stream(stream)));
    return ok();
}

int dit_timestep_embedding(float t, int32_t dim, float *cond_out, void *stream) {
    if (!cond_out) return fail(DIT_ERR_INVALID_ARG, "cond_out is NULL");
    if (dim <= 0 || dim % 2) return fail(DIT_ERR_INVALID_ARG, "dim must be positive and even");
    if (!isfinite(t)) return fail(DIT_ERR_INVALID_ARG, "t must be finite");
    DIT_TRY(device_check());
    DIT_TRY_HIP(launch_timestep_embedding(t, dim, cond_out, as_stream(stream)));
    return ok();
}

int dit_sigma_embedding(float sigma, int32_t dim, float *cond_out, void *stream) {
    if (!isfinite(sigma)) return fail(DIT_ERR_INVALID_ARG, "sigma must be finite");
    return dit_timestep_embedding(1000.0f * sigma, dim, cond_out, stream);
}

int dit_flowmatch_sigmas(int32_t steps, float shift, float *out) {
    if (!out) return fail(DIT_ERR_INVALID_ARG, "sigmas_out is NULL");
    if (steps <= 0) return fail(DIT_ERR_INVALID_ARG, "steps must be positive");
    if (!(shift > 0.f) || !isfinite(shift)) return fail(DIT_ERR_INVALID_ARG, "shift must be positive");
    for (int i = 0; i <= steps; ++i) {
        const double s = 1.0 - (double)i / steps;
        out[i] = (float)(shift * s / (1.0 + (shift - 1.0) * s));
    }
    return ok();
}

int dit_rope_tables(const int32_t *pos, int32_t seq, int32_t rope, const int32_t *axes, int32_t n_axes, float theta,
                    int32_t head_dim, float *cos_out, float *sin_out) {
    if (!pos || !axes || !cos_out || !sin_out) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
    if (seq <= 0 || head_dim <= 0 || head_dim % 2) return fail(DIT_ERR_INVALID_ARG, "bad seq/head_dim");
    if (!(theta > 0.f)) return fail(DIT_ERR_INVALID_ARG, "theta must be positive");
    int first_col;
    if (rope == DIT_ROPE_INTERLEAVED) {
        if (n_axes != 3) return fail(DIT_ERR_INVALID_ARG, "interleaved 3D RoPE takes 3 axes (t, h, w)");
        first_col = 0;
    } else if (rope == DIT_ROPE_HALF) {
        if (n_axes != 2) return fail(DIT_ERR_INVALID_ARG, "rotate-half 2D RoPE takes 2 axes (h, w)");
        first_col = 1;
    } else {
        return fail(DIT_ERR_INVALID_ARG, "bad rope layout");
    }
    int sum = 0;
    for (int a = 0; a < n_axes; ++a) {
        if (axes[a] <= 0 || axes[a] % 2) return fail(DIT_ERR_INVALID_ARG, "axis widths must be positive and even");
        sum += axes[a];
    }
    if (sum != head_dim) return fail(DIT_ERR_INVALID_ARG, "axis widths sum to %d, head_dim is %d", sum, head_dim);
    const int half = head_dim / 2;
    for (int s = 0; s < seq; ++s) {
        int m = 0;
        for (int a = 0; a < n_axes; ++a) {
            const double p = pos[s * 3 + first_col + a];
            for (int j = 0; j < axes[a] / 2; ++j, ++m) {
                const double ang = p * pow((double)theta, -2.0 * j / axes[a]);
                cos_out[(size_t)s * half + m] = (float)cos(ang);
                sin_out[(size_t)s * half + m] = (float)sin(ang);
            }
        }
    }
    return ok();
}

// ---------------------------------------------------------------------------
// stage entry points
// ---------------------------------------------------------------------------
int dit_adaln_modulation(const void *w, const float *b, const float *c, int32_t out_dim, int32_t in_dim,
                         int32_t silu_input, float *m, void *stream) {
    if (!w || !c || !m) return fail(DIT_ERR_INVALID_ARG, "w, c and m are required");
    if (out_dim <= 0 || in_dim <= 0) return fail(DIT_ERR_INVALID_ARG, "dims must be positive");
    if (in_dim % 8) return fail(DIT_ERR_UNSUPPORTED, "in_dim must be a multiple of 8");
    if (!aligned16(w) || !aligned16(c) || !aligned4(m) || (b && !aligned4(b)))
        return fail(DIT_ERR_ALIGNMENT, "w and c must be 16-byte aligned");
    DIT_TRY(device_check());
    DIT_TRY_HIP(launch_adaln_gemv(w, 0, b, c, out_dim, in_dim, silu_input, m, as_stream(stream)));
    return ok();
}

int dit_ln_modulate(const void *x, int32_t x_dtype, int64_t rows, int32_t dim, int32_t norm, const float *shift,
                    const float *scale, int32_t mode, float eps, void *h, void *stream) {
    if (!x || !h) return fail(DIT_ERR_INVALID_ARG, "x and h are required");
    if (rows <= 0 || dim <= 0) return fail(DIT_ERR_INVALID_ARG, "rows and dim must be positive");
    if (x_dtype != DIT_F32 && x_dtype != DIT_BF16) return fail(DIT_ERR_INVALID_ARG, "bad x_dtype");
    if (mode != 0 && mode != 1) return fail(DIT_ERR_INVALID_ARG, "mode must be 0 or 1");
    if (mode == 0 && !scale) return fail(DIT_ERR_INVALID_ARG, "mode 0 needs scale");
    if (norm != DIT_LAYERNORM && norm != DIT_RMSNORM) return fail(DIT_ERR_INVALID_ARG, "bad norm kind");
    if (!(eps > 0.f)) return fail(DIT_ERR_INVALID_ARG, "eps must be positive");
    if (dim % 256 || dim > 8192) return fail(DIT_ERR_UNSUPPORTED, "dim must be a multiple of 256 and <= 8192");
    if (!aligned16(x) || !aligned16(h) || (shift && !aligned16(shift)) || (scale && !aligned16(scale)))
        return fail(DIT_ERR_ALIGNMENT, "x, h, shift, scale must be 16-byte aligned");
    DIT_TRY(device_check());
    DIT_TRY_HIP(launch_ln_modulate(x, x_dtype == DIT_F32, rows, dim, norm == DIT_RMSNORM, shift, scale, mode, eps,
                                   (bf16 *)h, as_stream(stream)));
    return ok();
}

int dit_qkv_rope(const dit_block_desc *desc, const void *h, const void *w_qkv, const float *q_g, const float *q_b,
                 const float *k_g, const float *k_b, const float *rope_cos, const float *rope_sin, void *q, void *k,
                 void *vt, void *stream) {
    DIT_TRY(check_desc(desc));
    const dit_block_desc &d = *desc;
    if (!h || !w_qkv || !rope_cos || !rope_sin || !q || !k || !vt) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
    if (d.qk_norm && (!q_g || !q_b || !k_g || !k_b)) return fail(DIT_ERR_INVALID_ARG, "qk_norm needs gamma/beta");
    if (!aligned16(h) || !aligned16(w_qkv) || !aligned16(q) || !aligned16(k) || !aligned16(vt))
        return fail(DIT_ERR_ALIGNMENT, "h, w_qkv, q, k, vt must be 16-byte aligned");
    DIT_TRY(device_check());
    hipStream_t s = as_stream(stream);
    const int spad = seq_pad_of(d.seq);
    const int f32 = d.w_dtype == DIT_F32;
    DIT_TRY_HIP(launch_vt_pad_zero(vt, f32, d.batch * d.kv_heads * d.head_dim, d.seq, spad, s));
    QkvEpiArgs e{d.batch, d.seq, spad, d.heads, d.kv_heads, d.head_dim, d.qk_norm, d.rope == DIT_ROPE_HALF,
                 d.norm == DIT_RMSNORM, d.qk_order == DIT_QK_ROPE_NORM, d.eps, q_g, q_b, k_g, k_b, rope_cos, rope_sin,
                 q, k, vt};
    const int64_t N = (int64_t)d.batch * d.seq;
    const int qkv_dim = (d.heads + 2 * d.kv_heads) * d.head_dim;
    if (f32)
        DIT_TRY_HIP(launch_gemm_qkv_f32((const float *)h, (const float *)w_qkv, N, qkv_dim, d.hidden, e, s));
    else
        DIT_TRY_HIP(launch_gemm_qkv((const bf16 *)h, (const bf16 *)w_qkv, N, qkv_dim, d.hidden, e, s));
    return ok();
}

int dit_flash_attention(const dit_block_desc *desc, const void *q, const void *k, const void *vt, void *out,
                        void *stream) {
    DIT_TRY(check_desc(desc));
    const dit_block_desc &d = *desc;
    if (!q || !k || !vt || !out) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(out))
        return fail(DIT_ERR_ALIGNMENT, "q, k, vt, out must be 16-byte aligned");
    DIT_TRY(device_check());
    if (d.w_dtype == DIT_F32)
        DIT_TRY_HIP(launch_flash_attention_f32((const float *)q, (const float *)k, (const float *)vt, (float *)out,
                                               d.batch, d.seq, seq_pad_of(d.seq), d.heads, d.kv_heads, d.head_dim,
                                               as_stream(stream)));
    else
        DIT_TRY_HIP(launch_flash_attention((const bf16 *)q, (const bf16 *)k, (const bf16 *)vt, (bf16 *)out, d.batch,
                                           d.seq, seq_pad_of(d.seq), d.heads, d.kv_heads, d.head_dim, 1, nullptr,
                                           as_stream(stream)));
    return ok();
}

int dit_attention_workspace_size(const dit_block_desc *desc, int32_t nsplit, size_t *bytes) {
    DIT_TRY(check_desc(desc));
    if (!bytes) return fail(DIT_ERR_INVALID_ARG, "bytes is NULL");
    if (nsplit < 1 || nsplit > 64) return fail(DIT_ERR_INVALID_ARG, "nsplit must be in [1, 64]");
    *bytes = attention_split_bytes(desc->batch, desc->heads, desc->head_dim, nsplit);
    return ok();
}

int dit_flash_attention_split(const dit_block_desc *desc, const void *q, const void *k, const void *vt, void *out,
                              int32_t nsplit, void *ws, size_t ws_bytes, void *stream) {
    DIT_TRY(check_desc(desc));
    const dit_block_desc &d = *desc;
    if (!q || !k || !vt || !out) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
    if (nsplit < 1 || nsplit > 64) return fail(DIT_ERR_INVALID_ARG, "nsplit must be in [1, 64]");
    if (d.w_dtype == DIT_F32) return fail(DIT_ERR_UNSUPPORTED, "the fp32 path has no split-KV form");
    const size_t need = attention_split_bytes(d.batch, d.heads, d.head_dim, nsplit);
    if (need && !ws) return fail(DIT_ERR_INVALID_ARG, "ws is required for nsplit > 1");
    if (ws_bytes < need) return fail(DIT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, need);
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt) || !aligned16(out) || (ws && !aligned16(ws)))
        return fail(DIT_ERR_ALIGNMENT, "q, k, vt, out, ws must be 16-byte aligned");
    DIT_TRY(device_check());
    DIT_TRY_HIP(launch_flash_attention((const bf16 *)q, (const bf16 *)k, (const bf16 *)vt, (bf16 *)out, d.batch, d.seq,
                                       seq_pad_of(d.seq), d.heads, d.kv_heads, d.head_dim, nsplit, ws,
                                       as_stream(stream)));
    return ok();
}

int dit_gemm_gated_residual(const void *a, const void *w, int64_t M, int32_t N, int32_t K, const void *resid,
                            int32_t resid_dtype, const float *gate, int32_t gate_fn, const float *bias, void *out,
                            int32_t out_dtype, void *stream) {
    if (!a || !w || !out) return fail(DIT_ERR_INVALID_ARG, "a, w and out are required");
    if (M <= 0 || N <= 0 || K <= 0) return fail(DIT_ERR_INVALID_ARG, "dims must be positive");
    if ((resid && resid_dtype != DIT_F32 && resid_dtype != DIT_BF16) || (out_dtype != DIT_F32 && out_dtype != DIT_BF16))
        return fail(DIT_ERR_INVALID_ARG, "bad dtype");
    if (gate_fn < DIT_GATE_IDENTITY || gate_fn > DIT_GATE_SIGMOID) return fail(DIT_ERR_INVALID_ARG, "bad gate function");
    if (N % 128 || K % 64) return fail(DIT_ERR_UNSUPPORTED, "N must be a multiple of 128 and K of 64");
    if ((double)M * K >= 2147483648.0 || (double)N * K >= 2147483648.0)
        return fail(DIT_ERR_UNSUPPORTED, "operand exceeds 2^31 elements");
    if (!aligned16(a) || !aligned16(w) || !aligned16(out) || (resid && !aligned16(resid)) || (gate && !aligned4(gate)) ||
        (bias && !aligned4(bias)))
        return fail(DIT_ERR_ALIGNMENT, "a, w, out, resid must be 16-byte aligned");
    const size_t ob = (size_t)M * N * (out_dtype == DIT_F32 ? 4 : 2);
    const size_t rb = (size_t)M * N * (resid_dtype == DIT_F32 ? 4 : 2);
    if (resid && resid != out && overlaps(resid, rb, out, ob)) return fail(DIT_ERR_INVALID_ARG, "resid overlaps out");
    if (resid == out && resid && resid_dtype != out_dtype) return fail(DIT_ERR_INVALID_ARG, "in-place needs equal dtypes");
    DIT_TRY(device_check());
    DIT_TRY_HIP(launch_gemm_residual((const bf16 *)a, (const bf16 *)w, M, N, K, resid, resid_dtype == DIT_F32, gate,
                                     gate_fn, bias, out, out_dtype == DIT_F32, as_stream(stream)));
    return ok();
}

int dit_gemm_swiglu(const void *a, const void *w_gate_up, int64_t M, int32_t F, int32_t K, int32_t act, void *u,
                    void *stream) {
    if (!a || !w_gate_up || !u) return fail(DIT_ERR_INVALID_ARG, "a, w_gate_up and u are required");
    if (act != DIT_ACT_SILU && act != DIT_ACT_GELU_TANH) return fail(DIT_ERR_INVALID_ARG, "bad act");
    if (M <= 0 || F <= 0 || K <= 0) return fail(DIT_ERR_INVALID_ARG, "dims must be positive");
    if (F % 128 || K % 64) return fail(DIT_ERR_UNSUPPORTED, "F must be a multiple of 128 and K of 64");
    if ((double)M * K >= 2147483648.0 || 2.0 * F * K >= 2147483648.0 || (double)M * F >= 2147483648.0)
        return fail(DIT_ERR_UNSUPPORTED, "operand exceeds 2^31 elements");
    if (!aligned16(a) || !aligned16(w_gate_up) || !aligned16(u)) return fail(DIT_ERR_ALIGNMENT, "16-byte alignment required");
    DIT_TRY(device_check());
    DIT_TRY_HIP(launch_gemm_swiglu((const bf16 *)a, (const bf16 *)w_gate_up, M, F, K, act, (bf16 *)u, as_stream(stream)));
    return ok();
}

// ---------------------------------------------------------------------------
// W8A8 H256 stage entry points
// ---------------------------------------------------------------------------
int dit_quantize_h256(const void *x, int32_t x_dtype, int64_t rows, int32_t cols, void *q, float *scale,
                      void *stream) {
    if (!x || !q || !scale) return fail(DIT_ERR_INVALID_ARG, "x, q and scale are required");
    if (rows <= 0 || cols <= 0) return fail(DIT_ERR_INVALID_ARG, "rows and cols must be positive");
    if (x_dtype != DIT_F32 && x_dtype != DIT_BF16) return fail(DIT_ERR_INVALID_ARG, "bad x_dtype");
    if (!quantize_h256_supported(cols))
        return fail(DIT_ERR_UNSUPPORTED, "cols must be a multiple of 256 with ceil(cols / 1024) <= 7 or a multiple of 4 up to 32");
    if ((double)rows * cols >= 2147483648.0) return fail(DIT_ERR_UNSUPPORTED, "x exceeds 2^31 elements");
    if (!aligned16(x) || !aligned16(q) || !aligned4(scale)) return fail(DIT_ERR_ALIGNMENT, "x and q must be 16-byte aligned");
    const size_t xb = (size_t)rows * cols * (x_dtype == DIT_F32 ? 4 : 2);
    if (overlaps(x, xb, q, (size_t)rows * cols) || overlaps(x, xb, scale, (size_t)rows * 4) ||
        overlaps(q, (size_t)rows * cols, scale, (size_t)rows * 4))
        return fail(DIT_ERR_INVALID_ARG, "x, q and scale must not overlap");
    DIT_TRY(device_check());
    DIT_TRY_HIP(launch_quantize_h256(x, x_dtype == DIT_F32, rows, cols, (int8_t *)q, scale, as_stream(stream)));
    return ok();
}

int dit_ln_modulate_h256q(const void *x, int32_t x_dtype, int64_t rows, int32_t dim, int32_t norm,
                          const float *shift, const float *scale, int32_t mode, float eps, void *q, float *qscale,
                          void *stream) {
    if (!x || !q || !qscale) return fail(DIT_ERR_INVALID_ARG, "x, q and qscale are required");
    if (rows <= 0 || dim <= 0) return fail(DIT_ERR_INVALID_ARG, "rows and dim must be positive");
    if (x_dtype != DIT_F32 && x_dtype != DIT_BF16) return fail(DIT_ERR_INVALID_ARG, "bad x_dtype");
    if (mode != 0 && mode != 1) return fail(DIT_ERR_INVALID_ARG, "mode must be 0 or 1");
    if (mode == 0 && !scale) return fail(DIT_ERR_INVALID_ARG, "mode 0 needs scale");
    if (norm != DIT_LAYERNORM && norm != DIT_RMSNORM) return fail(DIT_ERR_INVALID_ARG, "bad norm kind");
    if (!(eps > 0.f)) return fail(DIT_ERR_INVALID_ARG, "eps must be positive");
    if (dim % 256 || dim > 8192) return fail(DIT_ERR_UNSUPPORTED, "dim must be a multiple of 256 and <= 8192");
    if (!aligned16(x) || !aligned16(q) || !aligned4(qscale) || (shift && !aligned16(shift)) ||
        (scale && !aligned16(scale)))
        return fail(DIT_ERR_ALIGNMENT, "x, q, shift, scale must be 16-byte aligned");
    DIT_TRY(device_check());
    DIT_TRY_HIP(launch_ln_modulate_q8(x, x_dtype == DIT_F32, rows, dim, norm == DIT_RMSNORM, shift, scale, mode, eps,
                                      (int8_t *)q, qscale, as_stream(stream)));
    return ok();
}

namespace {
int check_q8_operands(const void *a, const float *as, const void *w, const float *ws, int64_t M, int64_t wrows,
                      int32_t K) {
    if (!a || !as || !w || !ws) return fail(DIT_ERR_INVALID_ARG, "a, a_scale, w and w_scale are required");
    if (K % 128) return fail(DIT_ERR_UNSUPPORTED, "K must be a multiple of 128");
    if ((double)M * K >= 2147483648.0 || (double)wrows * K >= 2147483648.0)
        return fail(DIT_ERR_UNSUPPORTED, "operand exceeds 2^31 elements");
    if (!aligned16(a) || !aligned16(w) || !aligned16(as) || !aligned16(ws))
        return fail(DIT_ERR_ALIGNMENT, "codes and scales must be 16-byte aligned");
    return DIT_OK;
}
}  // namespace

int dit_gemm_w8a8_gated_residual(const void *a, const float *a_scale, const void *w, const float *w_scale, int64_t M,
                                 int32_t N, int32_t K, const void *resid, int32_t resid_dtype, const float *gate,
                                 int32_t gate_fn, const float *bias, void *out, int32_t out_dtype, void *stream) {
    if (!out) return fail(DIT_ERR_INVALID_ARG, "out is required");
    if (M <= 0 || N <= 0 || K <= 0) return fail(DIT_ERR_INVALID_ARG, "dims must be positive");
    if ((resid && resid_dtype != DIT_F32 && resid_dtype != DIT_BF16) || (out_dtype != DIT_F32 && out_dtype != DIT_BF16))
        return fail(DIT_ERR_INVALID_ARG, "bad dtype");
    if (gate_fn < DIT_GATE_IDENTITY || gate_fn > DIT_GATE_SIGMOID) return fail(DIT_ERR_INVALID_ARG, "bad gate function");
    if (N % 128) return fail(DIT_ERR_UNSUPPORTED, "N must be a multiple of 128");
    DIT_TRY(check_q8_operands(a, a_scale, w, w_scale, M, N, K));
    if (!aligned16(out) || (resid && !aligned16(resid)) || (gate && !aligned4(gate)) || (bias && !aligned4(bias)))
        return fail(DIT_ERR_ALIGNMENT, "out and resid must be 16-byte aligned");
    const size_t ob = (size_t)M * N * (out_dtype == DIT_F32 ? 4 : 2);
    const size_t rb = (size_t)M * N * (resid_dtype == DIT_F32 ? 4 : 2);
    if (resid && resid != out && overlaps(resid, rb, out, ob)) return fail(DIT_ERR_INVALID_ARG, "resid overlaps out");
    if (resid == out && resid && resid_dtype != out_dtype) return fail(DIT_ERR_INVALID_ARG, "in-place needs equal dtypes");
    DIT_TRY(device_check());
    DIT_TRY_HIP(launch_gemm_residual_q8((const int8_t *)a, a_scale, (const int8_t *)w, w_scale, M, N, K, resid,
                                        resid_dtype == DIT_F32, gate, gate_fn, bias, out, out_dtype == DIT_F32,
                                        as_stream(stream)));
    return ok();
}

int dit_gemm_w8a8_swiglu(const void *a, const float *a_scale, const void *w_gate_up, const float *w_scale, int64_t M,
                         int32_t F, int32_t K, int32_t act, void *u, void *stream) {
    if (!u) return fail(DIT_ERR_INVALID_ARG, "u is required");
    if (act != DIT_ACT_SILU && act != DIT_ACT_GELU_TANH) return fail(DIT_ERR_INVALID_ARG, "bad act");
    if (M <= 0 || F <= 0 || K <= 0) return fail(DIT_ERR_INVALID_ARG, "dims must be positive");
    if (F % 128) return fail(DIT_ERR_UNSUPPORTED, "F must be a multiple of 128");
    DIT_TRY(check_q8_operands(a, a_scale, w_gate_up, w_scale, M, 2 * (int64_t)F, K));
    if ((double)M * F >= 2147483648.0) return fail(DIT_ERR_UNSUPPORTED, "operand exceeds 2^31 elements");
    if (!aligned16(u)) return fail(DIT_ERR_ALIGNMENT, "u must be 16-byte aligned");
    DIT_TRY(device_check());
    DIT_TRY_HIP(launch_gemm_swiglu_q8((const int8_t *)a, a_scale, (const int8_t *)w_gate_up, w_scale, M, F, K, act,
                                      (bf16 *)u, as_stream(stream)));
    return ok();
}

int dit_qkv_rope_w8a8(const dit_block_desc *desc, const void *h, const float *h_scale, const void *w_qkv,
                      const float *w_scale, const float *q_g, const float *q_b, const float *k_g, const float *k_b,
                      const float *rope_cos, const float *rope_sin, void *q, void *k, void *vt, void *stream) {
    DIT_TRY(check_desc(desc));
    const dit_block_desc &d = *desc;
    if (!rope_cos || !rope_sin || !q || !k || !vt) return fail(DIT_ERR_INVALID_ARG, "NULL pointer");
    if (d.qk_norm && (!q_g || !q_b || !k_g || !k_b)) return fail(DIT_ERR_INVALID_ARG, "qk_norm needs gamma/beta");
    const int64_t N = (int64_t)d.batch * d.seq;
    const int qkv_dim = (d.heads + 2 * d.kv_heads) * d.head_dim;
    DIT_TRY(check_q8_operands(h, h_scale, w_qkv, w_scale, N, qkv_dim, d.hidden));
    if (!aligned16(q) || !aligned16(k) || !aligned16(vt)) return fail(DIT_ERR_ALIGNMENT, "q, k, vt must be 16-byte aligned");
    DIT_TRY(device_check());
    hipStream_t s = as_stream(stream);
    const int spad = seq_pad_of(d.seq);
    DIT_TRY_HIP(launch_vt_pad_zero(vt, 0, d.batch * d.kv_heads * d.head_dim, d.seq, spad, s));
    QkvEpiArgs e{d.batch, d.seq, spad, d.heads, d.kv_heads, d.head_dim, d.qk_norm, d.rope == DIT_ROPE_HALF,
                 d.norm == DIT_RMSNORM, d.qk_order == DIT_QK_ROPE_NORM, d.eps, q_g, q_b, k_g, k_b, rope_cos, rope_sin,
                 q, k, vt};
    DIT_TRY_HIP(launch_gemm_qkv_q8((const int8_t *)h, h_scale, (const int8_t *)w_qkv, w_scale, N, qkv_dim, d.hidden,
                                   e, s));
    return ok();
}


// ---------------------------------------------------------------------------
// whole denoising loop as HIP graphs
// ---------------------------------------------------------------------------
struct dit_loop {
    std::vector<hipGraphExec_t> steps;
};

namespace {
struct LoopWs {
    size_t stack, cond, vel, total;
};
LoopWs loop_ws(const dit_model &M) {
    LoopWs L;
    L.stack = 0;
    L.cond = align256(stack_ws(M).total);
    L.vel = L.cond + align256((size_t)M.blk.cond_dim * 4);
    L.total = L.vel + align256((size_t)M.blk.batch * M.blk.seq * M.latent_dim * 4);
    return L;
}
void free_loop(dit_loop *lp) {
    for (hipGraphExec_t e : lp->steps)
        if (e) (void)hipGraphExecDestroy(e);
    delete lp;
}
}  // namespace

int dit_loop_workspace_size(const dit_model *model, size_t *bytes) {
    DIT_TRY(check_model(model));
    if (!bytes) return fail(DIT_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = loop_ws(*model).total;
    return ok();
}

int dit_loop_create(const dit_model *model, float *latent, const float *rope_cos, const float *rope_sin,
                    int32_t steps, float shift, void *ws, size_t ws_bytes, dit_loop **loop) {
    if (!loop) return fail(DIT_ERR_INVALID_ARG, "loop is NULL");
    *loop = nullptr;
    DIT_TRY(check_model(model));
    const dit_model &M = *model;
    if (!latent || !rope_cos || !rope_sin || !ws) return fail(DIT_ERR_INVALID_ARG, "latent, rope tables and ws are required");
    if (steps < 1 || steps > 1000) return fail(DIT_ERR_INVALID_ARG, "steps must be in [1, 1000]");
    if (!(shift > 0.f) || !isfinite(shift)) return fail(DIT_ERR_INVALID_ARG, "shift must be positive");
    if (!aligned16(latent) || !aligned16(ws)) return fail(DIT_ERR_ALIGNMENT, "latent and ws must be 16-byte aligned");
    const LoopWs L = loop_ws(M);
    if (ws_bytes < L.total) return fail(DIT_ERR_WORKSPACE, "workspace %zu < required %zu bytes", ws_bytes, L.total);
    const int64_t n = (int64_t)M.blk.batch * M.blk.seq * M.latent_dim;
    if (overlaps(ws, L.total, latent, (size_t)n * 4)) return fail(DIT_ERR_INVALID_ARG, "workspace overlaps latent");
    DIT_TRY(device_check());
    std::vector<float> sig(steps + 1);
    DIT_TRY(dit_flowmatch_sigmas(steps, shift, sig.data()));
    uint8_t *wsb = (uint8_t *)ws;
    float *cond = (float *)(wsb + L.cond), *vel = (float *)(wsb + L.vel);

    // private capture stream (default priority); nothing is launched while capturing
    hipStream_t cs;
    DIT_TRY_HIP(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
    dit_loop *lp = new dit_loop();
    lp->steps.assign(steps, nullptr);
    int rc = DIT_OK;
    for (int i = 0; i < steps && rc == DIT_OK; ++i) {
        hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
        if (e != hipSuccess) {
            rc = fail(DIT_ERR_HIP, "hipStreamBeginCapture: %s", hipGetErrorString(e));
            break;
        }
        rc = dit_sigma_embedding(sig[i], M.blk.cond_dim, cond, cs);
        if (rc == DIT_OK) rc = dit_stack_step(model, latent, cond, rope_cos, rope_sin, vel, wsb + L.stack, L.cond, cs);
        if (rc == DIT_OK) rc = euler_flowmatch_update(latent, vel, n, sig[i], sig[i + 1], cs);
        const std::string err = g_err;              // keep the first error across the clean-up calls
        hipGraph_t g = nullptr;
        e = hipStreamEndCapture(cs, &g);
        if (rc == DIT_OK && e != hipSuccess) rc = fail(DIT_ERR_HIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
        if (rc == DIT_OK) {
            e = hipGraphInstantiate(&lp->steps[i], g, nullptr, nullptr, 0);
            if (e != hipSuccess) rc = fail(DIT_ERR_HIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
        } else {
            g_err = err;
        }
        if (g) (void)hipGraphDestroy(g);
    }
    (void)hipStreamDestroy(cs);
    if (rc != DIT_OK) {
        const std::string err = g_err;
        free_loop(lp);
        g_err = err;
        return rc;
    }
    *loop = lp;
    return ok();
}

int dit_loop_launch_step(dit_loop *loop, int32_t step, void *stream) {
    if (!loop) return fail(DIT_ERR_INVALID_ARG, "loop is NULL");
    if (step < 0 || step >= (int32_t)loop->steps.size())
        return fail(DIT_ERR_INVALID_ARG, "step %d outside [0, %zu)", step, loop->steps.size());
    DIT_TRY_HIP(hipGraphLaunch(loop->steps[step], as_stream(stream)));
    return ok();
}

int dit_loop_launch(dit_loop *loop, void *stream) {
    if (!loop) return fail(DIT_ERR_INVALID_ARG, "loop is NULL");
    for (size_t i = 0; i < loop->steps.size(); ++i) DIT_TRY_HIP(hipGraphLaunch(loop->steps[i], as_stream(stream)));
    return ok();
}

int dit_loop_destroy(dit_loop *loop) {
    if (loop) free_loop(loop);
    return ok();
}

}  // extern "C"
