// Host-side checks of libdit's C ABI for the AddressSanitizer / UBSan build:
// argument validation (including extreme shapes, where 32-bit products would
// overflow), workspace arithmetic, and the host helpers that compute on the
// CPU (sigma grid, RoPE tables) into buffers of exactly the documented size.
// No call here launches a kernel: the invalid calls return before any launch
// and the valid ones are made only when no GPU is visible (they then end in
// DIT_ERR_NO_DEVICE).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include <hip/hip_runtime.h>

#include "dit.h"

static int g_fail = 0;
#define EXPECT(cond, ...)                                 \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                 \
            fprintf(stderr, "\n");                        \
            ++g_fail;                                     \
        }                                                 \
    } while (0)

static dit_block_desc desc(int batch = 1, int seq = 256, int hidden = 256, int heads = 4, int kv = 4, int hd = 64,
                           int ffn = 768, int cond = 256) {
    dit_block_desc d;
    memset(&d, 0, sizeof d);
    d.batch = batch; d.seq = seq; d.hidden = hidden; d.heads = heads; d.kv_heads = kv; d.head_dim = hd;
    d.ffn = ffn; d.cond_dim = cond; d.qk_norm = 1; d.eps = 1e-6f; d.x_dtype = DIT_BF16; d.w_dtype = DIT_BF16;
    return d;
}

int main() {
    int ndev = 0;
    const bool no_gpu = hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0;
    void *const FAKE = (void *)(uintptr_t)(1u << 20);
    void *const FAR = (void *)((uintptr_t)1 << 40);

    // --- descriptor validation over extreme shapes (products past 2^31 must
    // be rejected, never computed in 32-bit) -------------------------------
    size_t bytes = 0;
    EXPECT(dit_block_workspace_size(nullptr, &bytes) == DIT_ERR_INVALID_ARG, "NULL desc");
    dit_block_desc d = desc();
    EXPECT(dit_block_workspace_size(&d, nullptr) == DIT_ERR_INVALID_ARG, "NULL bytes");
    EXPECT(dit_block_workspace_size(&d, &bytes) == DIT_OK && bytes > 0, "valid desc");
    const int big[] = {1 << 30, 0x7fffffff, -1, 0};
    for (int v : big) {
        dit_block_desc e = desc(v, v, 256, 4, 4, 64, 768, 256);
        const int rc = dit_block_workspace_size(&e, &bytes);
        EXPECT(rc != DIT_OK, "batch = seq = %d accepted", v);
        e = desc(1, 256, 256, v, v, 64, 768, 256);
        EXPECT(dit_block_workspace_size(&e, &bytes) != DIT_OK, "heads %d accepted", v);
        e = desc(1, 256, 256, 4, 4, v, 768, 256);
        EXPECT(dit_block_workspace_size(&e, &bytes) != DIT_OK, "head_dim %d accepted", v);
        e = desc(1, 256, v, 4, 4, 64, v, v);
        EXPECT(dit_block_workspace_size(&e, &bytes) != DIT_OK, "hidden = ffn = cond_dim %d accepted", v);
    }
    {   // the largest accepted bf16 block: 2^31 - 1 elements per operand at most
        dit_block_desc e = desc(1, 65536, 8192, 64, 64, 128, 32640, 256);
        const int rc = dit_block_workspace_size(&e, &bytes);
        EXPECT(rc == DIT_OK || rc == DIT_ERR_UNSUPPORTED, "large block rc %d", rc);
        if (rc == DIT_OK) EXPECT(bytes > (size_t)65536 * 32640 * 2, "workspace too small for u: %zu", bytes);
        e.w_dtype = DIT_F32; e.x_dtype = DIT_F32;
        EXPECT(dit_block_workspace_size(&e, &bytes) == DIT_ERR_UNSUPPORTED, "fp32 operand past 4 GiB accepted");
    }
    for (int f = 0; f < 8; ++f) {   // every enum field out of range
        dit_block_desc e = desc();
        int32_t *fields[] = {&e.norm, &e.rope, &e.x_dtype, &e.w_dtype, &e.act, &e.gate, &e.mod, &e.qk_order};
        *fields[f] = 1000;
        EXPECT(dit_block_workspace_size(&e, &bytes) == DIT_ERR_INVALID_ARG, "enum field %d", f);
        *fields[f] = -1000;
        EXPECT(dit_block_workspace_size(&e, &bytes) == DIT_ERR_INVALID_ARG, "enum field %d negative", f);
    }

    // --- block forward: every invalid argument is reported before a launch --
    dit_block_weights w;
    memset(&w, 0, sizeof w);
    w.w_ada = FAKE; w.b_ada = (const float *)FAKE; w.w_qkv = FAKE; w.w_o = FAKE; w.w_gate_up = FAKE;
    w.w_down = FAKE; w.q_g = w.q_b = w.k_g = w.k_b = (const float *)FAKE;
    dit_block_workspace_size(&d, &bytes);
    EXPECT(dit_block_forward(&d, &w, FAKE, (const float *)FAKE, (const float *)FAKE, (const float *)FAKE, FAKE,
                             (char *)FAKE + 4096, bytes, nullptr) == DIT_ERR_INVALID_ARG, "workspace overlapping x");
    EXPECT(dit_block_forward(&d, &w, FAKE, (const float *)FAKE, (const float *)FAKE, (const float *)FAKE,
                             (char *)FAKE + 256, FAR, bytes, nullptr) == DIT_ERR_INVALID_ARG, "partial overlap");
    EXPECT(dit_block_forward(&d, &w, FAKE, nullptr, (const float *)FAKE, (const float *)FAKE, FAR, FAR, bytes,
                             nullptr) == DIT_ERR_INVALID_ARG, "missing cond");
    EXPECT(dit_block_forward(&d, &w, (char *)FAKE + 4, (const float *)FAKE, (const float *)FAKE, (const float *)FAKE,
                             FAR, (char *)FAR + (1 << 30), bytes, nullptr) == DIT_ERR_ALIGNMENT, "misaligned x");
    EXPECT(dit_block_forward(&d, &w, FAKE, (const float *)FAKE, (const float *)FAKE, (const float *)FAKE, FAR,
                             (char *)FAR + (1 << 30), bytes - 1, nullptr) == DIT_ERR_WORKSPACE, "small workspace");
    EXPECT(dit_block_forward_noalloc(&d, nullptr, FAKE, (const float *)FAKE, (const float *)FAKE,
                                     (const float *)FAKE, FAR, nullptr) == DIT_ERR_INVALID_ARG, "noalloc NULL w");
    if (no_gpu) {
        EXPECT(dit_block_forward(&d, &w, FAKE, (const float *)FAKE, (const float *)FAKE, (const float *)FAKE, FAR,
                                 (char *)FAR + (1 << 30), bytes, nullptr) == DIT_ERR_NO_DEVICE, "valid call");
        EXPECT(dit_block_forward_noalloc(&d, &w, FAKE, (const float *)FAKE, (const float *)FAKE,
                                         (const float *)FAKE, FAR, nullptr) == DIT_ERR_NO_DEVICE, "noalloc valid");
    }
    EXPECT(strlen(dit_last_error()) > 0, "last error message");

    // --- stack, loop, chain: validation and workspace arithmetic -------------
    dit_model m;
    memset(&m, 0, sizeof m);
    m.blk = desc();
    m.blk.x_dtype = DIT_F32;
    m.layers = 3;
    m.latent_dim = 128;
    std::vector<dit_block_weights> blocks(3, w);
    m.blocks = blocks.data();
    m.w_in = m.w_fmod = m.w_out = FAKE;
    m.b_in = m.b_fmod = m.b_out = (const float *)FAKE;
    EXPECT(dit_stack_workspace_size(&m, &bytes) == DIT_OK && bytes > 0, "stack ws");
    size_t lb = 0;
    EXPECT(dit_loop_workspace_size(&m, &lb) == DIT_OK && lb > bytes, "loop ws");
    dit_loop *loop = (dit_loop *)FAKE;
    EXPECT(dit_loop_create(&m, (float *)FAKE, (const float *)FAKE, (const float *)FAKE, 0, 4.f, FAR, lb, &loop) ==
               DIT_ERR_INVALID_ARG && loop == nullptr, "loop steps 0");
    m.layers = 0;
    EXPECT(dit_stack_workspace_size(&m, &bytes) == DIT_ERR_INVALID_ARG, "no layers");
    m.layers = 3;
    m.latent_dim = 100;
    EXPECT(dit_stack_workspace_size(&m, &bytes) == DIT_ERR_UNSUPPORTED, "latent 100");
    size_t cb = 0;
    EXPECT(dit_block_chain_workspace_size(&d, &cb) == DIT_OK && cb > 0, "chain ws");
    EXPECT(dit_block_chain_forward(&d, blocks.data(), 0, FAKE, (const float *)FAKE, (const float *)FAKE,
                                   (const float *)FAKE, FAR, cb, nullptr, nullptr) == DIT_ERR_INVALID_ARG, "chain n 0");
    EXPECT(dit_loop_destroy(nullptr) == DIT_OK, "destroy NULL");

    // --- host helpers computing on the CPU into exactly sized buffers --------
    for (int steps : {1, 2, 8, 50}) {
        std::vector<float> sig((size_t)steps + 1);
        EXPECT(dit_flowmatch_sigmas(steps, 4.0f, sig.data()) == DIT_OK, "sigmas %d", steps);
        EXPECT(sig[0] == 1.0f && sig[steps] == 0.0f, "sigma ends %d", steps);
    }
    EXPECT(dit_flowmatch_sigmas(0, 4.0f, nullptr) == DIT_ERR_INVALID_ARG, "sigmas NULL");
    for (int seq : {1, 7, 300}) {
        std::vector<int32_t> pos((size_t)seq * 3);
        for (int i = 0; i < seq; ++i) { pos[i * 3] = i % 3; pos[i * 3 + 1] = i / 5; pos[i * 3 + 2] = i % 5; }
        const int32_t axes3[] = {32, 48, 48}, axes2[] = {32, 32};
        std::vector<float> c((size_t)seq * 64), s((size_t)seq * 64);
        EXPECT(dit_rope_tables(pos.data(), seq, DIT_ROPE_INTERLEAVED, axes3, 3, 256.f, 128, c.data(), s.data()) ==
                   DIT_OK, "rope 3d");
        std::vector<float> c2((size_t)seq * 32), s2((size_t)seq * 32);
        EXPECT(dit_rope_tables(pos.data(), seq, DIT_ROPE_HALF, axes2, 2, 100.f, 64, c2.data(), s2.data()) == DIT_OK,
               "rope half");
        EXPECT(dit_rope_tables(pos.data(), seq, DIT_ROPE_HALF, axes3, 3, 100.f, 128, c.data(), s.data()) ==
                   DIT_ERR_INVALID_ARG, "rope half with 3 axes");
    }
    for (int st = -7; st <= 1; ++st) EXPECT(dit_status_string(st) != nullptr, "status %d", st);
    EXPECT(dit_trace_end(nullptr) == DIT_ERR_INVALID_ARG, "trace end without begin");

    if (g_fail) {
        fprintf(stderr, "%d check(s) failed\n", g_fail);
        return 1;
    }
    printf("abi checks passed (%s)\n", no_gpu ? "no GPU: valid calls ended in DIT_ERR_NO_DEVICE" : "GPU present");
    return 0;
}
