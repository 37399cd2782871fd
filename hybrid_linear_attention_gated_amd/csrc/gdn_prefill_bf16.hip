// gdn_prefill_bf16.hip -- dispatch of the bf16 prefill.
//
// Head sizes 64 and 128 with chunks of 32 or 64 tokens run the fused MFMA
// chunk kernel (gdn_prefill_chunk.hip); the other supported sizes (a head or
// chunk of 16) run the fp32 VALU chunk kernel (gdn_prefill_valu.hip), which
// needs no workspace.  `chunk` is the longest chunk the chunk form may use.
#include "gdn_internal.h"

namespace gdn {

bool prefill_bf16_uses_mfma(int dk, int dv, int chunk) {
    return (dk == 64 || dk == 128) && (dv == 64 || dv == 128) && (chunk == 32 || chunk == 64);
}

// The chunk the MFMA kernels run for a requested (longest) chunk.  The gated delta rule runs
// 32-token chunks when 64 is allowed: its per-chunk dependency chain (the triangular inverse)
// is shorter and three workgroups fit per compute unit instead of two (64K prefill of 64-wide
// heads 0.65 against 0.82 ms; 3B-shaped 64K call 1.50 against 1.57 ms; packed prompts 0.54
// against 0.66 ms).  The rule without the erase term has no inverse and keeps 64 (0.49 against
// 0.51 ms).
int prefill_kernel_chunk(int dk, int dv, int chunk, bool delta) {
    return (delta && chunk == 64 && prefill_bf16_uses_mfma(dk, dv, 32)) ? 32 : chunk;
}

// Workspace for either rule (the size query takes no rule): the larger of the two plans.
// tfrag: with room for the gated delta rule's per-chunk T diag(b) fragments (128 x 128 heads).
size_t prefill_bf16_workspace(int B, int T, int H, int dk, int dv, int chunk, bool tfrag) {
    if (!prefill_bf16_uses_mfma(dk, dv, chunk)) return 0;
    const size_t a = prefill_chunk_workspace(B, T, H, dk, dv, prefill_kernel_chunk(dk, dv, chunk, true), tfrag);
    const size_t b = prefill_chunk_workspace(B, T, H, dk, dv, prefill_kernel_chunk(dk, dv, chunk, false));
    return a > b ? a : b;
}

hipError_t launch_prefill_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const float *g, const float *beta, const float *s0, float *o,
                               float *s_out, int B, int T, int H, int dk, int dv, int chunk,
                               bool delta, void *ws, hipStream_t stream, bool tfrag) {
    if (!prefill_bf16_uses_mfma(dk, dv, chunk))
        return launch_prefill_valu(q, k, v, g, beta, s0, o, s_out, B, T, H, dk, dv, chunk, GDN_BF16,
                                   delta, stream);
    return launch_prefill_chunk(q, k, v, g, beta, s0, o, s_out, B, T, H, dk, dv,
                                prefill_kernel_chunk(dk, dv, chunk, delta), delta, ws, stream, nullptr,
                                tfrag);
}

}  // namespace gdn
