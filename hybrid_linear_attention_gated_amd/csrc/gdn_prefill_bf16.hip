// gdn_prefill_bf16.hip -- dispatch of the bf16 prefill.
//
// Head sizes 64 and 128 with chunks of 32 or 64 tokens run the fused MFMA
// chunk kernel (gdn_prefill_chunk.hip); the other supported sizes (a head or
// chunk of 16) run the fp32 VALU chunk kernel (gdn_prefill_valu.hip), which
// needs no workspace.
#include "gdn_internal.h"

namespace gdn {

bool prefill_bf16_uses_mfma(int dk, int dv, int chunk) {
    return (dk == 64 || dk == 128) && (dv == 64 || dv == 128) && (chunk == 32 || chunk == 64);
}

size_t prefill_bf16_workspace(int B, int T, int H, int dk, int dv, int chunk) {
    if (!prefill_bf16_uses_mfma(dk, dv, chunk)) return 0;
    return prefill_chunk_workspace(B, T, H, dk, dv, chunk);
}

hipError_t launch_prefill_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const float *g, const float *beta, const float *s0, float *o,
                               float *s_out, int B, int T, int H, int dk, int dv, int chunk,
                               bool delta, void *ws, hipStream_t stream) {
    if (!prefill_bf16_uses_mfma(dk, dv, chunk))
        return launch_prefill_valu(q, k, v, g, beta, s0, o, s_out, B, T, H, dk, dv, chunk, GDN_BF16,
                                   delta, stream);
    return launch_prefill_chunk(q, k, v, g, beta, s0, o, s_out, B, T, H, dk, dv, chunk, delta, ws,
                                stream);
}

}  // namespace gdn
