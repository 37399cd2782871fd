// gdn_internal.h -- device helpers and launcher declarations shared by the
// libgdn translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "gdn.h"

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- scalar conversions --------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (inputs are finite here).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Loads one stored q/k/v element as fp32.
template <typename T> __device__ __forceinline__ float load_in(const T *p, size_t i);
template <> __device__ __forceinline__ float load_in<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_in<uint16_t>(const uint16_t *p, size_t i) {
    return bf16_bits_to_f32(p[i]);
}

// ---- launchers (host side; each returns the launch's hipError_t) ---------

// `delta` selects the rule everywhere: true = gated delta rule, false = no erase term.
// slots == NULL: sequence n uses state n; else state slots[n] of a pool of `pool` states
// (slots outside [0, pool) are padding: zero output, no state touched).
hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state, float *o, int N, int H, int dk, int dv,
                         gdn_dtype dt, bool delta, const int *slots, int pool, hipStream_t stream);

// Chunked prefill with fp32 VALU arithmetic (fp32 inputs, and bf16 inputs at
// sizes the MFMA path does not tile).  Needs no workspace.
// chunk_states (optional): receives the state every chunk starts from, [B*H][N][dk][dv].
hipError_t launch_prefill_valu(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *s0, float *o, float *s_out, int B,
                               int T, int H, int dk, int dv, int chunk, gdn_dtype dt,
                               bool delta, hipStream_t stream, float *chunk_states = nullptr);
// The same for packed sequences (cu, slots, init: host arrays as for the MFMA packed path); the
// workspace holds a table of prefill_valu_varlen_workspace(S) bytes built from them.
size_t prefill_valu_varlen_workspace(int S);
hipError_t launch_prefill_valu_varlen(const void *q, const void *k, const void *v, const float *g,
                                      const float *beta, const int *cu, int S, const int *slots,
                                      const int *init, float *pool, float *o, int H, int dk, int dv, int chunk,
                                      gdn_dtype dt, bool delta, void *ws, hipStream_t stream);

// bf16 inputs: chunked prefill with bf16 MFMA contractions.
bool prefill_bf16_uses_mfma(int dk, int dv, int chunk);
int prefill_kernel_chunk(int dk, int dv, int chunk, bool delta);
// the input preparation fused into the MFMA chunk kernels' loads (bf16 raw projections)
bool prepare_prefill_supported(int dk, int dv);
size_t prepare_prefill_workspace(int B, int T, int H, int dk, int dv);
hipError_t launch_prepare_prefill(const uint16_t *xq, const uint16_t *xk, const uint16_t *xv, const float *conv_w,
                                  const float *a_raw, const float *b_raw, const float *rate, const float *bias,
                                  const float *conv_in, float *conv_out, const float *s0, float *o, float *s_out,
                                  int B, int T, int H, int dk, int dv, bool delta, void *ws, hipStream_t stream);
hipError_t launch_prefill_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const float *g, const float *beta, const float *s0, float *o,
                               float *s_out, int B, int T, int H, int dk, int dv, int chunk,
                               bool delta, void *ws, hipStream_t stream, bool tfrag = true);
size_t prefill_bf16_workspace(int B, int T, int H, int dk, int dv, int chunk, bool tfrag = true);

// bf16 inputs, fused chunk kernel with sequence pieces (gdn_prefill_chunk.hip).
// chunk_states (optional): receives the state every chunk starts from, [B*H][N][dk][dv]; o is
// then not written (the gradients need the states, not the outputs).
// tfrag: 128 x 128 heads under the gated delta rule keep every chunk's T diag(b) fragments in the
// workspace (MAP writes them, OUT reads them); the workspace must then be the size
// prefill_chunk_workspace(..., true) gives.  Same results either way.
hipError_t launch_prefill_chunk(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const float *g, const float *beta, const float *s0, float *o,
                                float *s_out, int B, int T, int H, int dk, int dv, int chunk,
                                bool delta, void *ws, hipStream_t stream,
                                float *chunk_states = nullptr, bool tfrag = false);
size_t prefill_chunk_workspace(int B, int T, int H, int dk, int dv, int chunk, bool tfrag = false);

// Packed variable-length sequences (bf16, MFMA shapes).  cu, slots and init are host
// arrays (cu[S + 1] token offsets; slots[S] pool slots, NULL = slot s, -1 = none;
// init[S] start-from-stored-state flags, NULL = all).  The workspace holds a table
// built from them, the piece maps and the piece start states.
struct VarlenLayout {
    int pc, NP, NM, chunk;   // chunks per piece, global pieces, global maps, chunk size
    int out_per_xcd;         // OUT's piece slots per XCD (ceil(NP / 8))
    size_t table_ints, maps_off, starts_off, bytes;
};
bool varlen_layout(const int *cu, int S, int H, int dk, int dv, int chunk, VarlenLayout *L);
hipError_t launch_prefill_chunk_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                       const float *g, const float *beta, const int *cu, int S,
                                       const int *slots, const int *init, float *pool, float *o,
                                       int H, int dk, int dv, int chunk, bool delta, void *ws,
                                       hipStream_t stream);

// Input preparation ahead of the mixer (gdn_prepare.hip): convolution, SiLU, q/k norm, gates.
// prepare_grid_blocks: workgroups one call launches (at most kMaxPrepareBlocks is accepted).
constexpr size_t kMaxPrepareBlocks = 0x7fffff00u;
size_t prepare_grid_blocks(int B, int T, int H, int dk, int dv);
hipError_t launch_prepare(const void *xq, const void *xk, const void *xv, const float *w,
                          const float *a_raw, const float *b_raw, const float *rate,
                          const float *bias, const float *state_in, float *state_out, void *q,
                          void *k, void *v, float *g, float *beta, int B, int T, int H, int dk,
                          int dv, gdn_dtype dt, hipStream_t stream);

// Packed sequences: cu [S+1], slot [S], init [S] are device arrays (validated on the host);
// each sequence's convolution starts from pool[slot] (init != 0, slot >= 0) or zeros and its
// new state is written back to pool[slot], by the same launch for a sequence that lies in one
// tile and by a second launch otherwise.  cu_host and slot_host: host copies of cu and slot.
hipError_t launch_prepare_varlen(const void *xq, const void *xk, const void *xv, const float *w,
                                 const float *a_raw, const float *b_raw, const float *rate,
                                 const float *bias, const int *cu, const int *slot, const int *init, int S,
                                 int T_total, float *pool, void *q, void *k, void *v, float *g,
                                 float *beta, int H, int dk, int dv, gdn_dtype dt, hipStream_t stream,
                                 const int *cu_host, const int *slot_host);

// Gradients of the chunked prefill (gdn_backward.hip): a forward pass keeping chunk start
// states, then per-chunk maps, a reverse scan of the state gradient and per-chunk gradients.
bool backward_supported(int dk, int dv, gdn_dtype dt);
int backward_chunk();
size_t backward_workspace(int B, int T, int H, int dk, int dv);
hipError_t launch_backward(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *s0, const float *d_o,
                           const float *ds_final, float *dq, float *dk, float *dv, float *dg,
                           float *dbeta, float *ds0, int B, int T, int H, int d_k, int d_v,
                           gdn_dtype dt, bool delta, void *ws, hipStream_t stream);

// Copies (or zero-fills, when s0 == NULL) a start state into s_out.
hipError_t launch_state_copy(const float *s0, float *s_out, size_t n, hipStream_t stream);

}  // namespace gdn
