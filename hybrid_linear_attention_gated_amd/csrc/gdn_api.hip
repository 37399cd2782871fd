// gdn_api.hip -- the C ABI of libgdn: argument validation and dispatch.
//
// Every check runs on the host before anything is queued, so a call that
// returns an error has no side effect.  The library keeps no state and
// allocates nothing; scratch memory comes from the caller.
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "gdn_internal.h"

namespace gdn {
namespace {

__global__ void state_copy_kernel(const float *__restrict__ src, float *__restrict__ dst, size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src ? src[i] : 0.f;
}

bool supported_dim(int d) { return d == 16 || d == 64 || d == 128; }
bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64; }
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};
Span span(const void *p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return {a, a + bytes};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

// element count of a product of non-negative ints, or SIZE_MAX on overflow
size_t prod(std::initializer_list<long long> xs) {
    unsigned __int128 acc = 1;
    for (long long x : xs) {
        acc *= static_cast<unsigned __int128>(x);
        if (acc > (static_cast<unsigned __int128>(1) << 60)) return SIZE_MAX;
    }
    return static_cast<size_t>(acc);
}

size_t elem_bytes(gdn_dtype dt) { return dt == GDN_BF16 ? 2 : 4; }

gdn_status check_prefill_shape(int B, int T, int H, int d_k, int d_v, int chunk, gdn_dtype dt) {
    if (B <= 0 || H <= 0 || T < 0 || d_k <= 0 || d_v <= 0 || chunk <= 0) return GDN_ERR_SHAPE;
    if (dt != GDN_F32 && dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!supported_dim(d_k) || !supported_dim(d_v) || !supported_chunk(chunk))
        return GDN_ERR_UNSUPPORTED;
    if (prod({B, T, H, d_k > d_v ? d_k : d_v}) == SIZE_MAX) return GDN_ERR_SHAPE;
    if (prod({B, H, 16}) > 0x7fffffffULL) return GDN_ERR_SHAPE;  // grid limits
    return GDN_OK;
}

}  // namespace

hipError_t launch_state_copy(const float *s0, float *s_out, size_t n, hipStream_t stream) {
    if (n == 0 || s0 == s_out) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(state_copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       s0, s_out, n);
    return hipGetLastError();
}

// the fused decode step from raw projections (gdn_decode_prep.hip)
bool prepare_decode_supported(int dk, int dv);
hipError_t launch_prepare_decode(const void *xq, const void *xk, const void *xv, const float *w,
                                 const float *a_raw, const float *b_raw, const float *rate,
                                 const float *bias, float *conv_state, float *state, float *o, int N,
                                 int H, int d, gdn_dtype dt, bool delta, hipStream_t stream);

}  // namespace gdn

using namespace gdn;

// Scratch of gdn_chunk_prefill_noalloc: the piece maps and start states the prefill otherwise
// keeps in the caller's workspace, in one array per GPU that the library holds until the
// process ends.  In host code `scratch` names a host-side stand-in, not device memory: host code
// only ever passes the address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxScratchDevices];  // device address of `scratch`, per device id

// The current device's copy of `scratch`, looked up once per device (with that device current).
gdn_status scratch_of_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return GDN_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GDN_ERR_HIP;
        g_scratch_dev[dev] = ptr;
    }
    *out = g_scratch_dev[dev];
    return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_version(void) { return GDN_ABI_VERSION; }

const char *gdn_status_string(gdn_status status) {
    switch (status) {
    case GDN_OK: return "GDN_OK: success";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: invalid or too large size argument";
    case GDN_ERR_UNSUPPORTED:
        return "GDN_ERR_UNSUPPORTED: d_k/d_v must be 16, 64 or 128, chunk 16, 32 or 64, dtype F32 or BF16, "
               "rule GATED_DELTA or GATED_DECAY";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: a pointer is not 16-byte aligned";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: an output buffer overlaps another buffer";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
    case GDN_ERR_HIP: return "GDN_ERR_HIP: the HIP runtime failed to queue work";
    case GDN_ERR_CAPTURE:
        return "GDN_ERR_CAPTURE: the stream is capturing a graph; packed-sequence calls copy host data "
               "and run eagerly only";
    }
    return "unknown gdn_status";
}

size_t gdn_chunk_prefill_workspace_size(int B, int T, int H, int d_k, int d_v, int chunk,
                                        gdn_dtype qkv_dtype) {
    if (check_prefill_shape(B, T, H, d_k, d_v, chunk, qkv_dtype) != GDN_OK || T == 0) return 0;
    if (qkv_dtype == GDN_BF16) return prefill_bf16_workspace(B, T, H, d_k, d_v, chunk);
    return 0;  // the fp32 path keeps everything on chip
}

namespace {

// The dense prefill.  tfrag: the workspace has room for the per-chunk T diag(b) fragments of
// 128 x 128 heads (the size gdn_chunk_prefill_workspace_size reports); the call without allocation
// runs from its smaller static scratch without them (same results).
gdn_status prefill_rule(gdn_rule rule, const void *q, const void *k, const void *v, const float *g,
                        const float *beta, const float *initial_state, float *o, float *final_state,
                        int B, int T, int H, int d_k, int d_v, int chunk, gdn_dtype qkv_dtype,
                        void *workspace, size_t workspace_bytes, void *stream, bool tfrag) {
    if (rule != GDN_RULE_GATED_DELTA && rule != GDN_RULE_GATED_DECAY) return GDN_ERR_UNSUPPORTED;
    const bool delta = rule == GDN_RULE_GATED_DELTA;
    gdn_status st = check_prefill_shape(B, T, H, d_k, d_v, chunk, qkv_dtype);
    if (st != GDN_OK) return st;
    if (!final_state) return GDN_ERR_NULL;
    if (T > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    const void *ptrs[] = {q, k, v, g, beta, initial_state, o, final_state, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;

    const size_t es = elem_bytes(qkv_dtype);
    const size_t state_bytes = prod({B, H, d_k, d_v}) * 4;
    const Span s_fin = span(final_state, state_bytes);
    const Span s_init = initial_state ? span(initial_state, state_bytes) : Span{0, 0};
    if (initial_state && initial_state != final_state && overlap(s_init, s_fin)) return GDN_ERR_ALIAS;

    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (T == 0) {
        if (workspace && overlap(span(workspace, workspace_bytes), s_fin)) return GDN_ERR_ALIAS;
        return launch_state_copy(initial_state, final_state, state_bytes / 4, hs) == hipSuccess
                   ? GDN_OK
                   : GDN_ERR_HIP;
    }

    const Span s_q = span(q, prod({B, T, H, d_k}) * es), s_k = span(k, prod({B, T, H, d_k}) * es);
    const Span s_v = span(v, prod({B, T, H, d_v}) * es);
    const Span s_g = span(g, prod({B, T, H}) * 4), s_b = span(beta, prod({B, T, H}) * 4);
    const Span s_o = span(o, prod({B, T, H, d_v}) * 4);
    const Span inputs[] = {s_q, s_k, s_v, s_g, s_b};
    for (const Span &in : inputs)
        if (overlap(s_o, in) || overlap(s_fin, in)) return GDN_ERR_ALIAS;
    if (overlap(s_o, s_init) || overlap(s_o, s_fin)) return GDN_ERR_ALIAS;

    const size_t need = qkv_dtype == GDN_BF16 ? prefill_bf16_workspace(B, T, H, d_k, d_v, chunk, tfrag) : 0;
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;
        const Span s_ws = span(workspace, need);
        const Span all[] = {s_q, s_k, s_v, s_g, s_b, s_init, s_o, s_fin};
        for (const Span &x : all)
            if (overlap(s_ws, x)) return GDN_ERR_ALIAS;
    }

    hipError_t err;
    if (qkv_dtype == GDN_BF16)
        err = launch_prefill_bf16(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                                  static_cast<const uint16_t *>(v), g, beta, initial_state, o,
                                  final_state, B, T, H, d_k, d_v, chunk, delta, workspace, hs, tfrag);
    else
        err = launch_prefill_valu(q, k, v, g, beta, initial_state, o, final_state, B, T, H, d_k,
                                  d_v, chunk, GDN_F32, delta, hs);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace

gdn_status gdn_chunk_prefill_rule(gdn_rule rule, const void *q, const void *k, const void *v,
                                  const float *g, const float *beta, const float *initial_state,
                                  float *o, float *final_state, int B, int T, int H, int d_k,
                                  int d_v, int chunk, gdn_dtype qkv_dtype, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return prefill_rule(rule, q, k, v, g, beta, initial_state, o, final_state, B, T, H, d_k, d_v,
                        chunk, qkv_dtype, workspace, workspace_bytes, stream, true);
}

gdn_status gdn_chunk_prefill_noalloc(gdn_rule rule, const void *q, const void *k, const void *v,
                                     const float *g, const float *beta, const float *initial_state,
                                     float *o, float *final_state, int B, int T, int H, int d_k,
                                     int d_v, int chunk, gdn_dtype qkv_dtype, void *stream) {
    // the checks of gdn_chunk_prefill_rule that do not involve the workspace come first, so a
    // bad call reports what the allocating call would report
    if (rule != GDN_RULE_GATED_DELTA && rule != GDN_RULE_GATED_DECAY) return GDN_ERR_UNSUPPORTED;
    const gdn_status st = check_prefill_shape(B, T, H, d_k, d_v, chunk, qkv_dtype);
    if (st != GDN_OK) return st;
    const size_t need = (qkv_dtype == GDN_BF16 && T > 0) ? prefill_bf16_workspace(B, T, H, d_k, d_v, chunk, false) : 0;
    if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        const gdn_status s2 = scratch_of_current_device(&ws);
        if (s2 != GDN_OK) return s2;
    }
    return prefill_rule(rule, q, k, v, g, beta, initial_state, o, final_state, B, T, H, d_k, d_v, chunk,
                        qkv_dtype, ws, need > 0 ? GDN_NOALLOC_SCRATCH_BYTES : 0, stream, false);
}

gdn_status gdn_chunk_prefill(const void *q, const void *k, const void *v, const float *g,
                             const float *beta, const float *initial_state, float *o,
                             float *final_state, int B, int T, int H, int d_k, int d_v, int chunk,
                             gdn_dtype qkv_dtype, void *workspace, size_t workspace_bytes,
                             void *stream) {
    return gdn_chunk_prefill_rule(GDN_RULE_GATED_DELTA, q, k, v, g, beta, initial_state, o,
                                  final_state, B, T, H, d_k, d_v, chunk, qkv_dtype, workspace,
                                  workspace_bytes, stream);
}

namespace {

// Host checks of a packed batch: offsets from 0 to T_total, never decreasing; slots in
// [-1, pool) and the valid ones distinct.  Returns GDN_OK or the error to report.
gdn_status check_varlen_batch(const int32_t *cu, int S, int T_total, const int32_t *slots, int pool) {
    if (S < 0 || T_total < 0 || pool < 0) return GDN_ERR_SHAPE;
    if (S == 0) return T_total == 0 ? GDN_OK : GDN_ERR_SHAPE;
    if (!cu) return GDN_ERR_NULL;
    if (cu[0] != 0 || cu[S] != T_total) return GDN_ERR_SHAPE;
    for (int s = 0; s < S; ++s)
        if (cu[s + 1] < cu[s]) return GDN_ERR_SHAPE;
    if (!slots) return pool >= S ? GDN_OK : GDN_ERR_SHAPE;
    std::vector<unsigned char> used(static_cast<size_t>(pool), 0);
    for (int s = 0; s < S; ++s) {
        const int32_t sl = slots[s];
        if (sl < -1 || sl >= pool) return GDN_ERR_SHAPE;
        if (sl >= 0) {
            if (used[sl]) return GDN_ERR_ALIAS;  // two sequences would write one state
            used[sl] = 1;
        }
    }
    return GDN_OK;
}

// The packed-sequence calls copy a host table into the workspace.  Recorded into a graph,
// that copy would keep a pointer to the table, which dies when the call returns: refuse a
// stream that is capturing, before anything is queued.
gdn_status check_not_capturing(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return GDN_ERR_HIP;
    return cs == hipStreamCaptureStatusNone ? GDN_OK : GDN_ERR_CAPTURE;
}

bool varlen_supported(int d_k, int d_v, int chunk, gdn_dtype dt) {
    return (dt == GDN_BF16 || dt == GDN_F32) && supported_dim(d_k) && supported_dim(d_v) && supported_chunk(chunk);
}

// bf16 inputs at the MFMA shapes run the chunk kernels with sequence pieces; fp32 inputs and the
// 16-wide shapes the fp32 VALU kernel, one workgroup per sequence, head and 16 value columns
bool varlen_mfma(int d_k, int d_v, int chunk, gdn_dtype dt) {
    return dt == GDN_BF16 && prefill_bf16_uses_mfma(d_k, d_v, chunk);
}

}  // namespace

size_t gdn_chunk_prefill_varlen_workspace_size(const int32_t *cu_seqlens, int S, int H, int d_k, int d_v,
                                               int chunk, gdn_dtype qkv_dtype) {
    if (S <= 0 || H <= 0 || !cu_seqlens || !varlen_supported(d_k, d_v, chunk, qkv_dtype)) return 0;
    if (check_varlen_batch(cu_seqlens, S, cu_seqlens[S], nullptr, S) != GDN_OK) return 0;
    if (!varlen_mfma(d_k, d_v, chunk, qkv_dtype)) return prefill_valu_varlen_workspace(S);
    // either rule (the size query takes no rule): the larger of the two plans
    size_t bytes = 0;
    for (bool delta : {true, false}) {
        VarlenLayout L;
        if (!varlen_layout(cu_seqlens, S, H, d_k, d_v, prefill_kernel_chunk(d_k, d_v, chunk, delta), &L)) return 0;
        bytes = L.bytes > bytes ? L.bytes : bytes;
    }
    return bytes;
}

gdn_status gdn_chunk_prefill_varlen(gdn_rule rule, const void *q, const void *k, const void *v,
                                    const float *g, const float *beta, const int32_t *cu_seqlens, int S,
                                    int T_total, float *state_pool, int pool_size, const int32_t *slots,
                                    const int32_t *has_initial, float *o, int H, int d_k, int d_v,
                                    int chunk, gdn_dtype qkv_dtype, void *workspace,
                                    size_t workspace_bytes, void *stream) {
    if (rule != GDN_RULE_GATED_DELTA && rule != GDN_RULE_GATED_DECAY) return GDN_ERR_UNSUPPORTED;
    if (H <= 0 || d_k <= 0 || d_v <= 0 || chunk <= 0) return GDN_ERR_SHAPE;
    if (!varlen_supported(d_k, d_v, chunk, qkv_dtype)) return GDN_ERR_UNSUPPORTED;
    gdn_status st = check_varlen_batch(cu_seqlens, S, T_total, slots, pool_size);
    if (st != GDN_OK) return st;
    if (prod({T_total, H, d_k > d_v ? d_k : d_v}) == SIZE_MAX || prod({pool_size, H, d_k, d_v}) == SIZE_MAX)
        return GDN_ERR_SHAPE;
    if (S == 0) return GDN_OK;
    if (T_total > 0 && (!q || !k || !v || !g || !beta || !o)) return GDN_ERR_NULL;
    bool any_slot = !slots;
    for (int s = 0; slots && s < S; ++s) any_slot = any_slot || slots[s] >= 0;
    if (any_slot && !state_pool) return GDN_ERR_NULL;
    const void *ptrs[] = {q, k, v, g, beta, state_pool, o, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;

    const size_t es = elem_bytes(qkv_dtype);
    const Span s_q = span(q, prod({T_total, H, d_k}) * es), s_k = span(k, prod({T_total, H, d_k}) * es);
    const Span s_v = span(v, prod({T_total, H, d_v}) * es);
    const Span s_g = span(g, prod({T_total, H}) * 4), s_b = span(beta, prod({T_total, H}) * 4);
    const Span s_o = span(o, prod({T_total, H, d_v}) * 4);
    const Span s_p = state_pool ? span(state_pool, prod({pool_size, H, d_k, d_v}) * 4) : Span{0, 0};
    const Span inputs[] = {s_q, s_k, s_v, s_g, s_b};
    for (const Span &in : inputs)
        if (overlap(s_o, in) || overlap(s_p, in)) return GDN_ERR_ALIAS;
    if (overlap(s_o, s_p)) return GDN_ERR_ALIAS;

    if (prod({S, H, 16}) > 0x7fffffffULL) return GDN_ERR_SHAPE;  // the VALU kernel's grid
    const bool mfma = varlen_mfma(d_k, d_v, chunk, qkv_dtype);
    const int kchunk = mfma ? prefill_kernel_chunk(d_k, d_v, chunk, rule == GDN_RULE_GATED_DELTA) : chunk;
    VarlenLayout L{};
    if (mfma) {
        if (!varlen_layout(cu_seqlens, S, H, d_k, d_v, kchunk, &L)) return GDN_ERR_SHAPE;
    } else {
        L.bytes = prefill_valu_varlen_workspace(S);
    }
    if (!workspace || workspace_bytes < L.bytes) return GDN_ERR_WORKSPACE;
    const Span s_ws = span(workspace, L.bytes);
    const Span all[] = {s_q, s_k, s_v, s_g, s_b, s_o, s_p};
    for (const Span &x : all)
        if (overlap(s_ws, x)) return GDN_ERR_ALIAS;
    st = check_not_capturing(static_cast<hipStream_t>(stream));
    if (st != GDN_OK) return st;

    const hipError_t err =
        mfma ? launch_prefill_chunk_varlen(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                                           static_cast<const uint16_t *>(v), g, beta, cu_seqlens, S, slots,
                                           has_initial, state_pool, o, H, d_k, d_v, kchunk,
                                           rule == GDN_RULE_GATED_DELTA, workspace, static_cast<hipStream_t>(stream))
             : launch_prefill_valu_varlen(q, k, v, g, beta, cu_seqlens, S, slots, has_initial, state_pool, o, H,
                                          d_k, d_v, chunk, qkv_dtype, rule == GDN_RULE_GATED_DELTA, workspace,
                                          static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

namespace {

// shared by the decode entry points: slots == NULL means sequence n owns state n (pool = N)
gdn_status decode_impl(gdn_rule rule, const void *q, const void *k, const void *v, const float *g,
                       const float *beta, float *state, const int32_t *slots, int pool, float *o,
                       int N, int H, int d_k, int d_v, gdn_dtype qkv_dtype, void *stream) {
    if (rule != GDN_RULE_GATED_DELTA && rule != GDN_RULE_GATED_DECAY) return GDN_ERR_UNSUPPORTED;
    if (N < 0 || H <= 0 || d_k <= 0 || d_v <= 0 || pool < 0) return GDN_ERR_SHAPE;
    if (qkv_dtype != GDN_F32 && qkv_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return GDN_ERR_UNSUPPORTED;
    // the decode grid has up to 8 wavefronts per (sequence, head) (128-wide states)
    if (prod({N, H, d_k, d_v}) == SIZE_MAX || prod({pool, H, d_k, d_v}) == SIZE_MAX ||
        prod({N, H, 8}) > 0x7fffffffULL)
        return GDN_ERR_SHAPE;
    if (N == 0) return GDN_OK;
    if (!q || !k || !v || !g || !beta || !o) return GDN_ERR_NULL;
    if ((!state && pool > 0) || (slots == nullptr && !state)) return GDN_ERR_NULL;
    const void *ptrs[] = {q, k, v, g, beta, state, o, slots};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;

    const size_t es = elem_bytes(qkv_dtype);
    const Span s_q = span(q, prod({N, H, d_k}) * es), s_k = span(k, prod({N, H, d_k}) * es);
    const Span s_v = span(v, prod({N, H, d_v}) * es);
    const Span s_g = span(g, prod({N, H}) * 4), s_b = span(beta, prod({N, H}) * 4);
    const Span s_s = state ? span(state, prod({pool, H, d_k, d_v}) * 4) : Span{0, 0};
    const Span s_o = span(o, prod({N, H, d_v}) * 4);
    const Span s_slot = slots ? span(slots, static_cast<size_t>(N) * 4) : Span{0, 0};
    const Span inputs[] = {s_q, s_k, s_v, s_g, s_b, s_slot};
    for (const Span &in : inputs)
        if (overlap(s_o, in) || overlap(s_s, in)) return GDN_ERR_ALIAS;
    if (overlap(s_o, s_s)) return GDN_ERR_ALIAS;

    const hipError_t err = launch_decode(q, k, v, g, beta, state, o, N, H, d_k, d_v, qkv_dtype,
                                         rule == GDN_RULE_GATED_DELTA, slots, pool,
                                         static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // namespace

gdn_status gdn_decode_step_rule(gdn_rule rule, const void *q, const void *k, const void *v,
                                const float *g, const float *beta, float *state, float *o, int N,
                                int H, int d_k, int d_v, gdn_dtype qkv_dtype, void *stream) {
    return decode_impl(rule, q, k, v, g, beta, state, nullptr, N, o, N, H, d_k, d_v, qkv_dtype, stream);
}

gdn_status gdn_decode_step_slots(gdn_rule rule, const void *q, const void *k, const void *v,
                                 const float *g, const float *beta, float *state_pool,
                                 const int32_t *slots, int pool_size, float *o, int N, int H,
                                 int d_k, int d_v, gdn_dtype qkv_dtype, void *stream) {
    if (N > 0 && !slots) return GDN_ERR_NULL;
    return decode_impl(rule, q, k, v, g, beta, state_pool, slots, pool_size, o, N, H, d_k, d_v,
                       qkv_dtype, stream);
}

gdn_status gdn_decode_step(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state, float *o, int N, int H, int d_k,
                           int d_v, gdn_dtype qkv_dtype, void *stream) {
    return gdn_decode_step_rule(GDN_RULE_GATED_DELTA, q, k, v, g, beta, state, o, N, H, d_k, d_v,
                                qkv_dtype, stream);
}

gdn_status gdn_prepare_decode_step(gdn_rule rule, const void *xq, const void *xk, const void *xv,
                                   const float *conv_weight, const float *a_raw, const float *b_raw,
                                   const float *decay_rate, const float *gate_bias, float *conv_state,
                                   float *state, float *o, int N, int H, int d_k, int d_v,
                                   gdn_dtype x_dtype, void *stream) {
    if (rule != GDN_RULE_GATED_DELTA && rule != GDN_RULE_GATED_DECAY) return GDN_ERR_UNSUPPORTED;
    if (N < 0 || H <= 0 || d_k <= 0 || d_v <= 0) return GDN_ERR_SHAPE;
    if (x_dtype != GDN_F32 && x_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!prepare_decode_supported(d_k, d_v)) return GDN_ERR_UNSUPPORTED;
    const long long C = static_cast<long long>(H) * (2 * d_k + d_v);
    if (prod({N, H, d_k, d_v}) == SIZE_MAX || prod({N, C, 3}) == SIZE_MAX || prod({N, H}) > 0x7fffffffULL)
        return GDN_ERR_SHAPE;
    if (N == 0) return GDN_OK;
    if (!xq || !xk || !xv || !conv_weight || !a_raw || !b_raw || !conv_state || !state || !o)
        return GDN_ERR_NULL;
    const void *ptrs[] = {xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias, conv_state, state, o};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    const size_t es = elem_bytes(x_dtype);
    const Span in[] = {span(xq, prod({N, H, d_k}) * es), span(xk, prod({N, H, d_k}) * es),
                       span(xv, prod({N, H, d_v}) * es), span(conv_weight, static_cast<size_t>(C) * 16),
                       span(a_raw, prod({N, H}) * 4), span(b_raw, prod({N, H}) * 4),
                       span(decay_rate, decay_rate ? static_cast<size_t>(H) * 4 : 0),
                       span(gate_bias, gate_bias ? static_cast<size_t>(H) * 4 : 0)};
    const Span out[] = {span(conv_state, prod({N, C, 3}) * 4), span(state, prod({N, H, d_k, d_v}) * 4),
                        span(o, prod({N, H, d_v}) * 4)};
    for (int i = 0; i < 3; ++i) {
        for (int j = i + 1; j < 3; ++j)
            if (overlap(out[i], out[j])) return GDN_ERR_ALIAS;
        for (const Span &x : in)
            if (overlap(out[i], x)) return GDN_ERR_ALIAS;
    }
    const hipError_t err = launch_prepare_decode(xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias,
                                                 conv_state, state, o, N, H, d_k, x_dtype,
                                                 rule == GDN_RULE_GATED_DELTA, static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

gdn_status gdn_prepare(const void *xq, const void *xk, const void *xv, const float *conv_weight,
                       const float *a_raw, const float *b_raw, const float *decay_rate,
                       const float *gate_bias, const float *conv_state_in, float *conv_state_out,
                       void *q, void *k, void *v, float *g, float *beta, int B, int T, int H,
                       int d_k, int d_v, gdn_dtype x_dtype, void *stream) {
    if (B <= 0 || H <= 0 || T < 0 || d_k <= 0 || d_v <= 0) return GDN_ERR_SHAPE;
    if (x_dtype != GDN_F32 && x_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return GDN_ERR_UNSUPPORTED;
    const long long C = static_cast<long long>(H) * (2 * d_k + d_v);
    if (prod({B, T, C}) == SIZE_MAX || C > (1LL << 28)) return GDN_ERR_SHAPE;
    if (prepare_grid_blocks(B, T, H, d_k, d_v) > kMaxPrepareBlocks) return GDN_ERR_SHAPE;
    if (!conv_weight) return GDN_ERR_NULL;
    if (T > 0 && (!xq || !xk || !xv || !a_raw || !b_raw || !q || !k || !v || !g || !beta))
        return GDN_ERR_NULL;
    const void *ptrs[] = {xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias,
                          conv_state_in, conv_state_out, q, k, v, g, beta};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;

    const size_t es = elem_bytes(x_dtype);
    const size_t nk = prod({B, T, H, d_k}) * es, nv = prod({B, T, H, d_v}) * es;
    const size_t ngate = prod({B, T, H}) * 4, nstate = prod({B, C, 3}) * 4;
    const Span in[] = {span(xq, xq ? nk : 0), span(xk, xk ? nk : 0), span(xv, xv ? nv : 0),
                       span(conv_weight, static_cast<size_t>(C) * 16), span(a_raw, a_raw ? ngate : 0),
                       span(b_raw, b_raw ? ngate : 0),
                       span(decay_rate, decay_rate ? static_cast<size_t>(H) * 4 : 0),
                       span(gate_bias, gate_bias ? static_cast<size_t>(H) * 4 : 0),
                       span(conv_state_in, conv_state_in ? nstate : 0)};
    const Span out[] = {span(q, q ? nk : 0), span(k, k ? nk : 0), span(v, v ? nv : 0),
                        span(g, g ? ngate : 0), span(beta, beta ? ngate : 0),
                        span(conv_state_out, conv_state_out ? nstate : 0)};
    const int n_out = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(out[i], out[j])) return GDN_ERR_ALIAS;
        for (const Span &x : in) {
            const bool same_state = i == n_out - 1 && x.lo == out[i].lo && x.hi == out[i].hi &&
                                    conv_state_in == conv_state_out;
            if (!same_state && overlap(out[i], x)) return GDN_ERR_ALIAS;
        }
    }
    if (T == 0 && !conv_state_out) return GDN_OK;
    const hipError_t err =
        launch_prepare(xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias, conv_state_in,
                       conv_state_out, q, k, v, g, beta, B, T, H, d_k, d_v, x_dtype,
                       static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

size_t gdn_prepare_chunk_prefill_workspace_size(int B, int T, int H, int d_k, int d_v, int chunk,
                                                gdn_dtype x_dtype) {
    if (B <= 0 || H <= 0 || T <= 0 || x_dtype != GDN_BF16 || !prepare_prefill_supported(d_k, d_v)) return 0;
    if (chunk != 32 && chunk != 64) return 0;
    if (prod({B, T, H, d_k}) == SIZE_MAX || prod({B, H, 16}) > 0x7fffffffULL) return 0;
    return prepare_prefill_workspace(B, T, H, d_k, d_v);
}

gdn_status gdn_prepare_chunk_prefill(gdn_rule rule, const void *xq, const void *xk, const void *xv,
                                     const float *conv_weight, const float *a_raw, const float *b_raw,
                                     const float *decay_rate, const float *gate_bias, const float *conv_state_in,
                                     float *conv_state_out, const float *initial_state, float *o,
                                     float *final_state, int B, int T, int H, int d_k, int d_v, int chunk,
                                     gdn_dtype x_dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (rule != GDN_RULE_GATED_DELTA && rule != GDN_RULE_GATED_DECAY) return GDN_ERR_UNSUPPORTED;
    if (B <= 0 || H <= 0 || T < 0 || d_k <= 0 || d_v <= 0 || chunk <= 0) return GDN_ERR_SHAPE;
    if (x_dtype != GDN_BF16 || !prepare_prefill_supported(d_k, d_v) || (chunk != 32 && chunk != 64))
        return GDN_ERR_UNSUPPORTED;
    const long long C = static_cast<long long>(H) * (2 * d_k + d_v);
    if (prod({B, T, H, d_k}) == SIZE_MAX || prod({B, H, 16}) > 0x7fffffffULL || prod({B, C, 3}) == SIZE_MAX ||
        C > (1LL << 28))
        return GDN_ERR_SHAPE;
    if (!final_state || !conv_weight) return GDN_ERR_NULL;
    if (T > 0 && (!xq || !xk || !xv || !a_raw || !b_raw || !o)) return GDN_ERR_NULL;
    const void *ptrs[] = {xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias, conv_state_in,
                          conv_state_out, initial_state, o, final_state, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;

    const size_t nk = prod({B, T, H, d_k}) * 2, nv = prod({B, T, H, d_v}) * 2, ng = prod({B, T, H}) * 4;
    const size_t ns = prod({B, H, d_k, d_v}) * 4, nw = prod({B, C, 3}) * 4;
    const Span s_init = initial_state ? span(initial_state, ns) : Span{0, 0};
    const Span s_cin = conv_state_in ? span(conv_state_in, nw) : Span{0, 0};
    const Span in[] = {span(xq, xq ? nk : 0), span(xk, xk ? nk : 0), span(xv, xv ? nv : 0),
                       span(conv_weight, static_cast<size_t>(C) * 16), span(a_raw, a_raw ? ng : 0),
                       span(b_raw, b_raw ? ng : 0), span(decay_rate, decay_rate ? static_cast<size_t>(H) * 4 : 0),
                       span(gate_bias, gate_bias ? static_cast<size_t>(H) * 4 : 0), s_cin, s_init};
    const size_t need = gdn_prepare_chunk_prefill_workspace_size(B, T, H, d_k, d_v, chunk, x_dtype);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
    const Span out[] = {span(o, o && T > 0 ? prod({B, T, H, d_v}) * 4 : 0), span(final_state, ns),
                        conv_state_out ? span(conv_state_out, nw) : Span{0, 0},
                        span(workspace, workspace ? need : 0)};
    const int n_out = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(out[i], out[j])) return GDN_ERR_ALIAS;
        for (const Span &x : in) {
            // the allowed in-place updates: final state over the start state, window over window
            const bool same = (i == 1 && initial_state == final_state && x.lo == s_init.lo && x.hi == s_init.hi) ||
                              (i == 2 && conv_state_in == conv_state_out && x.lo == s_cin.lo && x.hi == s_cin.hi);
            if (!same && overlap(out[i], x)) return GDN_ERR_ALIAS;
        }
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (T == 0 && launch_state_copy(initial_state, final_state, ns / 4, hs) != hipSuccess) return GDN_ERR_HIP;
    const hipError_t err = launch_prepare_prefill(
        static_cast<const uint16_t *>(xq), static_cast<const uint16_t *>(xk), static_cast<const uint16_t *>(xv),
        conv_weight, a_raw, b_raw, decay_rate, gate_bias, conv_state_in, conv_state_out, initial_state, o,
        final_state, B, T, H, d_k, d_v, rule == GDN_RULE_GATED_DELTA, workspace, hs);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

size_t gdn_chunk_backward_workspace_size(int B, int T, int H, int d_k, int d_v, gdn_dtype qkv_dtype) {
    if (B <= 0 || H <= 0 || T < 0 || !backward_supported(d_k, d_v, qkv_dtype)) return 0;
    if (prod({B, T, H, d_k}) == SIZE_MAX) return 0;
    return backward_workspace(B, T, H, d_k, d_v);
}

gdn_status gdn_chunk_backward(gdn_rule rule, const void *q, const void *k, const void *v,
                              const float *g, const float *beta, const float *initial_state,
                              const float *d_o, const float *d_final_state, float *dq, float *dk,
                              float *dv, float *dg, float *dbeta, float *d_initial_state, int B,
                              int T, int H, int d_k, int d_v, gdn_dtype qkv_dtype, void *workspace,
                              size_t workspace_bytes, void *stream) {
    if (rule != GDN_RULE_GATED_DELTA && rule != GDN_RULE_GATED_DECAY) return GDN_ERR_UNSUPPORTED;
    if (B <= 0 || H <= 0 || T < 0 || d_k <= 0 || d_v <= 0) return GDN_ERR_SHAPE;
    if (qkv_dtype != GDN_F32 && qkv_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!backward_supported(d_k, d_v, qkv_dtype)) return GDN_ERR_UNSUPPORTED;
    if (prod({B, T, H, d_k}) == SIZE_MAX) return GDN_ERR_SHAPE;
    const long long chunks = (static_cast<long long>(T) + backward_chunk() - 1) / backward_chunk();
    if (static_cast<long long>(B) * H * (chunks > 0 ? chunks : 1) > 0x7fffff00LL) return GDN_ERR_SHAPE;
    if (T > 0 && (!q || !k || !v || !g || !beta || !d_o || !dq || !dk || !dv || !dg || !dbeta))
        return GDN_ERR_NULL;
    const void *ptrs[] = {q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv, dg, dbeta,
                          d_initial_state, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    const size_t need = backward_workspace(B, T, H, d_k, d_v);
    if (need > 0 && (!workspace || workspace_bytes < need)) return GDN_ERR_WORKSPACE;

    const size_t es = elem_bytes(qkv_dtype);
    const size_t nk = prod({B, T, H, d_k}), nv = prod({B, T, H, d_v}), ng = prod({B, T, H});
    const size_t ns = prod({B, H, d_k, d_v}) * 4;
    const Span in[] = {span(q, q ? nk * es : 0), span(k, k ? nk * es : 0), span(v, v ? nv * es : 0),
                       span(g, g ? ng * 4 : 0), span(beta, beta ? ng * 4 : 0),
                       span(initial_state, initial_state ? ns : 0), span(d_o, d_o ? nv * 4 : 0),
                       span(d_final_state, d_final_state ? ns : 0)};
    const Span out[] = {span(dq, dq ? nk * 4 : 0), span(dk, dk ? nk * 4 : 0), span(dv, dv ? nv * 4 : 0),
                        span(dg, dg ? ng * 4 : 0), span(dbeta, dbeta ? ng * 4 : 0),
                        span(d_initial_state, d_initial_state ? ns : 0),
                        span(workspace, workspace ? need : 0)};
    const int n_out = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(out[i], out[j])) return GDN_ERR_ALIAS;
        for (const Span &x : in)
            if (overlap(out[i], x)) return GDN_ERR_ALIAS;
    }
    if (T == 0 && !d_initial_state) return GDN_OK;
    const hipError_t err = launch_backward(q, k, v, g, beta, initial_state, d_o, d_final_state, dq, dk, dv, dg,
                                           dbeta, d_initial_state, B, T, H, d_k, d_v, qkv_dtype,
                                           rule == GDN_RULE_GATED_DELTA, workspace,
                                           static_cast<hipStream_t>(stream));
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

size_t gdn_prepare_varlen_workspace_size(int S) {
    return S > 0 ? ((static_cast<size_t>(3) * S + 1) * 4 + 255) & ~static_cast<size_t>(255) : 0;
}

gdn_status gdn_prepare_varlen(const void *xq, const void *xk, const void *xv, const float *conv_weight,
                              const float *a_raw, const float *b_raw, const float *decay_rate,
                              const float *gate_bias, const int32_t *cu_seqlens, int S, int T_total,
                              float *conv_pool, int pool_size, const int32_t *slots,
                              const int32_t *has_initial, void *q, void *k, void *v, float *g, float *beta,
                              int H, int d_k, int d_v, gdn_dtype x_dtype, void *workspace,
                              size_t workspace_bytes, void *stream) {
    if (H <= 0 || d_k <= 0 || d_v <= 0) return GDN_ERR_SHAPE;
    if (x_dtype != GDN_F32 && x_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!supported_dim(d_k) || !supported_dim(d_v)) return GDN_ERR_UNSUPPORTED;
    gdn_status st = check_varlen_batch(cu_seqlens, S, T_total, slots, pool_size);
    if (st != GDN_OK) return st;
    const long long C = static_cast<long long>(H) * (2 * d_k + d_v);
    if (C > (1LL << 28) || prod({T_total, C}) == SIZE_MAX || prod({pool_size, C, 3}) == SIZE_MAX)
        return GDN_ERR_SHAPE;
    if (prepare_grid_blocks(1, T_total, H, d_k, d_v) > kMaxPrepareBlocks ||
        static_cast<unsigned long long>((C / 4 + 255) / 256) * S > kMaxPrepareBlocks)
        return GDN_ERR_SHAPE;
    if (S == 0) return GDN_OK;
    if (!conv_weight) return GDN_ERR_NULL;
    if (T_total > 0 && (!xq || !xk || !xv || !a_raw || !b_raw || !q || !k || !v || !g || !beta))
        return GDN_ERR_NULL;
    bool any_slot = !slots;
    for (int s = 0; slots && s < S; ++s) any_slot = any_slot || slots[s] >= 0;
    if (any_slot && !conv_pool) return GDN_ERR_NULL;
    const void *ptrs[] = {xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias, conv_pool,
                          q, k, v, g, beta, workspace};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_ALIGN;
    const size_t need = gdn_prepare_varlen_workspace_size(S);
    if (!workspace || workspace_bytes < need) return GDN_ERR_WORKSPACE;

    const size_t es = elem_bytes(x_dtype);
    const size_t nk = prod({T_total, H, d_k}) * es, nv = prod({T_total, H, d_v}) * es;
    const size_t ngate = prod({T_total, H}) * 4, npool = prod({pool_size, C, 3}) * 4;
    const Span in[] = {span(xq, xq ? nk : 0), span(xk, xk ? nk : 0), span(xv, xv ? nv : 0),
                       span(conv_weight, static_cast<size_t>(C) * 16), span(a_raw, a_raw ? ngate : 0),
                       span(b_raw, b_raw ? ngate : 0),
                       span(decay_rate, decay_rate ? static_cast<size_t>(H) * 4 : 0),
                       span(gate_bias, gate_bias ? static_cast<size_t>(H) * 4 : 0)};
    const Span out[] = {span(q, q ? nk : 0), span(k, k ? nk : 0), span(v, v ? nv : 0),
                        span(g, g ? ngate : 0), span(beta, beta ? ngate : 0),
                        span(conv_pool, conv_pool ? npool : 0), span(workspace, need)};
    const int n_out = sizeof(out) / sizeof(out[0]);
    for (int i = 0; i < n_out; ++i) {
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(out[i], out[j])) return GDN_ERR_ALIAS;
        for (const Span &x : in)
            if (overlap(out[i], x)) return GDN_ERR_ALIAS;
    }

    st = check_not_capturing(static_cast<hipStream_t>(stream));
    if (st != GDN_OK) return st;

    // the batch table (offsets, slots, start flags) into the workspace, then the kernels
    std::vector<int32_t> table(static_cast<size_t>(3) * S + 1);
    for (int s = 0; s <= S; ++s) table[s] = cu_seqlens[s];
    for (int s = 0; s < S; ++s) {
        table[S + 1 + s] = slots ? slots[s] : s;
        table[2 * S + 1 + s] = has_initial ? (has_initial[s] != 0) : 1;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    int32_t *dt = static_cast<int32_t *>(workspace);
    if (hipMemcpyAsync(dt, table.data(), table.size() * 4, hipMemcpyHostToDevice, hs) != hipSuccess)
        return GDN_ERR_HIP;
    const hipError_t err = launch_prepare_varlen(xq, xk, xv, conv_weight, a_raw, b_raw, decay_rate, gate_bias,
                                                 dt, dt + S + 1, dt + 2 * S + 1, S, T_total, conv_pool, q, k,
                                                 v, g, beta, H, d_k, d_v, x_dtype, hs, table.data(),
                                                 table.data() + S + 1);
    return err == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

}  // extern "C"
