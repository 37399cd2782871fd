// gdn_prepare.hip -- the input preparation ahead of the mixer, in one pass.
//
// The GDN block feeds the mixer through a short causal convolution and gate
// and decay parameters (ftxj.github.io digest of arXiv 2604.24715, Method:
// these start from random values when an attention layer is converted).  The
// form computed here, per token t, head h and channel c:
//
//   conv   c_t = w[c,0] x_{t-3} + w[c,1] x_{t-2} + w[c,2] x_{t-1} + w[c,3] x_t
//          (depthwise, width 4; the three inputs before the first token come
//          from a carried state, or are zero)
//   q, k   silu(c) / sqrt(|silu(c)|^2 + 1e-6), the norm over the head's d_k channels
//   v      silu(c)
//   g      -A_h softplus(a_t + bias_h)
//   beta   sigmoid(b_t)
//
// Memory-bound: each raw value is read once (plus a three-token halo per
// tile) and each result written once.  A thread owns four adjacent channels of
// the concatenated q|k|v channel space and walks a tile of tokens, keeping the
// last three inputs in registers; the d_k/4 adjacent lanes that hold one head's
// q (or k) row sum their squares with cross-lane adds.  Workgroups after the
// convolution ones turn the gate logits into g and beta.
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int kTile = 64;    // tokens per convolution workgroup
constexpr int kCols = 256;   // channel columns (4 channels each) per workgroup
constexpr int kGateEl = 4;   // gate elements per thread
constexpr int kUnroll = 8;   // tokens whose loads are issued together
constexpr int kXcd = 8;
constexpr float kEps = 1e-6f;
constexpr float kLog2e = 1.4426950408889634f;

struct PrepArgs {
    const void *xq, *xk, *xv;
    const float *w;           // [C, 4]
    const float *a_raw, *b_raw, *rate, *bias;
    const float *state_in;    // [B, C, 3] or null
    float *state_out;         // [B, C, 3] or null
    void *q, *k, *v;
    float *g, *beta;
    int B, T, H, dv;
    int ncol;                 // C / 4
    int slabs, tiles;         // convolution workgroups = slabs * B * tiles
    int conv_blocks, gate_blocks, per_xcd;
    int state_in_kernel;      // 1: the last tile writes state_out
};

__device__ __forceinline__ float4 load4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ float4 load4(const uint16_t *p) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    return make_float4(lo_half_f32(u.x), hi_half_f32(u.x), lo_half_f32(u.y), hi_half_f32(u.y));
}
__device__ __forceinline__ void store4(float *p, float4 x) { *reinterpret_cast<float4 *>(p) = x; }
__device__ __forceinline__ void store4(uint16_t *p, float4 x) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(cvt2_bf16(x.x, x.y), cvt2_bf16(x.z, x.w));
}

__device__ __forceinline__ float silu(float c) {
    // c / (1 + e^-c); e^-c overflows to +inf for c < -88 and the quotient goes to -0
    return c * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-c * kLog2e));
}

template <int G> __device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int m = 1; m < G; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

template <int DK, typename TIn>
__global__ __launch_bounds__(kCols) void prepare_kernel(PrepArgs a) {
    const int w = static_cast<int>(blockIdx.x % kXcd) * a.per_xcd + static_cast<int>(blockIdx.x / kXcd);
    if (w >= a.conv_blocks + a.gate_blocks) return;
    const int tid = threadIdx.x;

    if (w >= a.conv_blocks) {  // gate logits -> g, beta
        const size_t n = static_cast<size_t>(a.B) * a.T * a.H;
        const size_t e0 = (static_cast<size_t>(w - a.conv_blocks) * kCols + tid) * kGateEl;
#pragma unroll
        for (int u = 0; u < kGateEl; ++u) {
            const size_t e = e0 + u;
            if (e >= n) break;
            const int h = static_cast<int>(e % a.H);
            const float z = a.a_raw[e] + (a.bias ? a.bias[h] : 0.f);
            const float sp = fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
            a.g[e] = -(a.rate ? a.rate[h] : 1.f) * sp;
            a.beta[e] = 1.f / (1.f + expf(-a.b_raw[e]));
        }
        return;
    }

    // convolution workgroup: (slab, b, tile), tile fastest so neighbouring tiles share an XCD
    const int tile = w % a.tiles;
    const int b = (w / a.tiles) % a.B;
    const int slab = w / (a.tiles * a.B);
    const int col = slab * kCols + tid;
    if (col >= a.ncol) return;  // whole cross-lane groups drop out together
    const int ch = 4 * col;
    const int HK = a.H * DK;

    const TIn *x;
    TIn *y;
    int rs;       // row stride (elements) of this thread's tensor
    bool norm;
    if (ch < HK) {
        x = static_cast<const TIn *>(a.xq) + ch; y = static_cast<TIn *>(a.q) + ch; rs = HK; norm = true;
    } else if (ch < 2 * HK) {
        x = static_cast<const TIn *>(a.xk) + (ch - HK); y = static_cast<TIn *>(a.k) + (ch - HK); rs = HK; norm = true;
    } else {
        x = static_cast<const TIn *>(a.xv) + (ch - 2 * HK); y = static_cast<TIn *>(a.v) + (ch - 2 * HK);
        rs = a.H * a.dv; norm = false;
    }
    const size_t row0 = static_cast<size_t>(b) * a.T;
    x += row0 * rs;
    y += row0 * rs;

    float4 wt[4];  // wt[j] = taps of channel ch + j
#pragma unroll
    for (int j = 0; j < 4; ++j) wt[j] = load4(a.w + static_cast<size_t>(ch + j) * 4);

    const int t0 = tile * kTile;
    const int t1 = min(t0 + kTile, a.T);
    float4 x3, x2, x1;  // inputs at t-3, t-2, t-1
    if (t0 == 0) {
        if (a.state_in) {
            const float *s = a.state_in + (static_cast<size_t>(b) * a.ncol * 4 + ch) * 3;
            const float4 p = load4(s), q = load4(s + 4), r = load4(s + 8);  // 4 channels x 3 taps
            x3 = make_float4(p.x, p.w, q.z, r.y);
            x2 = make_float4(p.y, q.x, q.w, r.z);
            x1 = make_float4(p.z, q.y, r.x, r.w);
        } else {
            x3 = x2 = x1 = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else {
        x3 = load4(x + static_cast<size_t>(t0 - 3) * rs);
        x2 = load4(x + static_cast<size_t>(t0 - 2) * rs);
        x1 = load4(x + static_cast<size_t>(t0 - 1) * rs);
    }

    for (int tb = t0; tb < t1; tb += kUnroll) {
        float4 xs[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            xs[u] = tb + u < t1 ? load4(x + static_cast<size_t>(tb + u) * rs) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (tb + u >= t1) break;  // uniform across the workgroup
            const float4 xt = xs[u];
            float4 c;
            c.x = fmaf(wt[0].w, xt.x, fmaf(wt[0].z, x1.x, fmaf(wt[0].y, x2.x, wt[0].x * x3.x)));
            c.y = fmaf(wt[1].w, xt.y, fmaf(wt[1].z, x1.y, fmaf(wt[1].y, x2.y, wt[1].x * x3.y)));
            c.z = fmaf(wt[2].w, xt.z, fmaf(wt[2].z, x1.z, fmaf(wt[2].y, x2.z, wt[2].x * x3.z)));
            c.w = fmaf(wt[3].w, xt.w, fmaf(wt[3].z, x1.w, fmaf(wt[3].y, x2.w, wt[3].x * x3.w)));
            float4 s = make_float4(silu(c.x), silu(c.y), silu(c.z), silu(c.w));
            const float ss = group_sum<DK / 4>(s.x * s.x + s.y * s.y + s.z * s.z + s.w * s.w);
            const float r = norm ? __builtin_amdgcn_rsqf(ss + kEps) : 1.f;
            s.x *= r; s.y *= r; s.z *= r; s.w *= r;
            store4(y + static_cast<size_t>(tb + u) * rs, s);
            x3 = x2; x2 = x1; x1 = xt;
        }
    }

    if (a.state_in_kernel && t1 == a.T && a.state_out) {  // last tile: the window is the new state
        float *s = a.state_out + (static_cast<size_t>(b) * a.ncol * 4 + ch) * 3;
        store4(s, make_float4(x3.x, x2.x, x1.x, x3.y));
        store4(s + 4, make_float4(x2.y, x1.y, x3.z, x2.z));
        store4(s + 8, make_float4(x1.z, x3.w, x2.w, x1.w));
    }
}

// New convolution state from the last three tokens (T >= 3), for calls whose
// state is updated in place and spans several tiles: run after prepare_kernel,
// which has then finished reading the old state.
template <typename TIn>
__global__ __launch_bounds__(kCols) void conv_state_tail_kernel(PrepArgs a, int DK) {
    const int col = static_cast<int>(blockIdx.x % a.slabs) * kCols + threadIdx.x;
    const int b = static_cast<int>(blockIdx.x / a.slabs);
    if (col >= a.ncol) return;
    const int ch = 4 * col;
    const int HK = a.H * DK;
    const TIn *x;
    int rs;
    if (ch < HK) { x = static_cast<const TIn *>(a.xq) + ch; rs = HK; }
    else if (ch < 2 * HK) { x = static_cast<const TIn *>(a.xk) + (ch - HK); rs = HK; }
    else { x = static_cast<const TIn *>(a.xv) + (ch - 2 * HK); rs = a.H * a.dv; }
    x += (static_cast<size_t>(b) * a.T + a.T - 3) * rs;
    const float4 x3 = load4(x), x2 = load4(x + rs), x1 = load4(x + 2 * static_cast<size_t>(rs));
    float *s = a.state_out + (static_cast<size_t>(b) * a.ncol * 4 + ch) * 3;
    store4(s, make_float4(x3.x, x2.x, x1.x, x3.y));
    store4(s + 4, make_float4(x2.y, x1.y, x3.z, x2.z));
    store4(s + 8, make_float4(x1.z, x3.w, x2.w, x1.w));
}

template <int DK, typename TIn> hipError_t run(PrepArgs &a, hipStream_t stream) {
    const int grid = a.per_xcd * kXcd;
    hipLaunchKernelGGL((prepare_kernel<DK, TIn>), dim3(grid), dim3(kCols), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.state_in_kernel || !a.state_out) return e;
    hipLaunchKernelGGL((conv_state_tail_kernel<TIn>), dim3(a.slabs * a.B), dim3(kCols), 0, stream, a, DK);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prepare(const void *xq, const void *xk, const void *xv, const float *w,
                          const float *a_raw, const float *b_raw, const float *rate,
                          const float *bias, const float *state_in, float *state_out, void *q,
                          void *k, void *v, float *g, float *beta, int B, int T, int H, int dk,
                          int dv, gdn_dtype dt, hipStream_t stream) {
    PrepArgs a{};
    a.xq = xq; a.xk = xk; a.xv = xv; a.w = w;
    a.a_raw = a_raw; a.b_raw = b_raw; a.rate = rate; a.bias = bias;
    a.state_in = state_in; a.state_out = state_out;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.B = B; a.T = T; a.H = H; a.dv = dv;
    a.ncol = H * (2 * dk + dv) / 4;
    a.slabs = (a.ncol + kCols - 1) / kCols;
    a.tiles = T > 0 ? (T + kTile - 1) / kTile : 1;  // T = 0: one empty tile carries the state over
    const size_t conv = static_cast<size_t>(a.slabs) * B * a.tiles;
    const size_t gates = (static_cast<size_t>(B) * T * H + kCols * kGateEl - 1) / (kCols * kGateEl);
    if (conv + gates > 0x7fffffffULL - kXcd) return hipErrorInvalidValue;
    a.conv_blocks = static_cast<int>(conv);
    a.gate_blocks = static_cast<int>(gates);
    a.per_xcd = static_cast<int>((conv + gates + kXcd - 1) / kXcd);
    // in place over several tiles: the first tile still reads the old state, so a second
    // launch writes the new one
    a.state_in_kernel = !(state_in && state_in == state_out && a.tiles > 1);
    const bool bf = dt == GDN_BF16;
    switch (dk) {
    case 16: return bf ? run<16, uint16_t>(a, stream) : run<16, float>(a, stream);
    case 64: return bf ? run<64, uint16_t>(a, stream) : run<64, float>(a, stream);
    case 128: return bf ? run<128, uint16_t>(a, stream) : run<128, float>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdn
