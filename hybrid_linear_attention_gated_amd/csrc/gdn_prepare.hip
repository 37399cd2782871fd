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

#ifndef GDN_PREP_CPT
#define GDN_PREP_CPT 4
#endif
#ifndef GDN_PREP_UNROLL
#define GDN_PREP_UNROLL 8
#endif
#ifndef GDN_PREP_TILE
#define GDN_PREP_TILE 32
#endif

constexpr int kCpt = GDN_PREP_CPT;        // adjacent channels per thread
constexpr int kTile = GDN_PREP_TILE;      // tokens per convolution workgroup
constexpr int kUnroll = GDN_PREP_UNROLL;  // tokens whose loads are issued together
constexpr int kCols = 256;                // threads (channel columns) per workgroup
constexpr int kGateEl = 4;                // gate elements per thread
constexpr int kXcd = 8;
constexpr float kEps = 1e-6f;
constexpr float kLog2e = 1.4426950408889634f;
static_assert(kCpt == 4 || kCpt == 8, "channels per thread");
static_assert(kTile % kUnroll == 0 && kTile >= 3, "tile");

struct PrepArgs {
    const void *xq, *xk, *xv;
    const float *w;           // [C, 4]
    const float *a_raw, *b_raw, *rate, *bias;
    const float *state_in;    // [B, C, 3] or null
    float *state_out;         // [B, C, 3] or null
    void *q, *k, *v;
    float *g, *beta;
    int B, T, H, dv;
    int C, ncol;              // channels, C / kCpt
    int slabs, tiles;         // convolution workgroups = slabs * B * tiles
    int tile_len;             // packed sequences: tokens per convolution workgroup (dense: kTile)
    int conv_blocks, gate_blocks, per_xcd;
    int state_in_kernel;      // 1: the last tile writes state_out
    // packed sequences (B = 1, T = all tokens): sequence s is tokens cu[s] .. cu[s+1]-1 and
    // starts from pool[slot[s]] when init[s] != 0 and slot[s] >= 0, else from zeros
    const int *cu, *slot, *init;
    int S;
    float *pool;              // [pool][C][3]
    int spanning;             // host: some sequence with a slot spans tiles or is empty
};

// The three raw inputs before a position (oldest first) of kCpt channels, from a state row
// [C][3] at channel ch; zeros for a NULL row.
__device__ __forceinline__ void read_window(const float *sp, float (&x3)[kCpt], float (&x2)[kCpt],
                                            float (&x1)[kCpt]) {
    float st[3 * kCpt];  // kCpt channels x 3 taps, channel-major
#pragma unroll
    for (int i = 0; i < 3 * kCpt / 4; ++i) {
        const float4 u = sp ? reinterpret_cast<const float4 *>(sp)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        st[4 * i] = u.x; st[4 * i + 1] = u.y; st[4 * i + 2] = u.z; st[4 * i + 3] = u.w;
    }
#pragma unroll
    for (int j = 0; j < kCpt; ++j) { x3[j] = st[3 * j]; x2[j] = st[3 * j + 1]; x1[j] = st[3 * j + 2]; }
}
__device__ __forceinline__ void write_window(float *sp, const float (&x3)[kCpt], const float (&x2)[kCpt],
                                             const float (&x1)[kCpt]) {
    float st[3 * kCpt];
#pragma unroll
    for (int j = 0; j < kCpt; ++j) { st[3 * j] = x3[j]; st[3 * j + 1] = x2[j]; st[3 * j + 2] = x1[j]; }
#pragma unroll
    for (int i = 0; i < 3 * kCpt / 4; ++i)
        reinterpret_cast<float4 *>(sp)[i] = make_float4(st[4 * i], st[4 * i + 1], st[4 * i + 2], st[4 * i + 3]);
}

// Packed sequences: the sequence holding token t (the last s with cu[s] <= t), and its start
// state row at channel ch (NULL = zeros).
__device__ __forceinline__ int seq_of(const PrepArgs &a, int t) {
    int lo = 0, hi = a.S;  // cu[lo] <= t < cu[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (a.cu[mid] <= t) lo = mid;
        else hi = mid;
    }
    return lo;
}
// A non-empty packed sequence [cs, ce) inside one tile (prepare_kernel writes its new state)
__host__ __device__ __forceinline__ bool single_tile(const PrepArgs &a, int cs, int ce) {
    return ce > cs && cs / a.tile_len == (ce - 1) / a.tile_len;
}
__device__ __forceinline__ const float *start_row(const PrepArgs &a, int s, int ch) {
    const int sl = a.slot[s];
    return (sl >= 0 && a.init[s]) ? a.pool + (static_cast<size_t>(sl) * a.C + ch) * 3 : nullptr;
}

// kCpt stored values as raw 32-bit words (bf16 pairs or fp32), and their fp32 widening
template <typename TIn> struct Raw {
    static constexpr int kWords = kCpt * static_cast<int>(sizeof(TIn)) / 4;
    uint32_t w[kWords];
};
template <typename TIn> __device__ __forceinline__ Raw<TIn> load_raw(const TIn *p) {
    Raw<TIn> r;
    if constexpr (Raw<TIn>::kWords == 2) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        r.w[0] = u.x; r.w[1] = u.y;
    } else {
#pragma unroll
        for (int i = 0; i < Raw<TIn>::kWords / 4; ++i) {
            const uint4 u = reinterpret_cast<const uint4 *>(p)[i];
            r.w[4 * i] = u.x; r.w[4 * i + 1] = u.y; r.w[4 * i + 2] = u.z; r.w[4 * i + 3] = u.w;
        }
    }
    return r;
}
__device__ __forceinline__ void widen(const Raw<uint16_t> &r, float (&x)[kCpt]) {
#pragma unroll
    for (int i = 0; i < kCpt / 2; ++i) { x[2 * i] = lo_half_f32(r.w[i]); x[2 * i + 1] = hi_half_f32(r.w[i]); }
}
__device__ __forceinline__ void widen(const Raw<float> &r, float (&x)[kCpt]) {
#pragma unroll
    for (int i = 0; i < kCpt; ++i) x[i] = __uint_as_float(r.w[i]);
}
__device__ __forceinline__ void store_out(float *p, const float (&x)[kCpt]) {
#pragma unroll
    for (int i = 0; i < kCpt / 4; ++i)
        reinterpret_cast<float4 *>(p)[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
}
__device__ __forceinline__ void store_out(uint16_t *p, const float (&x)[kCpt]) {
    if constexpr (kCpt == 4) {
        *reinterpret_cast<uint2 *>(p) = make_uint2(cvt2_bf16(x[0], x[1]), cvt2_bf16(x[2], x[3]));
    } else {
        *reinterpret_cast<uint4 *>(p) = make_uint4(cvt2_bf16(x[0], x[1]), cvt2_bf16(x[2], x[3]),
                                                   cvt2_bf16(x[4], x[5]), cvt2_bf16(x[6], x[7]));
    }
}

__device__ __forceinline__ float silu(float c) {
    // c / (1 + e^-c); e^-c overflows to +inf for c < -88 and the quotient goes to -0
    return c * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-c * kLog2e));
}

// v plus the value of another lane, picked by a DPP lane pattern (all lanes active)
template <int CTRL> __device__ __forceinline__ float dpp_plus(float v) {
    return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// sum over aligned groups of G adjacent lanes, left in every lane of the group
template <int G> __device__ __forceinline__ float group_sum(float v) {
    if constexpr (G >= 2) v = dpp_plus<0xB1>(v);    // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (G >= 4) v = dpp_plus<0x4E>(v);    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (G >= 8) v = dpp_plus<0x141>(v);   // row_half_mirror: the other quad of the 8
    if constexpr (G >= 16) v = dpp_plus<0x140>(v);  // row_mirror: the other 8 of the row
    if constexpr (G >= 32) v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));  // lane ^ 16
    static_assert(G <= 32, "group");
    return v;
}

// this thread's tensor, position and row stride, from its first channel in the q|k|v space
template <typename TIn> struct Route {
    const TIn *x;
    TIn *y;
    int rs;
    bool norm;
};
template <int DK, typename TIn> __device__ __forceinline__ Route<TIn> route(const PrepArgs &a, int ch) {
    const int HK = a.H * DK;
    if (ch < HK) return {static_cast<const TIn *>(a.xq) + ch, static_cast<TIn *>(a.q) + ch, HK, true};
    if (ch < 2 * HK)
        return {static_cast<const TIn *>(a.xk) + (ch - HK), static_cast<TIn *>(a.k) + (ch - HK), HK, true};
    return {static_cast<const TIn *>(a.xv) + (ch - 2 * HK), static_cast<TIn *>(a.v) + (ch - 2 * HK), a.H * a.dv,
            false};
}

// VL: packed sequences (the window restarts at every sequence start; the new state of a
// sequence inside one tile is written here, that of any other by a second launch).
template <int DK, typename TIn, bool VL>
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
    const int ch = kCpt * col;
    Route<TIn> r = route<DK, TIn>(a, ch);
    const size_t row0 = static_cast<size_t>(b) * a.T;
    r.x += row0 * r.rs;
    r.y += row0 * r.rs;

    float wt[4][kCpt];  // wt[i][j]: tap i of channel ch + j
#pragma unroll
    for (int j = 0; j < kCpt; ++j) {
        const float4 u = *reinterpret_cast<const float4 *>(a.w + static_cast<size_t>(ch + j) * 4);
        wt[0][j] = u.x; wt[1][j] = u.y; wt[2][j] = u.z; wt[3][j] = u.w;
    }

    const int len = VL ? a.tile_len : kTile;
    const int t0 = tile * len;
    const int t1 = min(t0 + len, a.T);
    float x3[kCpt], x2[kCpt], x1[kCpt];  // inputs at t-3, t-2, t-1
    int sq = 0, seq_end = a.T;           // packed: the current sequence and its end
    if (VL) {
        sq = seq_of(a, t0);
        const int cs = a.cu[sq];
        seq_end = a.cu[sq + 1];
        // the window before t0: earlier tokens of the sequence, else entries of its start state
        // (position p < cs is entry 3 - (cs - p), oldest first)
        const int back = t0 - cs;  // tokens of the sequence before t0 (0, 1, 2 or >= 3)
        if (back < 3) {
            read_window(start_row(a, sq, ch), x3, x2, x1);  // the start state ...
            // ... shifted by the sequence's own tokens before t0
            for (int p = cs; p < t0; ++p) {
                float xp[kCpt];
                widen(load_raw(r.x + static_cast<size_t>(p) * r.rs), xp);
#pragma unroll
                for (int j = 0; j < kCpt; ++j) { x3[j] = x2[j]; x2[j] = x1[j]; x1[j] = xp[j]; }
            }
        } else {
            widen(load_raw(r.x + static_cast<size_t>(t0 - 3) * r.rs), x3);
            widen(load_raw(r.x + static_cast<size_t>(t0 - 2) * r.rs), x2);
            widen(load_raw(r.x + static_cast<size_t>(t0 - 1) * r.rs), x1);
        }
    } else if (t0 == 0) {
        if (a.state_in) {
            float st[3 * kCpt];  // kCpt channels x 3 taps, channel-major
            const float *sp = a.state_in + (static_cast<size_t>(b) * a.C + ch) * 3;
#pragma unroll
            for (int i = 0; i < 3 * kCpt / 4; ++i) {
                const float4 u = reinterpret_cast<const float4 *>(sp)[i];
                st[4 * i] = u.x; st[4 * i + 1] = u.y; st[4 * i + 2] = u.z; st[4 * i + 3] = u.w;
            }
#pragma unroll
            for (int j = 0; j < kCpt; ++j) { x3[j] = st[3 * j]; x2[j] = st[3 * j + 1]; x1[j] = st[3 * j + 2]; }
        } else {
#pragma unroll
            for (int j = 0; j < kCpt; ++j) x3[j] = x2[j] = x1[j] = 0.f;
        }
    } else {
        widen(load_raw(r.x + static_cast<size_t>(t0 - 3) * r.rs), x3);
        widen(load_raw(r.x + static_cast<size_t>(t0 - 2) * r.rs), x2);
        widen(load_raw(r.x + static_cast<size_t>(t0 - 1) * r.rs), x1);
    }

    for (int tb = t0; tb < t1; tb += kUnroll) {
        Raw<TIn> raw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (tb + u < t1) raw[u] = load_raw(r.x + static_cast<size_t>(tb + u) * r.rs);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (tb + u >= t1) break;  // uniform across the workgroup
            if (VL && tb + u == seq_end) {  // a new sequence starts: its start state (uniform)
                do {
                    ++sq;
                } while (a.cu[sq + 1] <= tb + u);  // past empty sequences (cu[S] = T ends it)
                seq_end = a.cu[sq + 1];
                read_window(start_row(a, sq, ch), x3, x2, x1);
            }
            float xt[kCpt], y[kCpt];
            widen(raw[u], xt);
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < kCpt; ++j) {
                const float c = fmaf(wt[3][j], xt[j], fmaf(wt[2][j], x1[j], fmaf(wt[1][j], x2[j], wt[0][j] * x3[j])));
                y[j] = silu(c);
                ss = fmaf(y[j], y[j], ss);
            }
            ss = group_sum<DK / kCpt>(ss);
            const float rn = r.norm ? __builtin_amdgcn_rsqf(ss + kEps) : 1.f;
#pragma unroll
            for (int j = 0; j < kCpt; ++j) {
                y[j] *= rn;
                x3[j] = x2[j]; x2[j] = x1[j]; x1[j] = xt[j];
            }
            store_out(r.y + static_cast<size_t>(tb + u) * r.rs, y);
            // a sequence that lies wholly in this tile: its new state, the window after its last
            // token (no other workgroup reads its start state)
            if (VL && tb + u + 1 == seq_end && a.cu[sq] >= t0 && a.slot[sq] >= 0)
                write_window(a.pool + (static_cast<size_t>(a.slot[sq]) * a.C + ch) * 3, x3, x2, x1);
        }
    }

    if (!VL && a.state_in_kernel && t1 == a.T && a.state_out) {  // last tile: the window is the new state
        float st[3 * kCpt];
#pragma unroll
        for (int j = 0; j < kCpt; ++j) { st[3 * j] = x3[j]; st[3 * j + 1] = x2[j]; st[3 * j + 2] = x1[j]; }
        float *sp = a.state_out + (static_cast<size_t>(b) * a.C + ch) * 3;
#pragma unroll
        for (int i = 0; i < 3 * kCpt / 4; ++i)
            reinterpret_cast<float4 *>(sp)[i] = make_float4(st[4 * i], st[4 * i + 1], st[4 * i + 2], st[4 * i + 3]);
    }
}

// Packed sequences that span tiles, or are empty: the new state (the last three raw inputs of
// [start state, its tokens]) into the sequence's pool slot, after prepare_kernel has read the
// start states.
template <int DK, typename TIn>
__global__ __launch_bounds__(kCols) void conv_state_varlen_kernel(PrepArgs a) {
    const int s = static_cast<int>(blockIdx.x / a.slabs);
    const int col = static_cast<int>(blockIdx.x % a.slabs) * kCols + threadIdx.x;
    const int cs = a.cu[s], ce = a.cu[s + 1];
    if (col >= a.ncol || a.slot[s] < 0 || single_tile(a, cs, ce)) return;
    const int ch = kCpt * col;
    const Route<TIn> r = route<DK, TIn>(a, ch);
    float x3[kCpt], x2[kCpt], x1[kCpt];
    const int p0 = ce - cs < 3 ? cs : ce - 3;  // first token in the final window
    if (ce - cs < 3) read_window(start_row(a, s, ch), x3, x2, x1);
    for (int p = p0; p < ce; ++p) {  // shift in the sequence's last (up to) three tokens
        float xp[kCpt];
        widen(load_raw(r.x + static_cast<size_t>(p) * r.rs), xp);
#pragma unroll
        for (int j = 0; j < kCpt; ++j) { x3[j] = x2[j]; x2[j] = x1[j]; x1[j] = xp[j]; }
    }
    write_window(a.pool + (static_cast<size_t>(a.slot[s]) * a.C + ch) * 3, x3, x2, x1);
}

// New convolution state from the last three tokens (T >= 3), for calls whose
// state is updated in place and spans several tiles: run after prepare_kernel,
// which has then finished reading the old state.
template <int DK, typename TIn>
__global__ __launch_bounds__(kCols) void conv_state_tail_kernel(PrepArgs a) {
    const int col = static_cast<int>(blockIdx.x % a.slabs) * kCols + threadIdx.x;
    const int b = static_cast<int>(blockIdx.x / a.slabs);
    if (col >= a.ncol) return;
    const int ch = kCpt * col;
    Route<TIn> r = route<DK, TIn>(a, ch);
    const TIn *x = r.x + (static_cast<size_t>(b) * a.T + a.T - 3) * r.rs;
    float x3[kCpt], x2[kCpt], x1[kCpt];
    widen(load_raw(x), x3);
    widen(load_raw(x + r.rs), x2);
    widen(load_raw(x + 2 * static_cast<size_t>(r.rs)), x1);
    write_window(a.state_out + (static_cast<size_t>(b) * a.C + ch) * 3, x3, x2, x1);
}

template <int DK, typename TIn> hipError_t run(PrepArgs &a, hipStream_t stream) {
    const int grid = a.per_xcd * kXcd;
    if (a.cu) {
        if (a.conv_blocks + a.gate_blocks > 0)
            hipLaunchKernelGGL((prepare_kernel<DK, TIn, true>), dim3(grid), dim3(kCols), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || !a.pool || a.S == 0 || !a.spanning) return e;
        hipLaunchKernelGGL((conv_state_varlen_kernel<DK, TIn>), dim3(a.slabs * a.S), dim3(kCols), 0, stream, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((prepare_kernel<DK, TIn, false>), dim3(grid), dim3(kCols), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.state_in_kernel || !a.state_out) return e;
    hipLaunchKernelGGL((conv_state_tail_kernel<DK, TIn>), dim3(a.slabs * a.B), dim3(kCols), 0, stream, a);
    return hipGetLastError();
}

template <typename F> hipError_t dispatch(int dk, gdn_dtype dt, PrepArgs &a, hipStream_t stream) {
    const bool bf = dt == GDN_BF16;
    switch (dk) {
    case 16: return bf ? run<16, uint16_t>(a, stream) : run<16, float>(a, stream);
    case 64: return bf ? run<64, uint16_t>(a, stream) : run<64, float>(a, stream);
    case 128: return bf ? run<128, uint16_t>(a, stream) : run<128, float>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t prepare_grid_blocks(int B, int T, int H, int dk, int dv) {
    const size_t ncol = static_cast<size_t>(H) * (2 * dk + dv) / kCpt;
    const size_t slabs = (ncol + kCols - 1) / kCols;
    const size_t tiles = T > 0 ? (static_cast<size_t>(T) + kTile - 1) / kTile : 1;
    const size_t gates = (static_cast<size_t>(B) * T * H + kCols * kGateEl - 1) / (kCols * kGateEl);
    return slabs * B * tiles + gates;
}

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
    a.C = H * (2 * dk + dv);
    a.ncol = a.C / kCpt;
    a.slabs = (a.ncol + kCols - 1) / kCols;
    a.tiles = T > 0 ? (T + kTile - 1) / kTile : 1;  // T = 0: one empty tile carries the state over
    const size_t conv = static_cast<size_t>(a.slabs) * B * a.tiles;
    const size_t gates = prepare_grid_blocks(B, T, H, dk, dv) - conv;
    if (conv + gates > kMaxPrepareBlocks) return hipErrorInvalidValue;
    a.conv_blocks = static_cast<int>(conv);
    a.gate_blocks = static_cast<int>(gates);
    a.per_xcd = static_cast<int>((conv + gates + kXcd - 1) / kXcd);
    // in place over several tiles: the first tile still reads the old state, so a second
    // launch writes the new one
    a.state_in_kernel = !(state_in && state_in == state_out && a.tiles > 1);
    return dispatch<void>(dk, dt, a, stream);
}

hipError_t launch_prepare_varlen(const void *xq, const void *xk, const void *xv, const float *w,
                                 const float *a_raw, const float *b_raw, const float *rate,
                                 const float *bias, const int *cu, const int *slot, const int *init, int S,
                                 int T_total, float *pool, void *q, void *k, void *v, float *g,
                                 float *beta, int H, int dk, int dv, gdn_dtype dt, hipStream_t stream,
                                 const int *cu_host, const int *slot_host) {
    PrepArgs a{};
    a.xq = xq; a.xk = xk; a.xv = xv; a.w = w;
    a.a_raw = a_raw; a.b_raw = b_raw; a.rate = rate; a.bias = bias;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.cu = cu; a.slot = slot; a.init = init; a.S = S; a.pool = pool;
    a.B = 1; a.T = T_total; a.H = H; a.dv = dv;
    a.C = H * (2 * dk + dv);
    a.ncol = a.C / kCpt;
    a.slabs = (a.ncol + kCols - 1) / kCols;
    // Tiles as long as the mean sequence (a power of two up to kTile): a batch of one-token
    // decode sequences gets one workgroup per token and channel slab rather than one per 32
    // tokens.  No empty tile: an empty sequence's state is written by the second launch.
    a.tile_len = kTile;
    while (a.tile_len > 1 && S > 0 && static_cast<long long>(a.tile_len / 2) * S >= T_total) a.tile_len /= 2;
    a.tiles = (T_total + a.tile_len - 1) / a.tile_len;
    for (int s = 0; s < S && !a.spanning; ++s)
        a.spanning = slot_host[s] >= 0 && !single_tile(a, cu_host[s], cu_host[s + 1]);
    const size_t conv = static_cast<size_t>(a.slabs) * a.tiles;
    const size_t gates = (static_cast<size_t>(T_total) * H + kCols * kGateEl - 1) / (kCols * kGateEl);
    if (conv + gates > kMaxPrepareBlocks || static_cast<size_t>(a.slabs) * S > kMaxPrepareBlocks)
        return hipErrorInvalidValue;
    a.conv_blocks = static_cast<int>(conv);
    a.gate_blocks = static_cast<int>(gates);
    a.per_xcd = static_cast<int>((conv + gates + kXcd - 1) / kXcd);
    return dispatch<void>(dk, dt, a, stream);
}

}  // namespace gdn
