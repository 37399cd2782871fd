// gdn_decode_prep.hip -- one decode step from the raw projections: the input
// preparation ahead of the mixer and the state update in one kernel (gfx950).
//
// A serving loop runs, for every generated token, the preparation (causal
// depthwise convolution of width 4 over each raw q, k and v channel with the
// carried window, SiLU, L2 norm of each head's q and k, g = -A_h softplus(a +
// bias_h), beta = sigmoid(b)) and then the decode step of the rule.  Per
// (sequence, head) the preparation touches d_k + d_k + d_v channels and two
// logits, so one workgroup per (sequence, head) can do both: the prepared q,
// k, v never leave LDS, and one launch replaces two.  The arithmetic is that of
// the two separate kernels, except the order in which a head's squared norm is
// summed and that the prepared values stay in fp32 (the separate preparation
// stores them as bf16 for bf16 inputs): no rounding to the storage type sits
// between the preparation and the update.
//
// The convolution and gates follow the short convolution and gate/decay
// parameters a converted GDN block keeps (ftxj.github.io digest of arXiv
// 2604.24715, Method); the update is the decode step of the gated delta rule
// (or the gated-decay rule without the erase term).
//
// Layout, d_k = d_v = 64: workgroup = 2 wavefronts = one (sequence, head).
// Wavefront 0 prepares the q and v channels, wavefront 1 the two gates and the
// k channels (one channel per lane); then each wavefront updates one 32-column
// half of the state (32 state floats per lane, as the decode kernel).
// d_k = d_v = 128: workgroup = 4 wavefronts.  Wavefronts 0-1 prepare the q and
// v channels, 2-3 the k channels and the gates (each head's q and k norm adds
// two wavefronts' partial sums through LDS); then, as the decode kernel does
// for these states, each wavefront takes 32 key rows of whole 128-column rows
// (64 state floats per lane) and the four add their partial u, p through LDS.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kWave = 64;
constexpr int kD = 64;          // d_k = d_v
constexpr int kWC = 32;         // state columns per wavefront
constexpr int kLPR = kWC / 4;   // lanes per key row (one float4 each)
constexpr int kRG = kWave / kLPR;
constexpr int kRows = kD / kRG; // key rows per lane
constexpr float kEps = 1e-6f;
constexpr float kLog2e = 1.4426950408889634f;

struct PrepDecodeArgs {
    const void *xq, *xk, *xv;
    const float *w;                    // [C, 4]
    const float *a_raw, *b_raw;        // [N, H]
    const float *rate, *bias;          // [H] or NULL
    float *conv_state;                 // [N, C, 3], updated in place
    float *state;                      // [N, H, d_k, d_v], updated in place
    float *o;                          // [N, H, d_v]
    int H;
    float scale;
};

// Causal convolution of one channel over [window, x] (taps oldest first), SiLU; the
// window moves on by one token in place.
__device__ __forceinline__ float conv_silu(const float *w4, float *win, float x) {
    const float4 w = *reinterpret_cast<const float4 *>(w4);
    const float s0 = win[0], s1 = win[1], s2 = win[2];
    const float c = fmaf(w.w, x, fmaf(w.z, s2, fmaf(w.y, s1, w.x * s0)));
    win[0] = s1;
    win[1] = s2;
    win[2] = x;
    return c * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-c * kLog2e));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

template <typename TIn, bool DELTA>
__global__ __launch_bounds__(2 * kWave) void prep_decode_kernel(PrepDecodeArgs a) {
    __shared__ float qs[kD], ks[kD], vs[kD], gb[2];
    const size_t nh = blockIdx.x;  // n * H + h
    const int n = static_cast<int>(nh / a.H), h = static_cast<int>(nh % a.H);
    const int wave = static_cast<int>(threadIdx.x) / kWave, lane = static_cast<int>(threadIdx.x) % kWave;
    const int HK = a.H * kD, C = 3 * HK;
    float *cs = a.conv_state + static_cast<size_t>(n) * C * 3;

    // ---- preparation: one channel per lane
    if (wave == 0) {
        const int cq = h * kD + lane, cv = 2 * HK + h * kD + lane;
        const float yq = conv_silu(a.w + static_cast<size_t>(cq) * 4, cs + static_cast<size_t>(cq) * 3,
                                   load_in(static_cast<const TIn *>(a.xq), nh * kD + lane));
        const float yv = conv_silu(a.w + static_cast<size_t>(cv) * 4, cs + static_cast<size_t>(cv) * 3,
                                   load_in(static_cast<const TIn *>(a.xv), nh * kD + lane));
        qs[lane] = yq * __builtin_amdgcn_rsqf(wave_sum(yq * yq) + kEps);
        vs[lane] = yv;
    } else {
        if (lane == 0) {
            const float z = a.a_raw[nh] + (a.bias ? a.bias[h] : 0.f);
            const float sp = fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
            gb[0] = -(a.rate ? a.rate[h] : 1.f) * sp;
            gb[1] = 1.f / (1.f + expf(-a.b_raw[nh]));
        }
        const int ck = HK + h * kD + lane;
        const float yk = conv_silu(a.w + static_cast<size_t>(ck) * 4, cs + static_cast<size_t>(ck) * 3,
                                   load_in(static_cast<const TIn *>(a.xk), nh * kD + lane));
        ks[lane] = yk * __builtin_amdgcn_rsqf(wave_sum(yk * yk) + kEps);
    }
    __syncthreads();

    // ---- the decode step on this wavefront's 32 state columns
    const int c = lane % kLPR, rg = lane / kLPR;
    const int col = wave * kWC + 4 * c, row0 = rg * kRows;
    const float ga = gb[0], b = gb[1];
    const float av = __expf(ga);
    float *st = a.state + nh * kD * kD;
    // the state streams through with non-temporal hints, as in the plain decode step
    f32x4 s[kRows];
#pragma unroll
    for (int m = 0; m < kRows; ++m) s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(st + (row0 + m) * kD + col));
    f32x4 u = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < kRows; ++m) {
        const float kr = ks[row0 + m], qr = qs[row0 + m];
        u += s[m] * kr;
        p += s[m] * qr;
        kq += kr * qr;
    }
#pragma unroll
    for (int off = kLPR; off < kWave; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[e] += __shfl_xor(u[e], off, kWave);
            p[e] += __shfl_xor(p[e], off, kWave);
        }
        kq += __shfl_xor(kq, off, kWave);
    }
    const f32x4 vv = {vs[col], vs[col + 1], vs[col + 2], vs[col + 3]};
    const f32x4 delta = DELTA ? b * (vv - av * u) : b * vv;
    if (rg == 0) *reinterpret_cast<f32x4 *>(a.o + nh * kD + col) = a.scale * (av * p + delta * kq);
#pragma unroll
    for (int m = 0; m < kRows; ++m)
        __builtin_nontemporal_store(av * s[m] + delta * ks[row0 + m], reinterpret_cast<f32x4 *>(st + (row0 + m) * kD + col));
}

// d_k = d_v = 128 (layout above)
constexpr int kD2 = 128;
constexpr int kLPR2 = kD2 / 4;          // lanes per key row: whole 128-column rows
constexpr int kRG2 = kWave / kLPR2;     // 2 key-row groups per wavefront
constexpr int kRows2 = 32 / kRG2;       // 16 key rows per lane (32 per wavefront)

template <typename TIn, bool DELTA>
__global__ __launch_bounds__(4 * kWave) void prep_decode_kernel128(PrepDecodeArgs a) {
    __shared__ float qs[kD2], ks[kD2], vs[kD2], gb[2], nrm[4];
    __shared__ f32x4 xu[4][kLPR2], xp[4][kLPR2];
    __shared__ float xkq[4];
    const size_t nh = blockIdx.x;  // n * H + h
    const int n = static_cast<int>(nh / a.H), h = static_cast<int>(nh % a.H);
    const int tid = static_cast<int>(threadIdx.x);
    const int wave = tid / kWave, lane = tid % kWave;
    const int HK = a.H * kD2, C = 3 * HK;
    float *cs = a.conv_state + static_cast<size_t>(n) * C * 3;

    // ---- preparation: threads 0-127 a q and a v channel, 128-255 a k channel
    const int ch = tid % kD2;
    float y;  // q (threads < 128) or k, before the norm
    if (tid < kD2) {
        const int cq = h * kD2 + ch, cv = 2 * HK + h * kD2 + ch;
        y = conv_silu(a.w + static_cast<size_t>(cq) * 4, cs + static_cast<size_t>(cq) * 3,
                      load_in(static_cast<const TIn *>(a.xq), nh * kD2 + ch));
        vs[ch] = conv_silu(a.w + static_cast<size_t>(cv) * 4, cs + static_cast<size_t>(cv) * 3,
                           load_in(static_cast<const TIn *>(a.xv), nh * kD2 + ch));
    } else {
        if (tid == kD2) {
            const float z = a.a_raw[nh] + (a.bias ? a.bias[h] : 0.f);
            const float sp = fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
            gb[0] = -(a.rate ? a.rate[h] : 1.f) * sp;
            gb[1] = 1.f / (1.f + expf(-a.b_raw[nh]));
        }
        const int ck = HK + h * kD2 + ch;
        y = conv_silu(a.w + static_cast<size_t>(ck) * 4, cs + static_cast<size_t>(ck) * 3,
                      load_in(static_cast<const TIn *>(a.xk), nh * kD2 + ch));
    }
    const float part = wave_sum(y * y);
    if (lane == 0) nrm[wave] = part;
    __syncthreads();
    const int w0 = wave & ~1;  // the two wavefronts of this tensor, added in one order
    const float rn = __builtin_amdgcn_rsqf(nrm[w0] + nrm[w0 + 1] + kEps);
    if (tid < kD2) qs[ch] = y * rn;
    else ks[ch] = y * rn;
    __syncthreads();

    // ---- the decode step: this wavefront's 32 key rows of whole 128-column rows
    const int c = lane % kLPR2, rg = lane / kLPR2;
    const int col = 4 * c, row0 = wave * 32 + rg * kRows2;
    const float ga = gb[0], b = gb[1];
    const float av = __expf(ga);
    float *st = a.state + nh * kD2 * kD2;
    f32x4 s[kRows2];
#pragma unroll
    for (int m = 0; m < kRows2; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(st + (row0 + m) * kD2 + col));
    f32x4 u = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < kRows2; ++m) {
        const float kr = ks[row0 + m], qr = qs[row0 + m];
        u += s[m] * kr;
        p += s[m] * qr;
        kq += kr * qr;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        u[e] += __shfl_xor(u[e], kLPR2, kWave);
        p[e] += __shfl_xor(p[e], kLPR2, kWave);
    }
    kq += __shfl_xor(kq, kLPR2, kWave);
    // the other wavefronts' key rows, through LDS; every wavefront adds them in one order
    if (rg == 0) {
        xu[wave][c] = u;
        xp[wave][c] = p;
        if (c == 0) xkq[wave] = kq;
    }
    __syncthreads();
    u = xu[0][c];
    p = xp[0][c];
    kq = xkq[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
        u += xu[w][c];
        p += xp[w][c];
        kq += xkq[w];
    }
    const f32x4 vv = {vs[col], vs[col + 1], vs[col + 2], vs[col + 3]};
    const f32x4 delta = DELTA ? b * (vv - av * u) : b * vv;
    if (wave == 0 && rg == 0) *reinterpret_cast<f32x4 *>(a.o + nh * kD2 + col) = a.scale * (av * p + delta * kq);
#pragma unroll
    for (int m = 0; m < kRows2; ++m)
        __builtin_nontemporal_store(av * s[m] + delta * ks[row0 + m],
                                    reinterpret_cast<f32x4 *>(st + (row0 + m) * kD2 + col));
}

}  // namespace

bool prepare_decode_supported(int dk, int dv) { return dk == dv && (dk == kD || dk == kD2); }

hipError_t launch_prepare_decode(const void *xq, const void *xk, const void *xv, const float *w,
                                 const float *a_raw, const float *b_raw, const float *rate,
                                 const float *bias, float *conv_state, float *state, float *o, int N,
                                 int H, int d, gdn_dtype dt, bool delta, hipStream_t stream) {
    PrepDecodeArgs a{xq, xk, xv, w, a_raw, b_raw, rate, bias, conv_state, state, o, H,
                     1.0f / sqrtf(static_cast<float>(d))};
    const dim3 grid(static_cast<unsigned>(static_cast<long long>(N) * H)), block(2 * kWave);
    if (d == kD2) {
        const dim3 block4(4 * kWave);
        if (dt == GDN_BF16) {
            if (delta) hipLaunchKernelGGL((prep_decode_kernel128<uint16_t, true>), grid, block4, 0, stream, a);
            else hipLaunchKernelGGL((prep_decode_kernel128<uint16_t, false>), grid, block4, 0, stream, a);
        } else {
            if (delta) hipLaunchKernelGGL((prep_decode_kernel128<float, true>), grid, block4, 0, stream, a);
            else hipLaunchKernelGGL((prep_decode_kernel128<float, false>), grid, block4, 0, stream, a);
        }
        return hipGetLastError();
    }
    if (dt == GDN_BF16) {
        if (delta) hipLaunchKernelGGL((prep_decode_kernel<uint16_t, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((prep_decode_kernel<uint16_t, false>), grid, block, 0, stream, a);
    } else {
        if (delta) hipLaunchKernelGGL((prep_decode_kernel<float, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((prep_decode_kernel<float, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace gdn
