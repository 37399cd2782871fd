// gdn_decode.hip -- single-token GDN step for a batch of sequences (gfx950).
//
// One token of the gated delta rule per (sequence, head), applied to the
// stored fp32 state in place (the step the HyLo serving runs repeat for every
// generated token at a cost that does not grow with context: ftxj.github.io
// digest of arXiv 2604.24715, Figure 5; we0.ai Priming article, SSM
// comparison: same compute budget per token).  With u = S k and p = S q,
//
//     delta = b (v - a u)
//     S'    = a S + delta k^T                (= a S (I - b k k^T) + b v k^T)
//     o     = S' q / sqrt(d_k) = (a p + delta (k . q)) / sqrt(d_k)
//
// Without the erase term (DELTA = false, S' = a S + b v k^T) delta = b v and
// u is not needed; the readout and update formulas are unchanged.
//
// States may live in a pool indexed by a per-sequence slot (continuous
// batching: a serving engine keeps one fixed-size state per live request and
// batches whichever requests are decoding; the Priming article lists
// continuous batching among its serving plugin's features).  A slot outside
// [0, pool_size) marks a padding entry: its output is zero, no state is touched.
//
// The step is bound by HBM bandwidth: every state byte is read once and
// written once, ~0.25 FLOP per byte, so there is no MFMA here.  Layout of the
// work: a wavefront owns a column slice of one (sequence, head) state stored
// key-major [d_k][d_v]; each lane holds float4 columns of a contiguous block
// of key rows in registers, so the column sums u, p reduce over key rows with
// a few cross-lane xor shuffles, and the state is loaded and stored with
// fully coalesced 16-byte accesses exactly once.  Value columns evolve
// independently, so slices need no exchange; slices of at most 32 state
// floats per lane (d = 64: two wavefronts per state) keep seven wavefronts
// per SIMD resident, and two-wavefront workgroups spread them evenly.  On
// 256 sequences x 32 heads x 64 x 64 that ran the step in 43-44 us against
// 47 us for one wavefront per state with 64 floats per lane, four
// wavefronts per workgroup; a plain in-place scale of the same 128 MiB takes
// 41 us.
//
// The state is read and written with non-temporal (streaming) hints: a step touches each state
// byte once, and a serving loop cycles through every layer's states, far more than the 256 MB
// last-level cache holds.  Over eight 128 MiB states in rotation (every access from DRAM) the
// step reached 66% of HBM peak without the hints and 75% with them; with one 128 MiB state
// stepped back to back (cache-resident) 81% without and 74% with.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 2;
// wavefronts per workgroup: 128-wide keys split a slice's key rows over four of them
template <int DK> constexpr int kWPB = DK == 128 ? 4 : kWavesPerBlock;

template <int DK, int DV>
struct DecodeShape {
    // 128-wide keys: the four wavefronts of a workgroup split a slice's key rows (32 each) and
    // add their partial sums through LDS, so a slice can span whole 128-column rows (512-byte
    // segments, 64 state floats per lane).  On 256 x 24 states of 128 x 128 (402 MB, far above
    // the last-level cache), with the streaming hints below: 74% of HBM peak, against 70% for
    // 64-column slices and 69-70% for eight wavefronts or two-way splits; 16-column slices of
    // whole columns read and wrote half cache lines (61% without the hints).
    static constexpr int KSPLIT = DK == 128 ? 4 : 1;
    static constexpr int KR = DK / KSPLIT;  // key rows per wavefront
    // columns per wavefront: keep at most 32 state floats per lane
    static constexpr int WC = KSPLIT > 1 ? DV : ((2048 / DK < DV) ? 2048 / DK : DV);
    static constexpr int SLICES = DV / WC;
    static constexpr int LPR = WC / 4;       // lanes per key row (one float4 each)
    static constexpr int RG = kWave / LPR;   // key-row groups per wavefront
    static constexpr int ROWS = KR / RG;     // key rows per lane
    static_assert(WC % 4 == 0 && kWave % LPR == 0 && KR % RG == 0, "decode tiling");
    static_assert(KSPLIT == 1 || KSPLIT == kWPB<DK>, "a split spans one workgroup");

};

template <int DK, int DV, typename TIn, bool DELTA>
__global__ __launch_bounds__(kWave * kWPB<DK>) void decode_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ state,
    float *__restrict__ o, int items, float scale, const int *__restrict__ slots, int H, int pool) {
    using S = DecodeShape<DK, DV>;
    const int lane = threadIdx.x % kWave;
    // work item: one (sequence, head, column slice); with split key rows a workgroup's
    // wavefronts share one item (half = which key rows), else each wavefront has its own
    const int half = S::KSPLIT > 1 ? static_cast<int>(threadIdx.x) / kWave : 0;
    const int item = S::KSPLIT > 1 ? static_cast<int>(blockIdx.x)
                                   : static_cast<int>(blockIdx.x) * kWPB<DK> + static_cast<int>(threadIdx.x) / kWave;
    if (item >= items) return;  // the whole wavefront (with split rows: the whole workgroup) exits together
    const int slice = item % S::SLICES;
    const size_t nh = static_cast<size_t>(item / S::SLICES);  // n * H + h

    const int c = lane % S::LPR;   // float4 column index inside the slice
    const int rg = lane / S::LPR;  // key-row group
    const int col = slice * S::WC + 4 * c;
    const int row0 = half * S::KR + rg * S::ROWS;

    size_t sh = nh;  // state index: (slot * H + h) when states live in a pool
    if (slots) {
        const int n = static_cast<int>(nh / H), h = static_cast<int>(nh % H);
        const int slot = slots[n];  // the same for the whole wavefront
        if (slot < 0 || slot >= pool) {  // uniform over the workgroup's item
            if (half == 0 && rg == 0) *reinterpret_cast<f32x4 *>(o + nh * DV + col) = f32x4{0.f, 0.f, 0.f, 0.f};
            return;
        }
        sh = static_cast<size_t>(slot) * H + h;
    }

    const float a = __expf(g[nh]);
    const float b = beta[nh];

    float *st = state + sh * DK * DV;
    f32x4 s[S::ROWS];
#pragma unroll
    for (int m = 0; m < S::ROWS; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(st + static_cast<size_t>(row0 + m) * DV + col));

    float kr[S::ROWS], qr[S::ROWS];
#pragma unroll
    for (int m = 0; m < S::ROWS; ++m) {
        kr[m] = load_in(k, nh * DK + row0 + m);
        qr[m] = load_in(q, nh * DK + row0 + m);
    }

    f32x4 u = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < S::ROWS; ++m) {
        u += s[m] * kr[m];
        p += s[m] * qr[m];
        kq += kr[m] * qr[m];
    }
    // reduce over the key-row groups (lanes that share a column)
#pragma unroll
    for (int off = S::LPR; off < kWave; off <<= 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[e] += __shfl_xor(u[e], off, kWave);
            p[e] += __shfl_xor(p[e], off, kWave);
        }
        kq += __shfl_xor(kq, off, kWave);
    }
    if constexpr (S::KSPLIT > 1) {
        // the other key rows' partial sums, through LDS; both wavefronts add them in the same
        // order, so they hold the same totals
        __shared__ f32x4 xu[S::KSPLIT][S::LPR], xp[S::KSPLIT][S::LPR];
        __shared__ float xkq[S::KSPLIT];
        if (rg == 0) {
            xu[half][c] = u;
            xp[half][c] = p;
            if (c == 0) xkq[half] = kq;
        }
        __syncthreads();
        u = xu[0][c];
        p = xp[0][c];
        kq = xkq[0];
#pragma unroll
        for (int hh = 1; hh < S::KSPLIT; ++hh) {
            u += xu[hh][c];
            p += xp[hh][c];
            kq += xkq[hh];
        }
    }

    f32x4 vv;
#pragma unroll
    for (int e = 0; e < 4; ++e) vv[e] = load_in(v, nh * DV + col + e);
    const f32x4 delta = DELTA ? b * (vv - a * u) : b * vv;

    if (half == 0 && rg == 0) {
        const f32x4 out = scale * (a * p + delta * kq);
        *reinterpret_cast<f32x4 *>(o + nh * DV + col) = out;
    }
#pragma unroll
    for (int m = 0; m < S::ROWS; ++m)
        __builtin_nontemporal_store(a * s[m] + delta * kr[m],
                                    reinterpret_cast<f32x4 *>(st + static_cast<size_t>(row0 + m) * DV + col));
}

template <int DK, int DV, typename TIn>
hipError_t launch_decode_t(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state, float *o, int N, int H, bool delta,
                           const int *slots, int pool, hipStream_t stream) {
    using S = DecodeShape<DK, DV>;
    const long long items = static_cast<long long>(N) * H * S::SLICES;
    const int blocks = static_cast<int>(S::KSPLIT > 1 ? items : (items + kWPB<DK> - 1) / kWPB<DK>);
    const float scale = 1.0f / sqrtf(static_cast<float>(DK));
    if (delta)
        hipLaunchKernelGGL((decode_kernel<DK, DV, TIn, true>), dim3(blocks), dim3(kWave * kWPB<DK>),
                           0, stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                           static_cast<const TIn *>(v), g, beta, state, o, static_cast<int>(items),
                           scale, slots, H, pool);
    else
        hipLaunchKernelGGL((decode_kernel<DK, DV, TIn, false>), dim3(blocks), dim3(kWave * kWPB<DK>),
                           0, stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                           static_cast<const TIn *>(v), g, beta, state, o, static_cast<int>(items),
                           scale, slots, H, pool);
    return hipGetLastError();
}

template <typename TIn>
hipError_t dispatch_decode(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, float *state, float *o, int N, int H, int dk,
                           int dv, bool delta, const int *slots, int pool, hipStream_t s) {
#define GDN_DEC(DK_, DV_)                                                                        \
    if (dk == DK_ && dv == DV_)                                                                  \
        return launch_decode_t<DK_, DV_, TIn>(q, k, v, g, beta, state, o, N, H, delta, slots, pool, s);
    GDN_DEC(16, 16) GDN_DEC(16, 64) GDN_DEC(16, 128)
    GDN_DEC(64, 16) GDN_DEC(64, 64) GDN_DEC(64, 128)
    GDN_DEC(128, 16) GDN_DEC(128, 64) GDN_DEC(128, 128)
#undef GDN_DEC
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state, float *o, int N, int H, int dk, int dv,
                         gdn_dtype dt, bool delta, const int *slots, int pool, hipStream_t stream) {
    if (dt == GDN_BF16)
        return dispatch_decode<uint16_t>(q, k, v, g, beta, state, o, N, H, dk, dv, delta, slots, pool,
                                         stream);
    return dispatch_decode<float>(q, k, v, g, beta, state, o, N, H, dk, dv, delta, slots, pool, stream);
}

}  // namespace gdn
