// gdn_prefill_valu.hip -- chunked GDN prefill with fp32 VALU arithmetic (gfx950).
//
// This is the precise path: every product is an fp32 VALU product, so the
// result tracks the token-by-token rule to fp32 rounding.  It serves fp32
// q/k/v, and bf16 q/k/v at head or chunk sizes of 16 that the MFMA path in
// gdn_prefill_bf16.hip does not tile.
//
// Chunk form of the gated delta rule (derived from the rule; the pages give
// no chunked algorithm).  For a chunk of L tokens with start state S0
// (key-major St = S0^T, d_k x d_v), G_r = sum_{i<=r} g_i, gamma_r = exp(G_r):
//   A     = strict_tril(diag(b) (K K^T  .*  exp(G_r - G_j)))
//   T     = (I + A)^{-1}                      (forward substitution)
//   U     = T diag(b) V
//   Delta = U - T diag(b gamma) (K St)        (= U - W St with W = T diag(b gamma) K)
//   O     = scale (diag(gamma) Q St + (Q K^T .* exp(G_r - G_j) .* tril) Delta)
//   St'   = gamma_L St + K^T diag(exp(G_L - G)) Delta
// Row r of Delta is delta_r = b_r (v_r - a_r S_{r-1} k_r), the per-token
// correction of the rule, so the chunk form reproduces it exactly in real
// arithmetic.  Decays are always formed as exp of a non-positive difference
// of cumulative gates (never as a ratio of two exponentials).
//
// Without the erase term (DELTA = false: S_t = a_t S_{t-1} + b_t v_t k_t^T) the
// same chunk form holds with A = 0, T = I and no W St term: Delta = diag(b) V.
//
// Work layout: one workgroup per (sequence, head, 16-wide value slice);
// value columns of the state evolve independently, so slices never talk.
// Chunks run in order inside the workgroup with the state slice in LDS.
// Packed sequences (seqs != NULL) take the same layout with each sequence's
// token range and pool slot from a device table.
#include <vector>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kSW = 16;  // value columns per workgroup

// Packed sequences for this kernel: S sequences, table [4][S] of ints (first token, length, pool
// slot or -1, start from the stored state), states in pool [slots][H][DK][DV].
struct ValuSeqs {
    const int *table;
    int S;
    float *pool;
};

template <int DK, int C, typename TIn, bool DELTA>
__global__ __launch_bounds__(kThreads) void prefill_valu_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *__restrict__ s0,
    float *__restrict__ o, float *__restrict__ s_out, float *__restrict__ chunk_states, int T_dense, int H,
    int DV, float scale, ValuSeqs sq) {
    __shared__ float A[C][C + 1];   // A, then the intra-chunk output weights P
    __shared__ float Tm[C][C + 1];  // (I + A)^{-1}
    __shared__ float St[DK][kSW];
    __shared__ float U[C][kSW];
    __shared__ float Y[C][kSW];
    __shared__ float D[C][kSW];
    __shared__ float Gc[C], bet[C], gam[C];

    const int tid = threadIdx.x;
    const int nslices = DV / kSW;
    const int slice = blockIdx.x % nslices;
    const int h = (blockIdx.x / nslices) % H;
    const int b = blockIdx.x / (nslices * H);  // sequence
    const int col0 = slice * kSW;
    const size_t bh = static_cast<size_t>(b) * H + h;
    // the sequence's first token in the [tokens, H, d] layout, its length, and the state it starts
    // from (NULL = zeros) and ends in (NULL = dropped)
    size_t tok_base = static_cast<size_t>(b) * T_dense;
    int T = T_dense;
    const float *start = s0 ? s0 + bh * DK * DV : nullptr;
    float *fin = s_out ? s_out + bh * DK * DV : nullptr;
    if (sq.table) {
        tok_base = static_cast<size_t>(sq.table[b]);
        T = sq.table[sq.S + b];
        const int slot = sq.table[2 * sq.S + b];
        float *st = slot >= 0 ? sq.pool + (static_cast<size_t>(slot) * H + h) * DK * DV : nullptr;
        start = sq.table[3 * sq.S + b] ? st : nullptr;
        fin = st;
    }

    for (int e = tid; e < DK * kSW; e += kThreads) {
        const int m = e / kSW, c = e % kSW;
        St[m][c] = start ? start[m * DV + col0 + c] : 0.f;
    }

    for (int t0 = 0; t0 < T; t0 += C) {
        const int L = min(C, T - t0);
        if (chunk_states) {  // the state this chunk starts from, kept for the gradients
            float *cs = chunk_states + (bh * ((T + C - 1) / C) + t0 / C) * DK * DV;
            for (int e = tid; e < DK * kSW; e += kThreads) cs[(e / kSW) * DV + col0 + e % kSW] = St[e / kSW][e % kSW];
        }
        // rows of token t of this (sequence, h): index (first token + t)*H + h
        auto row = [&](int r) { return (tok_base + t0 + r) * H + h; };

        if (tid < L) bet[tid] = beta[row(tid)];
        if (tid == 0) {
            float acc = 0.f;
            for (int r = 0; r < L; ++r) {
                acc += g[row(r)];
                Gc[r] = acc;
                gam[r] = expf(acc);
            }
        }
        __syncthreads();

        // A (strictly lower) and the decayed Q K^T weights need K K^T / Q K^T.
        for (int e = tid; e < L * L; e += kThreads) {
            const int r = e / L, j = e % L;
            float val = 0.f;
            if (DELTA && j < r) {
                float dot = 0.f;
                for (int m = 0; m < DK; ++m) dot += load_in(k, row(r) * DK + m) * load_in(k, row(j) * DK + m);
                val = bet[r] * dot * expf(Gc[r] - Gc[j]);
            }
            A[r][j] = val;
            Tm[r][j] = (r == j) ? 1.f : 0.f;
        }
        __syncthreads();

        // forward substitution, one row at a time: T[r][j] = -(A[r][j] + sum_{j<m<r} A[r][m] T[m][j])
        for (int r = 1; DELTA && r < L; ++r) {
            if (tid < r) {
                const int j = tid;
                float acc = A[r][j];
                for (int m = j + 1; m < r; ++m) acc += A[r][m] * Tm[m][j];
                Tm[r][j] = -acc;
            }
            __syncthreads();
        }

        // U = T diag(b) V ;  Y = K St
        for (int e = tid; e < L * kSW; e += kThreads) {
            const int r = e / kSW, c = e % kSW;
            float u = 0.f;
            for (int j = 0; j <= r; ++j) u += Tm[r][j] * bet[j] * load_in(v, row(j) * DV + col0 + c);
            U[r][c] = u;
            float y = 0.f;
            if (DELTA)
                for (int m = 0; m < DK; ++m) y += load_in(k, row(r) * DK + m) * St[m][c];
            Y[r][c] = y;
        }
        __syncthreads();

        // Delta = U - T diag(b gamma) Y
        for (int e = tid; e < L * kSW; e += kThreads) {
            const int r = e / kSW, c = e % kSW;
            float w = 0.f;
            if (DELTA)
                for (int j = 0; j <= r; ++j) w += Tm[r][j] * bet[j] * gam[j] * Y[j][c];
            D[r][c] = U[r][c] - w;
        }
        // P = Q K^T .* exp(G_r - G_j) .* tril (inclusive), reusing A
        for (int e = tid; e < L * L; e += kThreads) {
            const int r = e / L, j = e % L;
            float val = 0.f;
            if (j <= r) {
                float dot = 0.f;
                for (int m = 0; m < DK; ++m) dot += load_in(q, row(r) * DK + m) * load_in(k, row(j) * DK + m);
                val = dot * expf(Gc[r] - Gc[j]);
            }
            A[r][j] = val;
        }
        __syncthreads();

        // O = scale (diag(gamma) Q St + P Delta)
        for (int e = tid; e < L * kSW; e += kThreads) {
            const int r = e / kSW, c = e % kSW;
            float qs = 0.f;
            for (int m = 0; m < DK; ++m) qs += load_in(q, row(r) * DK + m) * St[m][c];
            float pd = 0.f;
            for (int j = 0; j <= r; ++j) pd += A[r][j] * D[j][c];
            o[row(r) * DV + col0 + c] = scale * (gam[r] * qs + pd);
        }
        __syncthreads();

        // St' = gamma_L St + K^T diag(exp(G_L - G)) Delta
        const float gl = Gc[L - 1];
        for (int e = tid; e < DK * kSW; e += kThreads) {
            const int m = e / kSW, c = e % kSW;
            float acc = 0.f;
            for (int j = 0; j < L; ++j) acc += load_in(k, row(j) * DK + m) * expf(gl - Gc[j]) * D[j][c];
            St[m][c] = gam[L - 1] * St[m][c] + acc;
        }
        __syncthreads();
    }

    if (fin) {
        // every thread reads only its own columns of the start state above (and that before the
        // chunk loop's barriers), so writing the final state over it in place is safe
        for (int e = tid; e < DK * kSW; e += kThreads) {
            const int m = e / kSW, c = e % kSW;
            fin[m * DV + col0 + c] = St[m][c];
        }
    }
}

template <int DK, int C, typename TIn>
hipError_t launch_valu_t(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *s0, float *o, float *s_out, float *chunk_states,
                         int B, int T, int H, int dv, bool delta, hipStream_t stream, ValuSeqs sq) {
    const int blocks = B * H * (dv / kSW);  // B: sequences
    const float scale = 1.0f / sqrtf(static_cast<float>(DK));
    if (delta)
        hipLaunchKernelGGL((prefill_valu_kernel<DK, C, TIn, true>), dim3(blocks), dim3(kThreads), 0,
                           stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                           static_cast<const TIn *>(v), g, beta, s0, o, s_out, chunk_states, T, H, dv, scale, sq);
    else
        hipLaunchKernelGGL((prefill_valu_kernel<DK, C, TIn, false>), dim3(blocks), dim3(kThreads), 0,
                           stream, static_cast<const TIn *>(q), static_cast<const TIn *>(k),
                           static_cast<const TIn *>(v), g, beta, s0, o, s_out, chunk_states, T, H, dv, scale, sq);
    return hipGetLastError();
}

template <typename TIn>
hipError_t dispatch_valu(const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *s0, float *o, float *s_out, float *chunk_states,
                         int B, int T, int H, int dk, int dv, int chunk, bool delta, hipStream_t stream,
                         ValuSeqs sq = ValuSeqs{}) {
#define GDN_VALU(DK_, C_)                                                                         \
    if (dk == DK_ && chunk == C_)                                                                 \
        return launch_valu_t<DK_, C_, TIn>(q, k, v, g, beta, s0, o, s_out, chunk_states, B, T, H, dv, delta, \
                                           stream, sq);
    GDN_VALU(16, 16) GDN_VALU(16, 32) GDN_VALU(16, 64)
    GDN_VALU(64, 16) GDN_VALU(64, 32) GDN_VALU(64, 64)
    GDN_VALU(128, 16) GDN_VALU(128, 32) GDN_VALU(128, 64)
#undef GDN_VALU
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill_valu(const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *s0, float *o, float *s_out, int B,
                               int T, int H, int dk, int dv, int chunk, gdn_dtype dt,
                               bool delta, hipStream_t stream, float *chunk_states) {
    if (dt == GDN_BF16)
        return dispatch_valu<uint16_t>(q, k, v, g, beta, s0, o, s_out, chunk_states, B, T, H, dk, dv, chunk,
                                       delta, stream);
    return dispatch_valu<float>(q, k, v, g, beta, s0, o, s_out, chunk_states, B, T, H, dk, dv, chunk, delta,
                                stream);
}

size_t prefill_valu_varlen_workspace(int S) { return S > 0 ? (static_cast<size_t>(4) * S * 4 + 255) & ~static_cast<size_t>(255) : 0; }

hipError_t launch_prefill_valu_varlen(const void *q, const void *k, const void *v, const float *g,
                                      const float *beta, const int *cu, int S, const int *slots,
                                      const int *init, float *pool, float *o, int H, int dk, int dv, int chunk,
                                      gdn_dtype dt, bool delta, void *ws, hipStream_t stream) {
    if (S <= 0) return hipSuccess;
    // the table [4][S]: first token, length, slot (-1: none), start from the stored state
    std::vector<int> t(static_cast<size_t>(4) * S);
    for (int s = 0; s < S; ++s) {
        t[s] = cu[s];
        t[S + s] = cu[s + 1] - cu[s];
        t[2 * S + s] = slots ? slots[s] : s;
        t[3 * S + s] = init ? (init[s] != 0) : 1;
    }
    hipError_t err = hipMemcpyAsync(ws, t.data(), t.size() * sizeof(int), hipMemcpyHostToDevice, stream);
    if (err != hipSuccess) return err;
    const ValuSeqs sq{static_cast<const int *>(ws), S, pool};
    if (dt == GDN_BF16)
        return dispatch_valu<uint16_t>(q, k, v, g, beta, nullptr, o, nullptr, nullptr, S, 0, H, dk, dv, chunk,
                                       delta, stream, sq);
    return dispatch_valu<float>(q, k, v, g, beta, nullptr, o, nullptr, nullptr, S, 0, H, dk, dv, chunk, delta,
                                stream, sq);
}

}  // namespace gdn
