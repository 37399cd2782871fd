// gdn_backward.hip -- gradients of the chunked prefill, both rules.
//
// The loss seen from the mixer is L = sum_t <dO_t, o_t> + <dS_T, S_T>.  Per
// chunk of C tokens, in the key-major state layout S (d_k x d_v) and with the
// chunk quantities of the forward (G the cumulative log-gate inside the chunk,
// gam = exp(G), eps_r = exp(G_last - G_r), Gam_rj = exp(G_r - G_j),
// A = strict_tril(diag(b) (K K^T .* Gam)), T = (I + A)^-1, W = T diag(b gam) K,
// U = T diag(b) V, P = tril(Q K^T .* Gam)):
//
//   Delta = U - W S                 O = scale (diag(gam) Q S + P Delta)
//   S'    = gam_last S + K^T diag(eps) Delta
//
// (the gated-decay rule has A = 0, T = I and no W S term).  With Y = dL/dS',
// the gradient reaching the chunk's start state is affine in Y:
//
//   dS = F Y + R,  F = gam_last I - W^T diag(eps) K,  R = scale (diag(gam) Q - P W)^T dO
//
// and inside the chunk, with dDelta = scale P^T dO + diag(eps) K Y:
//
//   dQ = scale diag(gam) dO S^T + (dP .* Gam) K,          dP = scale tril(dO Delta^T)
//   dK = (dP .* Gam)^T Q + diag(eps) Delta Y^T + diag(b gam) T^T dW + E K + E^T K
//   dV = diag(b) T^T dDelta,                               dW = -dDelta S^T
//   dA = -T^T (dW (diag(b gam) K)^T + dDelta (diag(b) V)^T) T^T,  E = diag(b) dA .* Gam
//   db, dG from the same terms; dg = reverse cumulative sum of dG over the chunk.
//
// Three launches after a forward pass that keeps every chunk's start state
// (gdn_prefill_chunk.hip): bwd_map_kernel (F and R of every chunk, chunks in
// parallel), bwd_scan_kernel (Y of every chunk, chunks in reverse order, 16
// state columns per workgroup) and bwd_grad_kernel (all gradients, chunks in
// parallel).  fp32 VALU arithmetic on LDS-resident chunk matrices.
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kBT = 256;          // threads per workgroup
constexpr int kC = 32;            // tokens per chunk
constexpr int kCP = kC + 1;       // padded C x C row
constexpr int kSl = 16;           // state columns per scan workgroup

struct BwdArgs {
    const void *q, *k, *v;
    const float *g, *beta, *d_o, *ds_final;
    const float *states;  // [BH][N][DK][DV] state each chunk starts from
    float *F;             // [BH][N][DK][DK] backward map of each chunk
    float *R;             // [BH][N][DK][DV] its constant term
    float *Y;             // [BH][N][DK][DV] gradient with respect to each chunk's end state
    float *dq, *dk, *dv, *dg, *dbeta, *ds0;
    int T, H, N, BH;
    float scale;
};

// out(i, j) = sum_kk A(i, kk) B(kk, j) for i < M, j < N: thread (ti, tj) owns
// column tj and rows ti + (kBT / N) x.
template <int M, int N, int K, class FA, class FB, class FS>
__device__ __forceinline__ void mm(FA A, FB Bm, FS store) {
    constexpr int NI = kBT / N;
    constexpr int RI = M / NI;
    static_assert(kBT % N == 0 && M % NI == 0, "tile");
    const int tj = threadIdx.x % N, ti = threadIdx.x / N;
    float acc[RI];
#pragma unroll
    for (int x = 0; x < RI; ++x) acc[x] = 0.f;
#pragma unroll 4
    for (int kk = 0; kk < K; ++kk) {
        const float bv = Bm(kk, tj);
#pragma unroll
        for (int x = 0; x < RI; ++x) acc[x] = fmaf(A(ti + NI * x, kk), bv, acc[x]);
    }
#pragma unroll
    for (int x = 0; x < RI; ++x) store(ti + NI * x, tj, acc[x]);
}

// One chunk's rows and its keyside matrices (shared by the map and gradient kernels).
template <int DK, int DV> struct ChunkLds {
    float q[kC][DK + 1], k[kC][DK + 1];
    float dO[kC][DV + 1];
    float T[kC][kCP];    // (I + A)^-1 (gated delta)
    float KG[kC][kCP];   // (k_r . k_j) Gam_rj, j < r
    float P[kC][kCP];    // (q_r . k_j) Gam_rj, j <= r
    float W[kC][DK + 1];
    float G[kC], gam[kC], eps[kC], b[kC];
};

// Loads q, k, dO, g, beta of chunk n of head bh (rows past the end read as zeros) and
// builds G, gam, eps, KG, P and, for the delta rule, T and W.
template <int DK, int DV, typename TIn, bool DELTA>
__device__ void chunk_keyside(const BwdArgs &a, ChunkLds<DK, DV> &s, int bh, int n, size_t &tok, int &L) {
    const int tid = threadIdx.x;
    const int bb = bh / a.H, h = bh % a.H;
    const int t0 = n * kC;
    L = min(kC, a.T - t0);
    tok = static_cast<size_t>(bb) * a.T + t0;
    const TIn *q = static_cast<const TIn *>(a.q), *k = static_cast<const TIn *>(a.k);
    for (int e = tid; e < kC * DK; e += kBT) {
        const int r = e / DK, c = e % DK;
        const size_t i = ((tok + r) * a.H + h) * DK + c;
        s.q[r][c] = r < L ? load_in(q, i) : 0.f;
        s.k[r][c] = r < L ? load_in(k, i) : 0.f;
    }
    for (int e = tid; e < kC * DV; e += kBT) {
        const int r = e / DV, c = e % DV;
        s.dO[r][c] = r < L ? a.d_o[((tok + r) * a.H + h) * DV + c] : 0.f;
    }
    if (tid < kC) {
        const size_t i = (tok + tid) * a.H + h;
        s.G[tid] = tid < L ? a.g[i] : 0.f;
        s.b[tid] = tid < L ? a.beta[i] : 0.f;
    }
    __syncthreads();
    if (tid == 0) {
        float acc = 0.f;
        for (int r = 0; r < kC; ++r) { acc += s.G[r]; s.G[r] = acc; }
    }
    __syncthreads();
    if (tid < kC) {
        s.gam[tid] = expf(s.G[tid]);
        s.eps[tid] = expf(s.G[kC - 1] - s.G[tid]);
    }
    // P and K K^T with the decay of every pair (exponents are <= 0 below the diagonal)
    mm<kC, kC, DK>([&](int i, int kk) { return s.q[i][kk]; }, [&](int kk, int j) { return s.k[j][kk]; },
                   [&](int i, int j, float x) { s.P[i][j] = j <= i ? x * expf(s.G[i] - s.G[j]) : 0.f; });
    if (DELTA)
        mm<kC, kC, DK>([&](int i, int kk) { return s.k[i][kk]; }, [&](int kk, int j) { return s.k[j][kk]; },
                       [&](int i, int j, float x) { s.KG[i][j] = j < i ? x * expf(s.G[i] - s.G[j]) : 0.f; });
    __syncthreads();
    if (!DELTA) return;
    // T = (I + diag(b) KG)^-1 by forward substitution, one column per thread
    if (tid < kC) {
        const int c = tid;
        float t[kC];
#pragma unroll
        for (int r = 0; r < kC; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < r; ++j) acc = fmaf(s.KG[r][j], t[j], acc);
            t[r] = (r == c ? 1.f : 0.f) - s.b[r] * acc;
        }
#pragma unroll
        for (int r = 0; r < kC; ++r) s.T[r][c] = t[r];
    }
    __syncthreads();
    // W = T diag(b gam) K
    mm<kC, DK, kC>([&](int i, int j) { return s.T[i][j]; },
                   [&](int j, int c) { return s.b[j] * s.gam[j] * s.k[j][c]; },
                   [&](int i, int c, float x) { s.W[i][c] = x; });
    __syncthreads();
}

// ---- F and R of every chunk ---------------------------------------------------
template <int DK, int DV, typename TIn, bool DELTA>
__global__ __launch_bounds__(kBT) void bwd_map_kernel(BwdArgs a) {
    __shared__ ChunkLds<DK, DV> s;
    __shared__ float X[kC][DK + 1];  // diag(gam) Q - P W
    const int bh = blockIdx.x / a.N, n = blockIdx.x % a.N;
    size_t tok;
    int L;
    chunk_keyside<DK, DV, TIn, DELTA>(a, s, bh, n, tok, L);
    if (DELTA) {
        mm<kC, DK, kC>([&](int i, int j) { return s.P[i][j]; }, [&](int j, int c) { return s.W[j][c]; },
                       [&](int i, int c, float x) { X[i][c] = s.gam[i] * s.q[i][c] - x; });
    } else {
        for (int e = threadIdx.x; e < kC * DK; e += kBT) X[e / DK][e % DK] = s.gam[e / DK] * s.q[e / DK][e % DK];
    }
    __syncthreads();
    const size_t base = static_cast<size_t>(bh) * a.N + n;
    float *R = a.R + base * DK * DV;
    mm<DK, DV, kC>([&](int j, int r) { return X[r][j]; }, [&](int r, int i) { return s.dO[r][i]; },
                   [&](int j, int i, float x) { R[j * DV + i] = a.scale * x; });
    float *F = a.F + base * DK * DK;
    const float gl = s.gam[kC - 1];
    if (DELTA) {
        mm<DK, DK, kC>([&](int j, int r) { return s.W[r][j]; }, [&](int r, int m) { return s.eps[r] * s.k[r][m]; },
                       [&](int j, int m, float x) { F[j * DK + m] = (j == m ? gl : 0.f) - x; });
    } else {
        for (int e = threadIdx.x; e < DK * DK; e += kBT) F[e] = (e / DK == e % DK) ? gl : 0.f;
    }
}

// ---- reverse scan: Y of every chunk, 16 state columns per workgroup --------------------
template <int DK, int DV>
__global__ __launch_bounds__(kBT) void bwd_scan_kernel(BwdArgs a) {
    constexpr int RJ = DK * kSl / kBT;  // rows per thread
    static_assert(RJ >= 1 && DK * kSl % kBT == 0, "scan tile");
    __shared__ float Fb[2][DK][DK + 1];
    __shared__ float Yb[2][DK][kSl + 1];
    const int slices = DV / kSl;
    const int bh = blockIdx.x / slices, c0 = (blockIdx.x % slices) * kSl;
    const int tid = threadIdx.x, c = tid % kSl, j0 = tid / kSl;
    constexpr int JS = kBT / kSl;  // row stride between a thread's rows
    const size_t head = static_cast<size_t>(bh) * a.N;

    for (int x = 0; x < RJ; ++x) {
        const int j = j0 + JS * x;
        Yb[0][j][c] = a.ds_final ? a.ds_final[(static_cast<size_t>(bh) * DK + j) * DV + c0 + c] : 0.f;
    }
    if (a.N > 0) {
        const float *F = a.F + (head + a.N - 1) * DK * DK;
        for (int e = tid; e < DK * DK; e += kBT) Fb[0][e / DK][e % DK] = F[e];
    }
    __syncthreads();
    for (int s = 0; s < a.N; ++s) {
        const int n = a.N - 1 - s, cur = s & 1;
        constexpr int FPT = DK * DK / kBT;
        float fn[FPT];
        if (n > 0) {
            const float *F = a.F + (head + n - 1) * DK * DK;
#pragma unroll
            for (int i = 0; i < FPT; ++i) fn[i] = F[tid + kBT * i];
        }
        const float *R = a.R + (head + n) * DK * DV;
        float *Yo = a.Y + (head + n) * DK * DV;
#pragma unroll
        for (int x = 0; x < RJ; ++x) {
            const int j = j0 + JS * x;
            Yo[j * DV + c0 + c] = Yb[cur][j][c];
            float acc = R[j * DV + c0 + c];
#pragma unroll 8
            for (int m = 0; m < DK; ++m) acc = fmaf(Fb[cur][j][m], Yb[cur][m][c], acc);
            Yb[cur ^ 1][j][c] = acc;
        }
        if (n > 0) {
#pragma unroll
            for (int i = 0; i < FPT; ++i) {
                const int e = tid + kBT * i;
                Fb[cur ^ 1][e / DK][e % DK] = fn[i];
            }
        }
        __syncthreads();
    }
    if (a.ds0) {
        const int fin = a.N & 1;
        for (int x = 0; x < RJ; ++x) {
            const int j = j0 + JS * x;
            a.ds0[(static_cast<size_t>(bh) * DK + j) * DV + c0 + c] = Yb[fin][j][c];
        }
    }
}

// ---- all gradients of one chunk -----------------------------------------------
template <int DK, int DV> struct GradLds {
    float v[kC][DV + 1];
    float S[DK][DV + 1], Yv[DK][DV + 1];
    float D[kC][DV + 1];     // Delta
    float dD[kC][DV + 1];    // dDelta
    float KY[kC][DV + 1];    // K Y, later dW (DV == DK)
    float TdW[kC][DK + 1];   // T^T dW
    float TdU[kC][DV + 1];   // T^T dDelta
    float dPg[kC][kCP];      // dP .* Gam
    float X1[kC][kCP];       // dP .* P, later dA .* A
    float dT[kC][kCP];       // dT, later dA
    float Z[kC][kCP];        // dT T^T
    float dG[kC], dbv[kC];   // dG[r]: written by thread r only
    float dlast;             // gate terms of the chunk's last position, from many threads
};

template <int DK, int DV, typename TIn, bool DELTA>
__global__ __launch_bounds__(kBT) void bwd_grad_kernel(BwdArgs a) {
    static_assert(DK == DV, "the dW buffer reuses K Y's");
    __shared__ ChunkLds<DK, DV> s;
    __shared__ GradLds<DK, DV> u;
    const int tid = threadIdx.x;
    const int bh = blockIdx.x / a.N, n = blockIdx.x % a.N;
    const int h = bh % a.H;
    size_t tok;
    int L;
    chunk_keyside<DK, DV, TIn, DELTA>(a, s, bh, n, tok, L);
    const size_t base = static_cast<size_t>(bh) * a.N + n;
    const TIn *vin = static_cast<const TIn *>(a.v);
    for (int e = tid; e < kC * DV; e += kBT) {
        const int r = e / DV, c = e % DV;
        u.v[r][c] = r < L ? load_in(vin, ((tok + r) * a.H + h) * DV + c) : 0.f;
    }
    for (int e = tid; e < DK * DV; e += kBT) {
        u.S[e / DV][e % DV] = a.states[base * DK * DV + e];
        u.Yv[e / DV][e % DV] = a.Y[base * DK * DV + e];
    }
    if (tid < kC) { u.dG[tid] = 0.f; u.dbv[tid] = 0.f; }
    if (tid == 0) u.dlast = 0.f;
    __syncthreads();

    // Delta = T diag(b) V - W S  (decay rule: diag(b) V);  K Y
    if (DELTA) {
        mm<kC, DV, kC>([&](int i, int j) { return s.T[i][j]; }, [&](int j, int c) { return s.b[j] * u.v[j][c]; },
                       [&](int i, int c, float x) { u.D[i][c] = x; });
    } else {
        for (int e = tid; e < kC * DV; e += kBT) u.D[e / DV][e % DV] = s.b[e / DV] * u.v[e / DV][e % DV];
    }
    mm<kC, DV, DK>([&](int i, int j) { return s.k[i][j]; }, [&](int j, int c) { return u.Yv[j][c]; },
                   [&](int i, int c, float x) { u.KY[i][c] = x; });
    __syncthreads();
    if (DELTA) {
        mm<kC, DV, DK>([&](int i, int j) { return s.W[i][j]; }, [&](int j, int c) { return u.S[j][c]; },
                       [&](int i, int c, float x) { u.D[i][c] -= x; });
        __syncthreads();
    }
    // dDelta = scale P^T dO + diag(eps) K Y;  dP = scale tril(dO Delta^T)
    mm<kC, DV, kC>([&](int i, int r) { return s.P[r][i]; }, [&](int r, int c) { return s.dO[r][c]; },
                   [&](int i, int c, float x) { u.dD[i][c] = a.scale * x + s.eps[i] * u.KY[i][c]; });
    mm<kC, kC, DV>([&](int r, int c) { return s.dO[r][c]; }, [&](int c, int j) { return u.D[j][c]; },
                   [&](int r, int j, float x) {
                       const float dp = j <= r ? a.scale * x : 0.f;
                       u.dPg[r][j] = dp * (j <= r ? expf(s.G[r] - s.G[j]) : 0.f);
                       u.X1[r][j] = dp * s.P[r][j];
                   });
    __syncthreads();
    // gate terms: readout decay, P, the end-state decay (eps and gam_last)
    if (tid < kC) {
        const int r = tid;
        float rs = 0.f, cs = 0.f, e = 0.f;
        for (int j = 0; j < kC; ++j) { rs += u.X1[r][j]; cs += u.X1[j][r]; }
        for (int c = 0; c < DV; ++c) e = fmaf(u.KY[r][c], u.D[r][c], e);
        e *= s.eps[r];
        u.dG[r] += rs - cs - e;
        atomicAdd(&u.dlast, e);
    }
    if (tid >= 64 && tid < 128) {  // gam_last <Y, S>: one wavefront
        float x = 0.f;
        for (int e = tid - 64; e < DK * DV; e += 64) x = fmaf(u.Yv[e / DV][e % DV], u.S[e / DV][e % DV], x);
        for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
        if (tid == 64) atomicAdd(&u.dlast, s.gam[kC - 1] * x);
    }
    // dQ = scale diag(gam) dO S^T (+ its gate term) + (dP .* Gam) K, into W's buffer
    mm<kC, DK, DV>([&](int r, int i) { return s.dO[r][i]; }, [&](int i, int c) { return u.S[c][i]; },
                   [&](int r, int c, float x) { s.W[r][c] = a.scale * s.gam[r] * x; });
    __syncthreads();
    if (tid < kC) {
        float x = 0.f;
        for (int c = 0; c < DK; ++c) x = fmaf(s.q[tid][c], s.W[tid][c], x);
        u.dG[tid] += x;
    }
    mm<kC, DK, kC>([&](int r, int j) { return u.dPg[r][j]; }, [&](int j, int c) { return s.k[j][c]; },
                   [&](int r, int c, float x) {
                       if (r < L) a.dq[((tok + r) * a.H + h) * DK + c] = s.W[r][c] + x;
                   });
    // dW = -dDelta S^T (into K Y's buffer), T^T dDelta
    __syncthreads();
    if (DELTA) {
        mm<kC, DK, DV>([&](int i, int l) { return u.dD[i][l]; }, [&](int l, int c) { return u.S[c][l]; },
                       [&](int i, int c, float x) { u.KY[i][c] = -x; });
        mm<kC, DV, kC>([&](int j, int i) { return s.T[i][j]; }, [&](int i, int c) { return u.dD[i][c]; },
                       [&](int j, int c, float x) { u.TdU[j][c] = x; });
        __syncthreads();
        mm<kC, DK, kC>([&](int j, int i) { return s.T[i][j]; }, [&](int i, int c) { return u.KY[i][c]; },
                       [&](int j, int c, float x) { u.TdW[j][c] = x; });
        // dT = dW (diag(b gam) K)^T + dDelta (diag(b) V)^T
        mm<kC, kC, DK>([&](int i, int c) { return u.KY[i][c]; },
                       [&](int c, int j) { return s.b[j] * s.gam[j] * s.k[j][c]; },
                       [&](int i, int j, float x) { u.dT[i][j] = x; });
        __syncthreads();
        mm<kC, kC, DV>([&](int i, int c) { return u.dD[i][c]; }, [&](int c, int j) { return s.b[j] * u.v[j][c]; },
                       [&](int i, int j, float x) { u.dT[i][j] += x; });
        __syncthreads();
        // dA = -T^T (dT T^T), strictly lower
        mm<kC, kC, kC>([&](int i, int l) { return u.dT[i][l]; }, [&](int l, int j) { return s.T[j][l]; },
                       [&](int i, int j, float x) { u.Z[i][j] = x; });
        __syncthreads();
        mm<kC, kC, kC>([&](int i, int l) { return s.T[l][i]; }, [&](int l, int j) { return u.Z[l][j]; },
                       [&](int i, int j, float x) {
                           const float da = j < i ? -x : 0.f;
                           u.dT[i][j] = da;                        // dA
                           u.X1[i][j] = da * s.b[i] * s.KG[i][j];  // dA .* A
                       });
        __syncthreads();
        if (tid < kC) {
            const int r = tid;
            float rs = 0.f, cs = 0.f, dbA = 0.f, wk = 0.f, uv = 0.f;
            for (int j = 0; j < kC; ++j) {
                rs += u.X1[r][j];
                cs += u.X1[j][r];
                dbA = fmaf(u.dT[r][j], s.KG[r][j], dbA);
            }
            for (int c = 0; c < DK; ++c) wk = fmaf(u.TdW[r][c], s.k[r][c], wk);
            for (int c = 0; c < DV; ++c) uv = fmaf(u.TdU[r][c], u.v[r][c], uv);
            u.dG[r] += rs - cs + s.b[r] * s.gam[r] * wk;
            u.dbv[r] = uv + s.gam[r] * wk + dbA;
        }
        // E = diag(b) dA .* Gam, kept in Z
        for (int e = tid; e < kC * kC; e += kBT) {
            const int i = e / kC, j = e % kC;
            u.Z[i][j] = j < i ? s.b[i] * u.dT[i][j] * expf(s.G[i] - s.G[j]) : 0.f;
        }
        __syncthreads();
    } else {
        if (tid < kC) {
            float uv = 0.f;
            for (int c = 0; c < DV; ++c) uv = fmaf(u.dD[tid][c], u.v[tid][c], uv);
            u.dbv[tid] = uv;
        }
        __syncthreads();
    }
    // dV = diag(b) T^T dDelta (decay rule: diag(b) dDelta)
    for (int e = tid; e < kC * DV; e += kBT) {
        const int r = e / DV, c = e % DV;
        if (r < L) a.dv[((tok + r) * a.H + h) * DV + c] = s.b[r] * (DELTA ? u.TdU[r][c] : u.dD[r][c]);
    }
    // dK = (dP .* Gam)^T Q + diag(eps) Delta Y^T [+ diag(b gam) T^T dW + E K + E^T K]
    mm<kC, DK, kC>([&](int j, int r) { return u.dPg[r][j]; }, [&](int r, int c) { return s.q[r][c]; },
                   [&](int j, int c, float x) { s.W[j][c] = x; });
    __syncthreads();
    mm<kC, DK, DV>([&](int j, int i) { return u.D[j][i]; }, [&](int i, int c) { return u.Yv[c][i]; },
                   [&](int j, int c, float x) { s.W[j][c] += s.eps[j] * x; });
    __syncthreads();
    if (DELTA) {
        mm<kC, DK, kC>([&](int i, int j) { return u.Z[i][j] + u.Z[j][i]; }, [&](int j, int c) { return s.k[j][c]; },
                       [&](int i, int c, float x) { s.W[i][c] += x + s.b[i] * s.gam[i] * u.TdW[i][c]; });
        __syncthreads();
    }
    for (int e = tid; e < kC * DK; e += kBT) {
        const int r = e / DK, c = e % DK;
        if (r < L) a.dk[((tok + r) * a.H + h) * DK + c] = s.W[r][c];
    }
    // dg: reverse cumulative sum of dG inside the chunk; dbeta
    if (tid == 0) {
        float acc = u.dlast;
        for (int r = kC - 1; r >= 0; --r) {
            acc += u.dG[r];
            if (r < L) a.dg[(tok + r) * a.H + h] = acc;
        }
    }
    if (tid < L) a.dbeta[(tok + tid) * a.H + h] = u.dbv[tid];
}

template <int DK, int DV, bool DELTA>
hipError_t run_backward(BwdArgs &a, gdn_dtype dt, hipStream_t stream) {
    const int items = a.BH * a.N;
    const bool bf = dt == GDN_BF16;
    if (items > 0) {
        if (bf) hipLaunchKernelGGL((bwd_map_kernel<DK, DV, uint16_t, DELTA>), dim3(items), dim3(kBT), 0, stream, a);
        else hipLaunchKernelGGL((bwd_map_kernel<DK, DV, float, DELTA>), dim3(items), dim3(kBT), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_scan_kernel<DK, DV>), dim3(a.BH * (DV / kSl)), dim3(kBT), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || items == 0) return e;
    if (bf) hipLaunchKernelGGL((bwd_grad_kernel<DK, DV, uint16_t, DELTA>), dim3(items), dim3(kBT), 0, stream, a);
    else hipLaunchKernelGGL((bwd_grad_kernel<DK, DV, float, DELTA>), dim3(items), dim3(kBT), 0, stream, a);
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct BwdLayout {
    size_t fwd, o, sfin, states, F, R, Y, total;
};
BwdLayout bwd_layout(int B, int T, int H, int dk, int dv) {
    const size_t BH = static_cast<size_t>(B) * H, N = (static_cast<size_t>(T) + kC - 1) / kC;
    BwdLayout L{};
    size_t off = 0;
    L.fwd = off; off += T > 0 ? align256(prefill_chunk_workspace(B, T, H, dk, dv, kC)) : 0;
    L.o = off; off += align256(static_cast<size_t>(B) * T * H * dv * 4);
    L.sfin = off; off += align256(BH * dk * dv * 4);
    L.states = off; off += align256(BH * N * dk * dv * 4);
    L.F = off; off += align256(BH * N * dk * dk * 4);
    L.R = off; off += align256(BH * N * dk * dv * 4);
    L.Y = off; off += align256(BH * N * dk * dv * 4);
    L.total = off;
    return L;
}

}  // namespace

bool backward_supported(int dk, int dv, gdn_dtype dt) { return dk == 64 && dv == 64 && dt == GDN_BF16; }

int backward_chunk() { return kC; }

size_t backward_workspace(int B, int T, int H, int dk, int dv) { return bwd_layout(B, T, H, dk, dv).total; }

hipError_t launch_backward(const void *q, const void *k, const void *v, const float *g,
                           const float *beta, const float *s0, const float *d_o,
                           const float *ds_final, float *dq, float *dk, float *dv, float *dg,
                           float *dbeta, float *ds0, int B, int T, int H, int d_k, int d_v,
                           gdn_dtype dt, bool delta, void *ws, hipStream_t stream) {
    if (!backward_supported(d_k, d_v, dt)) return hipErrorInvalidValue;
    const BwdLayout L = bwd_layout(B, T, H, d_k, d_v);
    char *w = static_cast<char *>(ws);
    BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.d_o = d_o; a.ds_final = ds_final;
    a.states = reinterpret_cast<float *>(w + L.states);
    a.F = reinterpret_cast<float *>(w + L.F);
    a.R = reinterpret_cast<float *>(w + L.R);
    a.Y = reinterpret_cast<float *>(w + L.Y);
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.ds0 = ds0;
    a.T = T; a.H = H; a.BH = B * H; a.N = (T + kC - 1) / kC;
    a.scale = 1.0f / sqrtf(static_cast<float>(d_k));
    if (T > 0) {
        // forward pass again, keeping the state every chunk starts from
        hipError_t e = launch_prefill_chunk(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                                            static_cast<const uint16_t *>(v), g, beta, s0,
                                            reinterpret_cast<float *>(w + L.o), reinterpret_cast<float *>(w + L.sfin),
                                            B, T, H, d_k, d_v, kC, delta, w + L.fwd, stream,
                                            reinterpret_cast<float *>(w + L.states));
        if (e != hipSuccess) return e;
    }
    return delta ? run_backward<64, 64, true>(a, dt, stream) : run_backward<64, 64, false>(a, dt, stream);
}

}  // namespace gdn
