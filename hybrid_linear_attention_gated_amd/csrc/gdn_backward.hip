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
// Three passes after a forward pass that keeps every chunk's start state
// (gdn_prefill_chunk.hip): bwd_map_kernel (F and R of every chunk, chunks in
// parallel), bwd_scan_kernel (Y of every chunk, chunks in reverse order; long
// sequences in two levels of pieces) and bwd_grad_kernel (all gradients, chunks in
// parallel), on LDS-resident chunk matrices; 128-wide heads keep the gradient pass's largest
// matrices (the state and its gradient alone are 128 KB) in a global scratch slot per workgroup
// instead (bwd_grad_gs_kernel).  Products run on the matrix cores: for bf16 inputs as three-pass
// hi/lo bf16 MFMA (fp32-class results; one or two passes measured over the error bar), except the
// gate prefix sums and the 16 x 16 blocks of the inverse, which stay fp32; fp32 inputs keep every
// product in fp32.
#include "gdn_mfma.h"

namespace gdn {
namespace {

// Launch shapes and LDS padding (overridable at build time for tuning sweeps).
#ifndef GDN_BWD_THREADS
#define GDN_BWD_THREADS 1024
#endif
#ifndef GDN_BWD_MAP_THREADS
#define GDN_BWD_MAP_THREADS 512
#endif
#ifndef GDN_BWD_PAD_D
#define GDN_BWD_PAD_D 2
#endif
#ifndef GDN_BWD_PAD_C
#define GDN_BWD_PAD_C 4
#endif
constexpr int kC = 32;                     // tokens per chunk
template <int DK> constexpr int kBT = 4 * DK;  // threads per scan workgroup: one 16-row tile per wavefront
constexpr int kBTM = GDN_BWD_MAP_THREADS;  // threads per map workgroup
constexpr int kBTG = GDN_BWD_THREADS;      // threads per gradient workgroup
constexpr int kPD = GDN_BWD_PAD_D;         // row padding of d-wide LDS matrices (floats)
constexpr int kCP = kC + GDN_BWD_PAD_C;    // padded C x C row (a multiple of 4: float4 row reads)
static_assert(kCP % 4 == 0, "C x C rows read as float4");
// A chunk's stored keyside, in floats: T, KG, P (C x C each), W (C x DK), G, gam, eps (C each)
template <int DK> constexpr int ks_floats() { return 3 * kC * kC + kC * DK + 3 * kC; }

struct BwdArgs {
    const void *q, *k, *v;
    const float *g, *beta, *d_o, *ds_final;
    const float *states;  // [BH][N][DK][DV] state each chunk starts from
    float *F;             // [BH][N][DK][DK] backward map of each chunk
    float *R;             // [BH][N][DK][DV] its constant term
    float *Y;             // [BH][N][DK][DV] gradient with respect to each chunk's end state
    float *KS;            // [BH][N] keyside of each chunk: T, KG, P, W, G, gam, eps (ks_floats)
    float *dq, *dk, *dv, *dg, *dbeta, *ds0;
    int T, H, N, BH;
    float scale;
    void *gscratch;       // 128-wide heads: the gradient pass's global scratch slots
};

// threadIdx.x, read so that the compiler takes it as a new value: a kernel that loops over chunks
// reads it once per chunk and passes it to the chunk's products, which then derive their per-lane
// LDS addresses inside the iteration instead of holding them all in registers across the loop
// (which spills).
__device__ __forceinline__ int thread_id() {
    int t = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(t));
    return t;
}

// out(i, j) = sum_kk A(i, kk) B(kk, j) for i < M, j < N, on the fp32 matrix cores:
// 16 x 16 output tiles dealt round-robin to wavefronts w0 .. w0 + nw - 1 (nw = 0: all of
// the workgroup's), so independent products can run side by side; each tile accumulated by
// v_mfma_f32_16x16x4_f32 over K in steps of 4.  Lane l feeds A(i0 + l % 16, k0 + l / 16)
// and B(k0 + l / 16, j0 + l % 16) and receives out(i0 + 4 (l / 16) + r, j0 + l % 16), r < 4.
//
// HL (bf16 inputs, K a multiple of 32): the same tiles on v_mfma_f32_16x16x32_bf16 instead, both
// operands split into hi + lo bf16 and three passes (hi.hi + hi.lo + lo.hi): about 16 significant
// bits per operand, fp32 accumulation.  Lane (lk, li) feeds the k-slots kmap(s, lk, e) of row
// i0 + li of A and of column j0 + li of B; the output layout is the same.
// NP (with HL): the passes taken, a mask of 1 = hi.hi, 2 = hi(A).lo(B), 4 = lo(A).hi(B).  Where an
// operand is exact in bf16 (the q and k inputs, the ones of a row sum) its lo part is zero, and the
// pass that would multiply it is left out (and the part not computed): the same results.
// tid: threadIdx.x, passed in (see thread_id).
template <int M, int N, int K, bool HL = false, int NP = 7, class FA, class FB, class FS>
__device__ __forceinline__ void mm_t(int tid, FA A, FB Bm, FS store, int w0 = 0, int nw = 0) {
    static_assert(M % 16 == 0 && N % 16 == 0 && K % 4 == 0, "tile");
    constexpr int TN = N / 16, TILES = (M / 16) * TN;
    const int lane = tid % 64, wave = __builtin_amdgcn_readfirstlane(tid / 64) - w0;
    const int li = lane % 16, lk = lane / 16;
    const int waves = nw > 0 ? nw : static_cast<int>(blockDim.x) / 64;
    if (wave < 0 || wave >= waves) return;
    if constexpr (HL && K % 32 == 0) {
        for (int t = wave; t < TILES; t += waves) {
            const int i0 = (t / TN) * 16, j0 = (t % TN) * 16;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < K / 32; ++s) {
                float xa[8], xb[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int kk = kmap(s, lk, e);
                    xa[e] = A(i0 + li, kk);
                    xb[e] = Bm(kk, j0 + li);
                }
                bf16x8 ah, al, bh, bl;
                if constexpr ((NP & 4) != 0) split_bf16(xa, ah, al);
                else ah = pack_bf16(xa);
                if constexpr ((NP & 2) != 0) split_bf16(xb, bh, bl);
                else bh = pack_bf16(xb);
                acc = mfma_bf16(ah, bh, acc);
                if constexpr ((NP & 2) != 0) acc = mfma_bf16(ah, bl, acc);
                if constexpr ((NP & 4) != 0) acc = mfma_bf16(al, bh, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) store(i0 + 4 * lk + r, j0 + li, acc[r]);
        }
        return;
    }
    // operands read before the products, a block of at most 64 along K at a time (128-wide
    // contractions would otherwise hold 64 operand registers per lane)
    constexpr int KB = K > 64 ? 64 : K;
    static_assert(K % KB == 0, "K blocks");
    for (int t = wave; t < TILES; t += waves) {
        const int i0 = (t / TN) * 16, j0 = (t % TN) * 16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int k0 = 0; k0 < K; k0 += KB) {
            float av[KB / 4], bv[KB / 4];
#pragma unroll
            for (int s = 0; s < KB / 4; ++s) {
                av[s] = A(i0 + li, k0 + 4 * s + lk);
                bv[s] = Bm(k0 + 4 * s + lk, j0 + li);
            }
#pragma unroll
            for (int s = 0; s < KB / 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s], bv[s], acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) store(i0 + 4 * lk + r, j0 + li, acc[r]);
    }
}

template <int M, int N, int K, bool HL = false, int NP = 7, class FA, class FB, class FS>
__device__ __forceinline__ void mm(FA A, FB Bm, FS store, int w0 = 0, int nw = 0) {
    mm_t<M, N, K, HL, NP>(static_cast<int>(threadIdx.x), A, Bm, store, w0, nw);
}

// sum_kk A(i, kk) for i < M, by a product with a block of ones; store(i, x).
template <int M, int K, bool HL = false, class FA, class FS>
__device__ __forceinline__ void rowsum_t(int tid, FA A, FS store, int w0 = 0, int nw = 0) {
    mm_t<M, 16, K, HL, 5>(tid, A, [](int, int) { return 1.f; }, [&](int i, int j, float x) { if (j == 0) store(i, x); },
                          w0, nw);
}

// x as held by lane l of the wavefront (l a constant; a uniform value)
__device__ __forceinline__ float lane_value(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// One chunk's rows and its keyside matrices (shared by the map and gradient kernels).
template <int DK, int DV> struct alignas(16) ChunkLds {
    float q[kC][DK + kPD], k[kC][DK + kPD];
    float dO[kC][DV + kPD];
    float T[kC][kCP];    // (I + A)^-1 (gated delta)
    float KG[kC][kCP];   // (k_r . k_j) Gam_rj, j < r
    float P[kC][kCP];    // (q_r . k_j) Gam_rj, j <= r
    float W[kC][DK + kPD];
    float graw[kC], G[kC], gam[kC], eps[kC], b[kC];
};

// One chunk's rows in registers, loaded from HBM ahead of their use; rows past the end of the
// sequence are zeros.  Thread tid holds a contiguous run of each tensor (elements
// tid * n .. tid * n + n - 1, inside one row), read with one 4-, 8- or 16-byte load.  GRAD also
// takes v and the chunk's start state and end-state gradient.
template <int NT, int DK, int DV, bool GRAD> struct ChunkRows {
    static constexpr int NQ = kC * DK / NT, NV = kC * DV / NT, NS = GRAD ? DK * DV / NT : 1;
    static_assert((NQ == 2 || NQ == 4 || NQ == 8) && (NV == 2 || NV == 4 || NV == 8) && (!GRAD || NS == 4 || NS == 8),
                  "runs per thread");
    float q[NQ], k[NQ], dO[NV], v[GRAD ? NV : 1], S[NS], Y[NS], g, b;
};

struct ChunkPos {
    size_t tok;  // row of the chunk's first token in [B*T]
    int h, L;    // head, valid tokens
};
__device__ __forceinline__ ChunkPos chunk_pos(const BwdArgs &a, int w) {
    const int bh = w / a.N, n = w % a.N;
    ChunkPos p;
    p.h = bh % a.H;
    p.L = min(kC, a.T - n * kC);
    p.tok = static_cast<size_t>(bh / a.H) * a.T + static_cast<size_t>(n) * kC;
    return p;
}

// n consecutive stored values (n = 2, 4 or 8) widened to fp32, or zeros
template <int n> __device__ __forceinline__ void load_run(const uint16_t *p, bool in, float (&x)[n]) {
    uint32_t u[n / 2];
    if (n == 2) u[0] = in ? *reinterpret_cast<const uint32_t *>(p) : 0u;
    else {
#pragma unroll
        for (int i = 0; i < n / 4; ++i) {
            const uint2 w = in ? reinterpret_cast<const uint2 *>(p)[i] : make_uint2(0u, 0u);
            u[2 * i] = w.x;
            u[2 * i + 1] = w.y;
        }
    }
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
        x[2 * i] = bf16_bits_to_f32(static_cast<uint16_t>(u[i] & 0xffffu));
        x[2 * i + 1] = bf16_bits_to_f32(static_cast<uint16_t>(u[i] >> 16));
    }
}
template <int n> __device__ __forceinline__ void load_run(const float *p, bool in, float (&x)[n]) {
    if (n == 2) {
        const float2 w = in ? *reinterpret_cast<const float2 *>(p) : make_float2(0.f, 0.f);
        x[0] = w.x;
        x[n - 1] = w.y;
    } else {
#pragma unroll
        for (int i = 0; i < n / 4; ++i) {
            const float4 w = in ? reinterpret_cast<const float4 *>(p)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            x[4 * i] = w.x; x[4 * i + 1] = w.y; x[4 * i + 2] = w.z; x[4 * i + 3] = w.w;
        }
    }
}

template <int NT, int DK, int DV, typename TIn, bool GRAD>
__device__ __forceinline__ void chunk_load(const BwdArgs &a, int w, ChunkRows<NT, DK, DV, GRAD> &R) {
    using CR = ChunkRows<NT, DK, DV, GRAD>;
    const int tid = threadIdx.x;
    const ChunkPos p = chunk_pos(a, w);
    {
        const int e = tid * CR::NQ, r = e / DK, c = e % DK;
        const size_t x = ((p.tok + r) * a.H + p.h) * DK + c;
        load_run<CR::NQ>(static_cast<const TIn *>(a.q) + x, r < p.L, R.q);
        load_run<CR::NQ>(static_cast<const TIn *>(a.k) + x, r < p.L, R.k);
    }
    {
        const int e = tid * CR::NV, r = e / DV, c = e % DV;
        const size_t x = ((p.tok + r) * a.H + p.h) * DV + c;
        load_run<CR::NV>(a.d_o + x, r < p.L, R.dO);
        if constexpr (GRAD) load_run<CR::NV>(static_cast<const TIn *>(a.v) + x, r < p.L, R.v);
    }
    if constexpr (GRAD) {
        const size_t x = static_cast<size_t>(w) * DK * DV + static_cast<size_t>(tid) * CR::NS;
        load_run<CR::NS>(a.states + x, true, R.S);
        load_run<CR::NS>(a.Y + x, true, R.Y);
    }
    const size_t x = (p.tok + tid) * a.H + p.h;
    R.g = tid < p.L ? a.g[x] : 0.f;
    R.b = tid < p.L ? a.beta[x] : 0.f;
}

template <int NT, int DK, int DV, bool GRAD>
__device__ __forceinline__ void chunk_stage(const ChunkRows<NT, DK, DV, GRAD> &R, ChunkLds<DK, DV> &s,
                                            float (*v)[DV + kPD], float (*S)[DV + kPD], float (*Y)[DV + kPD]) {
    using CR = ChunkRows<NT, DK, DV, GRAD>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < CR::NQ; ++i) {
        const int e = tid * CR::NQ + i;
        s.q[e / DK][e % DK] = R.q[i];
        s.k[e / DK][e % DK] = R.k[i];
    }
#pragma unroll
    for (int i = 0; i < CR::NV; ++i) {
        const int e = tid * CR::NV + i;
        s.dO[e / DV][e % DV] = R.dO[i];
        if (GRAD) v[e / DV][e % DV] = R.v[i];
    }
    if (GRAD) {
#pragma unroll
        for (int i = 0; i < CR::NS; ++i) {
            const int e = tid * CR::NS + i;
            S[e / DV][e % DV] = R.S[i];
            Y[e / DV][e % DV] = R.Y[i];
        }
    }
    if (tid < kC) {
        s.graw[tid] = R.g;
        s.b[tid] = R.b;
    }
}

// The chunk's keyside from its staged rows (the caller has synchronised after staging):
// G, gam, eps, P, KG and, for the delta rule, T and W.
template <int DK, int DV, bool DELTA, bool HL>
__device__ void chunk_keyside(ChunkLds<DK, DV> &s) {
    const int tid = threadIdx.x;
    // G = (lower-triangular ones) g
    mm<kC, 16, kC>([](int i, int j) { return j <= i ? 1.f : 0.f; }, [&](int j, int) { return s.graw[j]; },
                   [&](int i, int c, float x) { if (c == 0) s.G[i] = x; });
    __syncthreads();
    if (tid < kC) {
        s.gam[tid] = expf(s.G[tid]);
        s.eps[tid] = expf(s.G[kC - 1] - s.G[tid]);
    }
    // P and K K^T with the decay of every pair (exponents are <= 0 below the diagonal)
    const int half = static_cast<int>(blockDim.x) / 128;  // wavefronts in each half of the workgroup
    mm<kC, kC, DK, HL, 1>([&](int i, int kk) { return s.q[i][kk]; }, [&](int kk, int j) { return s.k[j][kk]; },
                   [&](int i, int j, float x) { s.P[i][j] = j <= i ? x * expf(s.G[i] - s.G[j]) : 0.f; }, 0, half);
    if (DELTA)
        mm<kC, kC, DK, HL, 1>([&](int i, int kk) { return s.k[i][kk]; }, [&](int kk, int j) { return s.k[j][kk]; },
                       [&](int i, int j, float x) { s.KG[i][j] = j < i ? x * expf(s.G[i] - s.G[j]) : 0.f; },
                       half, half);
    __syncthreads();
    if (!DELTA) return;
    // T = (I + diag(b) KG)^-1.  Its two diagonal 16 x 16 blocks by forward substitution, one
    // column per lane (the first block on wavefront 0, the second on wavefront 1, so the two run
    // at once); the upper-right block is zero; the lower-left one is T21 = -T22 (A21 T11), with
    // A21 = diag(b) KG restricted to those rows and columns, by two 16 x 16 products.
    static_assert(kC == 32, "two diagonal blocks of 16");
    {
        const int wave = tid / 64, c = tid % 64;
        if (wave < 2 && c < 16) {
            // lane c holds row c of the block and b of that row; row r reaches every lane by a
            // read of lane r, so the substitution waits on no LDS access
            const int o = 16 * wave;
            float kr[16];
#pragma unroll
            for (int j = 0; j < 16; j += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(&s.KG[o + c][o + j]);
                kr[j] = x.x; kr[j + 1] = x.y; kr[j + 2] = x.z; kr[j + 3] = x.w;
            }
            const float br = s.b[o + c];
            float t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < r; ++j) acc = fmaf(lane_value(kr[j], r), t[j], acc);
                t[r] = fmaf(-lane_value(br, r), acc, r == c ? 1.f : 0.f);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) s.T[o + r][o + c] = t[r];
        } else if (wave == 2) {
#pragma unroll
            for (int r = 0; r < 4; ++r) s.T[4 * r + c / 16][16 + c % 16] = 0.f;
        }
    }
    __syncthreads();
    // A21 T11, parked in W's rows (W is written after T)
    mm<16, 16, 16>([&](int i, int j) { return s.b[16 + i] * s.KG[16 + i][j]; }, [&](int j, int c) { return s.T[j][c]; },
                   [&](int i, int c, float x) { s.W[i][c] = x; }, 0, 1);
    __syncthreads();
    mm<16, 16, 16>([&](int i, int j) { return s.T[16 + i][16 + j]; }, [&](int j, int c) { return s.W[j][c]; },
                   [&](int i, int c, float x) { s.T[16 + i][c] = -x; }, 0, 1);
    __syncthreads();
    // W = T diag(b gam) K
    mm<kC, DK, kC, HL>([&](int i, int j) { return s.T[i][j]; },
                   [&](int j, int c) { return s.b[j] * s.gam[j] * s.k[j][c]; },
                   [&](int i, int c, float x) { s.W[i][c] = x; });
    __syncthreads();
}

// The keyside the map kernel stored, in registers (1,024 threads, d_k = 64): thread tid holds
// float4 number tid of T | KG | P | W rows 0-15 (4,096 floats), float tid of W rows 16-31, and for
// tid < 96 one of G | gam | eps.  The decay rule reads only P and the gates.
struct KsRows {
    float4 m;
    float w, gate;
};
template <int DK, bool DELTA>
__device__ __forceinline__ void keyside_load(const BwdArgs &a, int w, KsRows &R) {
    static_assert(kBTG == 1024 && DK == 64 && kC == 32, "laid out for 1,024 threads and d_k = 64");
    const int tid = threadIdx.x;
    const float *ks = a.KS + static_cast<size_t>(w) * ks_floats<DK>();
    // (the decay rule: every wavefront reads a float4 of P, and only P's own ones stage theirs;
    // an unconditional load keeps R in registers)
    R.m = reinterpret_cast<const float4 *>(ks)[DELTA ? tid : kC * kC / 2 + tid % (kC * kC / 4)];
    if (DELTA) R.w = ks[4 * kBTG + tid];
    if (tid < 3 * kC) R.gate = ks[3 * kC * kC + kC * DK + tid];
}
template <int DK, int DV, bool DELTA>
__device__ __forceinline__ void keyside_stage(const KsRows &R, ChunkLds<DK, DV> &s) {
    const int tid = threadIdx.x, e = 4 * tid, m = e / (kC * kC), i = e % (kC * kC);
    if (m < 3) {
        // (m is uniform over each wavefront)
        if (m == 2) *reinterpret_cast<float4 *>(&s.P[i / kC][i % kC]) = R.m;
        else if (DELTA && m == 1) *reinterpret_cast<float4 *>(&s.KG[i / kC][i % kC]) = R.m;
        else if (DELTA) *reinterpret_cast<float4 *>(&s.T[i / kC][i % kC]) = R.m;
    } else if (DELTA) {
        float *row = &s.W[i / DK][i % DK];
        *reinterpret_cast<float2 *>(row) = make_float2(R.m.x, R.m.y);
        *reinterpret_cast<float2 *>(row + 2) = make_float2(R.m.z, R.m.w);
    }
    if (DELTA) s.W[(kC * kC + tid) / DK][(kC * kC + tid) % DK] = R.w;
    if (tid < kC) s.G[tid] = R.gate;
    else if (tid < 2 * kC) s.gam[tid - kC] = R.gate;
    else if (tid < 3 * kC) s.eps[tid - 2 * kC] = R.gate;
}

// ---- F and R of every chunk ---------------------------------------------------
template <int DK, int DV, typename TIn, bool DELTA>
__global__ __launch_bounds__(kBTM) void bwd_map_kernel(BwdArgs a) {
    __shared__ ChunkLds<DK, DV> s;  // (its q rows become diag(gam) Q - P W)
    constexpr bool kHL = sizeof(TIn) == 2;  // bf16 inputs: hi/lo bf16 products
    const int w = blockIdx.x;
    {
        ChunkRows<kBTM, DK, DV, false> rows;
        chunk_load<kBTM, DK, DV, TIn, false>(a, w, rows);
        chunk_stage<kBTM, DK, DV, false>(rows, s, nullptr, nullptr, nullptr);
    }
    __syncthreads();
    chunk_keyside<DK, DV, DELTA, kHL>(s);
    {
        // the keyside, for the gradient kernel
        float *ks = a.KS + static_cast<size_t>(w) * ks_floats<DK>();
        for (int e = threadIdx.x; e < 3 * kC * kC / 4; e += kBTM) {
            const int m = e / (kC * kC / 4), r = (e / (kC / 4)) % kC, c = 4 * (e % (kC / 4));
            float4 *out = reinterpret_cast<float4 *>(ks) + e;
            if (m == 2) *out = *reinterpret_cast<const float4 *>(&s.P[r][c]);
            else if (DELTA && m == 1) *out = *reinterpret_cast<const float4 *>(&s.KG[r][c]);
            else if (DELTA) *out = *reinterpret_cast<const float4 *>(&s.T[r][c]);
        }
        if (DELTA)
            for (int e = threadIdx.x; e < kC * DK / 2; e += kBTM)
                reinterpret_cast<float2 *>(ks + 3 * kC * kC)[e] =
                    *reinterpret_cast<const float2 *>(&s.W[e / (DK / 2)][2 * (e % (DK / 2))]);
        if (threadIdx.x < 3 * kC) {
            const int r = threadIdx.x % kC, m = threadIdx.x / kC;
            ks[3 * kC * kC + kC * DK + threadIdx.x] = m == 0 ? s.G[r] : m == 1 ? s.gam[r] : s.eps[r];
        }
    }
    if (DELTA) {
        // in place: each element is read and rewritten by the thread that computes it, and the
        // product reads P and W only
        mm<kC, DK, kC, kHL>([&](int i, int j) { return s.P[i][j]; }, [&](int j, int c) { return s.W[j][c]; },
                       [&](int i, int c, float x) { s.q[i][c] = s.gam[i] * s.q[i][c] - x; });
    } else {
        for (int e = threadIdx.x; e < kC * DK; e += kBTM) s.q[e / DK][e % DK] *= s.gam[e / DK];
    }
    __syncthreads();
    const size_t base = static_cast<size_t>(w);
    float *R = a.R + base * DK * DV;
    const int half = static_cast<int>(blockDim.x) / 128;
    mm<DK, DV, kC, kHL>([&](int j, int r) { return s.q[r][j]; }, [&](int r, int i) { return s.dO[r][i]; },
                   [&](int j, int i, float x) { R[j * DV + i] = a.scale * x; }, 0, half);
    float *F = a.F + base * DK * DK;
    const float gl = s.gam[kC - 1];
    if (DELTA) {
        mm<DK, DK, kC, kHL>([&](int j, int r) { return s.W[r][j]; }, [&](int r, int m) { return s.eps[r] * s.k[r][m]; },
                       [&](int j, int m, float x) { F[j * DK + m] = (j == m ? gl : 0.f) - x; }, half, half);
    } else {
        for (int e = threadIdx.x; e < DK * DK; e += kBTM) F[e] = (e / DK == e % DK) ? gl : 0.f;
    }
}

// ---- reverse scan of the state gradient ------------------------------------------
// Y_{n-1} = F_n Y_n + R_n over the chunks [n0, n1) of one head, on the matrix cores, the
// columns of Y split over workgroups of kSW columns: wavefront w owns rows 16 w .. 16 w + 15.
// Its rows of F_n and R_n are loaded into registers one chunk ahead; within a block of 16
// keys, lane group lk takes keys 4 lk .. 4 lk + 3 (a float4 of F) and Y is read from LDS
// with the same key order.  Modes:
//   kScanAll   one range per head (all chunks, or all pieces when F and R are piece maps):
//              starts from the final-state gradient, stores Y at the end of every step's
//              chunk, writes the start-state gradient;
//   kScanMap   one range per piece: the piece's own map, on [constant | identity] columns
//              (the constant part starts at 0 and adds R, the identity part starts at I):
//              the result is the piece's affine map (G_p, c_p) with Y_start = G_p Y_end + c_p;
//   kScanPiece one range per piece: starts from the piece's end value and stores every
//              chunk's Y.
constexpr int kSW = 16;
enum { kScanAll = 0, kScanMap = 1, kScanPiece = 2 };

struct ScanArgs {
    const float *F, *R;      // [BH][steps][DK][DK], [BH][steps][DK][DV]
    float *Y;                // kScanAll / kScanPiece: [BH][steps][DK][DV], Y at the end of each step
    const float *y_end;      // kScanAll: final gradient [BH][DK][DV] (NULL = 0); kScanPiece: [BH][P][DK][DV]
    float *y_start;          // kScanAll: start gradient [BH][DK][DV] (NULL = not kept)
    float *Gp, *cp;          // kScanMap: piece maps [BH][P][DK][DK], [BH][P][DK][DV]
    int steps, m, P;         // steps per head, steps per piece, pieces per head
    int items;               // workgroups with work (the grid is rounded up to a multiple of 8)
};

// HL (bf16 inputs): the products F_n Y_n as three-pass hi/lo bf16 MFMA (F's rows already sit in
// the k-slot order kmap gives: slots 0-3 and 4-7 of step s are F's float4s 2 s and 2 s + 1)
template <int DK, int DV, int MODE, bool HL = false>
__global__ __launch_bounds__(kBT<DK>) void bwd_scan_kernel(ScanArgs a) {
    static_assert(DK % 16 == 0 && DV % kSW == 0, "one 16-row tile of Y per wavefront");
    constexpr int BT = kBT<DK>;
    constexpr int SW = kSW, YP = SW + 4, NCOL = MODE == kScanMap ? DV + DK : DV;
    constexpr int SLICES = NCOL / SW;
    __shared__ float Yb[2][DK][YP];
    // work items round-robin over the 8 XCDs so that the slices of one head and piece, which read
    // the same maps, run on one XCD at the same time and share its L2
    const int per_xcd = static_cast<int>(gridDim.x) / 8;
    const int w = static_cast<int>(blockIdx.x % 8) * per_xcd + static_cast<int>(blockIdx.x / 8);
    if (w >= a.items) return;
    const int slice = w % SLICES, rest = w / SLICES;
    const int piece = MODE == kScanAll ? 0 : rest % a.P;
    const int bh = MODE == kScanAll ? rest : rest / a.P;
    const int c0 = slice * SW, tid = threadIdx.x;
    const bool has_r = c0 < DV;  // constant columns take R; the identity part of a map does not
    const int lane = tid % 64, wave = tid / 64, li = lane % 16, lk = lane / 16, i0 = 16 * wave;
    const int n0 = MODE == kScanAll ? 0 : piece * a.m;
    const int n1 = MODE == kScanAll ? a.steps : min(n0 + a.m, a.steps);
    const size_t head = static_cast<size_t>(bh) * a.steps;
    const size_t hp = static_cast<size_t>(bh) * a.P + piece;
    for (int e = tid; e < DK * SW; e += BT) {
        const int j = e / SW, c = e % SW;
        float y = 0.f;
        if (MODE == kScanAll) y = a.y_end ? a.y_end[static_cast<size_t>(bh) * DK * DV + j * DV + c0 + c] : 0.f;
        if (MODE == kScanPiece) y = a.y_end[hp * DK * DV + j * DV + c0 + c];
        if (MODE == kScanMap && !has_r) y = (j == c0 - DV + c) ? 1.f : 0.f;
        Yb[0][j][c] = y;
    }
    // F and R of three steps in registers: step s reads the ones loaded two steps earlier, and
    // issues the loads of step s + 2 into the buffer step s - 1 read, so a load has two steps to
    // arrive (with one, every step waited on the memory latency: 3B-shaped 8K scan 795 us)
    float4 F0[DK / 16], F1[DK / 16], F2[DK / 16];
    f32x4 R0[SW / 16], R1[SW / 16], R2[SW / 16];
    auto load_f = [&](int n, float4 (&f)[DK / 16]) {
        const float *F = a.F + (head + n) * DK * DK + (i0 + li) * DK + 4 * lk;
#pragma unroll
        for (int blk = 0; blk < DK / 16; ++blk) f[blk] = *reinterpret_cast<const float4 *>(F + 16 * blk);
    };
    auto load_r = [&](int n, f32x4 (&r)[SW / 16]) {
        const float *R = a.R + (head + n) * DK * DV + c0;
#pragma unroll
        for (int t = 0; t < SW / 16; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) r[t][q] = has_r ? R[(i0 + 4 * lk + q) * DV + 16 * t + li] : 0.f;
    };
    const int S = n1 - n0;
    if (S > 0) {
        load_f(n1 - 1, F0);
        load_r(n1 - 1, R0);
    }
    if (S > 1) {
        load_f(n1 - 2, F1);
        load_r(n1 - 2, R1);
    }
    __syncthreads();
    auto step = [&](int s, const float4 (&Fc)[DK / 16], const f32x4 (&Rc)[SW / 16], float4 (&Fl)[DK / 16],
                    f32x4 (&Rl)[SW / 16]) {
        const int n = n1 - 1 - s, cur = s & 1;
        if (n - 2 >= n0) {
            load_f(n - 2, Fl);
            load_r(n - 2, Rl);
        }
        if (MODE != kScanMap) {  // this step's Y, before the update
            float *Yo = a.Y + (head + n) * DK * DV + c0;
            for (int e = lane; e < 16 * SW / 4; e += 64) {
                const int row = i0 + e / (SW / 4), c4 = e % (SW / 4);
                *reinterpret_cast<float4 *>(Yo + row * DV + 4 * c4) =
                    *reinterpret_cast<const float4 *>(&Yb[cur][row][4 * c4]);
            }
        }
        f32x4 acc[SW / 16];
#pragma unroll
        for (int t = 0; t < SW / 16; ++t) acc[t] = Rc[t];
        if constexpr (HL) {
#pragma unroll
            for (int s2 = 0; s2 < DK / 32; ++s2) {
                const float4 f0 = Fc[2 * s2], f1 = Fc[2 * s2 + 1];
                const float xa[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
                bf16x8 fh, fl;
                split_bf16(xa, fh, fl);
#pragma unroll
                for (int t = 0; t < SW / 16; ++t) {
                    float xb[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) xb[e] = Yb[cur][kmap(s2, lk, e)][16 * t + li];
                    bf16x8 yh, yl;
                    split_bf16(xb, yh, yl);
                    acc[t] = mfma_bf16(fh, yh, acc[t]);
                    acc[t] = mfma_bf16(fh, yl, acc[t]);
                    acc[t] = mfma_bf16(fl, yh, acc[t]);
                }
            }
        } else {
#pragma unroll
            for (int blk = 0; blk < DK / 16; ++blk) {
                const float fa[4] = {Fc[blk].x, Fc[blk].y, Fc[blk].z, Fc[blk].w};
#pragma unroll
                for (int mm = 0; mm < 4; ++mm)
#pragma unroll
                    for (int t = 0; t < SW / 16; ++t)
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[mm], Yb[cur][16 * blk + 4 * lk + mm][16 * t + li],
                                                                      acc[t], 0, 0, 0);
            }
        }
#pragma unroll
        for (int t = 0; t < SW / 16; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) Yb[cur ^ 1][i0 + 4 * lk + q][16 * t + li] = acc[t][q];
        __syncthreads();
    };
    for (int s = 0; s < S; s += 3) {
        step(s, F0, R0, F2, R2);
        if (s + 1 < S) step(s + 1, F1, R1, F0, R0);
        if (s + 2 < S) step(s + 2, F2, R2, F1, R1);
    }
    const int fin = (n1 - n0) & 1;
    if (MODE == kScanAll && a.y_start) {
        for (int e = tid; e < DK * SW; e += BT)
            a.y_start[static_cast<size_t>(bh) * DK * DV + (e / SW) * DV + c0 + e % SW] = Yb[fin][e / SW][e % SW];
    }
    if (MODE == kScanMap) {
        for (int e = tid; e < DK * SW; e += BT) {
            const int j = e / SW, c = e % SW;
            if (has_r) a.cp[hp * DK * DV + j * DV + c0 + c] = Yb[fin][j][c];
            else a.Gp[hp * DK * DK + j * DK + c0 - DV + c] = Yb[fin][j][c];
        }
    }
}

// ---- all gradients of one chunk -----------------------------------------------
// The gradient pass's matrices in two parts: GradLds always in LDS, GradBig in LDS for 64-wide
// heads and in a global scratch slot for 128-wide ones (the start state and its gradient alone are
// 128 KB there).
template <int DK, int DV> struct alignas(16) GradLds {
    float D[kC][DV + kPD];     // Delta
    float dD[kC][DV + kPD];    // dDelta
    float KY[kC][DV + kPD];    // K Y, later dW (DV == DK)
    float dPg[kC][kCP];      // dP .* Gam
    float X1[kC][kCP];       // dP .* P, later dA .* A
    float dT[kC][kCP];       // dT, later dA
    float Z[kC][kCP];        // dT T^T
    float red[9][kC];        // per-row reductions, combined into dG and db
    float red64[DK];         // row sums of Y .* S
    float dG[kC], dbv[kC];
};
template <int DK, int DV> struct alignas(16) GradBig {
    float v[kC][DV + kPD];
    float S[DK][DV + kPD], Yv[DK][DV + kPD];
    float TdW[kC][DK + kPD];   // T^T dW
    float TdU[kC][DV + kPD];   // T^T dDelta
};

// Independent products of a phase run side by side on disjoint wavefronts of the 16
// (ranges in the calls' last two arguments).
// The gradient phases of one chunk, from its staged rows, start state S, end-state gradient Y and
// keyside (the caller has synchronised after staging and zeroed u.red); tid = threadIdx.x.  s and u
// are LDS, or (u, for 128-wide heads) a global scratch slot of the workgroup's; the products are the
// same.
template <int DK, int DV, bool DELTA, bool HL>
__device__ __forceinline__ void grad_phases(const BwdArgs &a, ChunkLds<DK, DV> &s, GradLds<DK, DV> &u, GradBig<DK, DV> &g,
                                            size_t tok, int h, int L, int tid) {
    static_assert(DK == DV, "the dW buffer reuses K Y's");
    static_assert(kBTG == 1024, "the phases below are laid out for 16 wavefronts");
    // Delta = T diag(b) V - W S  (decay rule: diag(b) V);  K Y
    if (DELTA) {
        mm_t<kC, DV, kC, HL>(tid, [&](int i, int j) { return s.T[i][j]; }, [&](int j, int c) { return s.b[j] * g.v[j][c]; },
                       [&](int i, int c, float x) { u.D[i][c] = x; }, 0, 8);
    } else {
        for (int e = tid; e < kC * DV; e += kBTG) u.D[e / DV][e % DV] = s.b[e / DV] * g.v[e / DV][e % DV];
    }
    mm_t<kC, DV, DK, HL, 3>(tid, [&](int i, int j) { return s.k[i][j]; }, [&](int j, int c) { return g.Yv[j][c]; },
                   [&](int i, int c, float x) { u.KY[i][c] = x; }, 8, 8);
    __syncthreads();
    if (DELTA) {
        mm_t<kC, DV, DK, HL>(tid, [&](int i, int j) { return s.W[i][j]; }, [&](int j, int c) { return g.S[j][c]; },
                       [&](int i, int c, float x) { u.D[i][c] -= x; }, 0, 8);
        rowsum_t<DK, DV, HL>(tid, [&](int j, int i) { return g.Yv[j][i] * g.S[j][i]; }, [&](int j, float x) { u.red64[j] = x; },
                       8, 4);
        __syncthreads();
    }
    // dDelta = scale P^T dO + diag(eps) K Y;  dP = scale tril(dO Delta^T)
    mm_t<kC, DV, kC, HL>(tid, [&](int i, int r) { return s.P[r][i]; }, [&](int r, int c) { return s.dO[r][c]; },
                   [&](int i, int c, float x) { u.dD[i][c] = a.scale * x + s.eps[i] * u.KY[i][c]; }, 0, 8);
    mm_t<kC, kC, DV, HL>(tid, [&](int r, int c) { return s.dO[r][c]; }, [&](int c, int j) { return u.D[j][c]; },
                   [&](int r, int j, float x) {
                       const float dp = j <= r ? a.scale * x : 0.f;
                       u.dPg[r][j] = dp * (j <= r ? expf(s.G[r] - s.G[j]) : 0.f);
                       u.X1[r][j] = dp * s.P[r][j];
                   },
                   8, 4);
    if (!DELTA)
        rowsum_t<DK, DV, HL>(tid, [&](int j, int i) { return g.Yv[j][i] * g.S[j][i]; }, [&](int j, float x) { u.red64[j] = x; },
                       12, 4);
    __syncthreads();
    // row reductions for the gate and write-strength gradients: P, the end-state decay
    rowsum_t<kC, kC, HL>(tid, [&](int i, int k) { return u.X1[i][k]; }, [&](int i, float x) { u.red[0][i] = x; }, 8, 2);
    rowsum_t<kC, kC, HL>(tid, [&](int i, int k) { return u.X1[k][i]; }, [&](int i, float x) { u.red[1][i] = x; }, 10, 2);
    rowsum_t<kC, DV, HL>(tid, [&](int i, int c) { return u.KY[i][c] * u.D[i][c]; }, [&](int i, float x) { u.red[2][i] = x; }, 12, 2);

    // dQ = scale diag(gam) dO S^T (+ its gate term) + (dP .* Gam) K, into W's buffer
    mm_t<kC, DK, DV, HL>(tid, [&](int r, int i) { return s.dO[r][i]; }, [&](int i, int c) { return g.S[c][i]; },
                   [&](int r, int c, float x) { s.W[r][c] = a.scale * s.gam[r] * x; }, 0, 8);
    __syncthreads();
    rowsum_t<kC, DK, HL>(tid, [&](int i, int c) { return s.q[i][c] * s.W[i][c]; }, [&](int i, float x) { u.red[3][i] = x; }, 8, 2);
    mm_t<kC, DK, kC, HL, 5>(tid, [&](int r, int j) { return u.dPg[r][j]; }, [&](int j, int c) { return s.k[j][c]; },
                   [&](int r, int c, float x) {
                       if (r < L) a.dq[((tok + r) * a.H + h) * DK + c] = s.W[r][c] + x;
                   },
                   0, 8);
    // dW = -dDelta S^T (into K Y's buffer), T^T dDelta
    __syncthreads();
    if (DELTA) {
        mm_t<kC, DK, DV, HL>(tid, [&](int i, int l) { return u.dD[i][l]; }, [&](int l, int c) { return g.S[c][l]; },
                       [&](int i, int c, float x) { u.KY[i][c] = -x; }, 0, 8);
        mm_t<kC, DV, kC, HL>(tid, [&](int j, int i) { return s.T[i][j]; }, [&](int i, int c) { return u.dD[i][c]; },
                       [&](int j, int c, float x) { g.TdU[j][c] = x; }, 8, 8);
        __syncthreads();
        mm_t<kC, DK, kC, HL>(tid, [&](int j, int i) { return s.T[i][j]; }, [&](int i, int c) { return u.KY[i][c]; },
                       [&](int j, int c, float x) { g.TdW[j][c] = x; }, 0, 8);
        // dT = dW (diag(b gam) K)^T + dDelta (diag(b) V)^T
        mm_t<kC, kC, DK, HL>(tid, [&](int i, int c) { return u.KY[i][c]; },
                       [&](int c, int j) { return s.b[j] * s.gam[j] * s.k[j][c]; },
                       [&](int i, int j, float x) { u.dT[i][j] = x; }, 8, 4);
        __syncthreads();
        mm_t<kC, kC, DV, HL>(tid, [&](int i, int c) { return u.dD[i][c]; }, [&](int c, int j) { return s.b[j] * g.v[j][c]; },
                       [&](int i, int j, float x) { u.dT[i][j] += x; }, 0, 4);
        rowsum_t<kC, DK, HL>(tid, [&](int i, int c) { return g.TdW[i][c] * s.k[i][c]; }, [&](int i, float x) { u.red[7][i] = x; }, 4, 2);
        rowsum_t<kC, DV, HL>(tid, [&](int i, int c) { return g.TdU[i][c] * g.v[i][c]; }, [&](int i, float x) { u.red[8][i] = x; }, 6, 2);
        __syncthreads();
        // dA = -T^T (dT T^T), strictly lower
        mm_t<kC, kC, kC, HL>(tid, [&](int i, int l) { return u.dT[i][l]; }, [&](int l, int j) { return s.T[j][l]; },
                       [&](int i, int j, float x) { u.Z[i][j] = x; });
        __syncthreads();
        mm_t<kC, kC, kC, HL>(tid, [&](int i, int l) { return s.T[l][i]; }, [&](int l, int j) { return u.Z[l][j]; },
                       [&](int i, int j, float x) {
                           const float da = j < i ? -x : 0.f;
                           u.dT[i][j] = da;                        // dA
                           u.X1[i][j] = da * s.b[i] * s.KG[i][j];  // dA .* A
                       });
        __syncthreads();
        rowsum_t<kC, kC, HL>(tid, [&](int i, int k) { return u.X1[i][k]; }, [&](int i, float x) { u.red[4][i] = x; }, 0, 2);
        rowsum_t<kC, kC, HL>(tid, [&](int i, int k) { return u.X1[k][i]; }, [&](int i, float x) { u.red[5][i] = x; }, 2, 2);
        rowsum_t<kC, kC, HL>(tid, [&](int i, int k) { return u.dT[i][k] * s.KG[i][k]; }, [&](int i, float x) { u.red[6][i] = x; }, 4, 2);
        // E = diag(b) dA .* Gam, kept in Z
        for (int e = tid; e < kC * kC; e += kBTG) {
            const int i = e / kC, j = e % kC;
            u.Z[i][j] = j < i ? s.b[i] * u.dT[i][j] * expf(s.G[i] - s.G[j]) : 0.f;
        }
    } else {
        rowsum_t<kC, DV, HL>(tid, [&](int i, int c) { return u.dD[i][c] * g.v[i][c]; }, [&](int i, float x) { u.red[8][i] = x; }, 6, 2);
    }
    __syncthreads();
    // combine: dG per position, db, and the last position's end-state terms (one wavefront)
    if (tid < 64) {
        float ys = 0.f;
        for (int j = tid; j < DK; j += 64) ys += u.red64[j];
        float last = s.gam[kC - 1] * ys;
        if (tid < kC) {
            const int r = tid;
            const float e = s.eps[r] * u.red[2][r];
            float dg = u.red[0][r] - u.red[1][r] - e + u.red[3][r];
            float db = u.red[8][r];
            if (DELTA) {
                dg += u.red[4][r] - u.red[5][r] + s.b[r] * s.gam[r] * u.red[7][r];
                db += s.gam[r] * u.red[7][r] + u.red[6][r];
            }
            u.dG[r] = dg;
            u.dbv[r] = db;
            last += e;
        }
        for (int m = 32; m >= 1; m >>= 1) last += __shfl_xor(last, m);
        if (tid == kC - 1) u.dG[kC - 1] += last;
    }
    // dV = diag(b) T^T dDelta (decay rule: diag(b) dDelta)
    for (int e = tid; e < kC * DV; e += kBTG) {
        const int r = e / DV, c = e % DV;
        if (r < L) a.dv[((tok + r) * a.H + h) * DV + c] = s.b[r] * (DELTA ? g.TdU[r][c] : u.dD[r][c]);
    }
    // dK = (dP .* Gam)^T Q + diag(eps) Delta Y^T [+ diag(b gam) T^T dW + E K + E^T K]
    mm_t<kC, DK, kC, HL, 5>(tid, [&](int j, int r) { return u.dPg[r][j]; }, [&](int r, int c) { return s.q[r][c]; },
                   [&](int j, int c, float x) { s.W[j][c] = x; }, 8, 8);
    __syncthreads();
    // dg: reverse cumulative sum of dG inside the chunk (upper-triangular ones); dbeta
    mm_t<kC, 16, kC>(tid, [](int i, int j) { return j >= i ? 1.f : 0.f; }, [&](int j, int) { return u.dG[j]; },
                   [&](int i, int c, float x) { if (c == 0 && i < L) a.dg[(tok + i) * a.H + h] = x; }, 0, 2);
    if (tid < L) a.dbeta[(tok + tid) * a.H + h] = u.dbv[tid];
    mm_t<kC, DK, DV, HL>(tid, [&](int j, int i) { return u.D[j][i]; }, [&](int i, int c) { return g.Yv[c][i]; },
                   [&](int j, int c, float x) { s.W[j][c] += s.eps[j] * x; }, 8, 8);
    __syncthreads();
    if (DELTA) {
        mm_t<kC, DK, kC, HL, 5>(tid, [&](int i, int j) { return u.Z[i][j] + u.Z[j][i]; }, [&](int j, int c) { return s.k[j][c]; },
                       [&](int i, int c, float x) { s.W[i][c] += x + s.b[i] * s.gam[i] * g.TdW[i][c]; }, 8, 8);
        __syncthreads();
    }
    for (int e = tid; e < kC * DK; e += kBTG) {
        const int r = e / DK, c = e % DK;
        if (r < L) a.dk[((tok + r) * a.H + h) * DK + c] = s.W[r][c];
    }
}

template <int DK, int DV, typename TIn, bool DELTA>
__global__ __launch_bounds__(kBTG) void bwd_grad_kernel(BwdArgs a) {
    __shared__ ChunkLds<DK, DV> s;
    __shared__ GradLds<DK, DV> u;
    __shared__ GradBig<DK, DV> g;
    const int tid = threadIdx.x;
    const int w = blockIdx.x;
    const ChunkPos pos = chunk_pos(a, w);
    {
        // the chunk's rows and the keyside its map pass stored
        ChunkRows<kBTG, DK, DV, true> rows;
        KsRows ks{};
        chunk_load<kBTG, DK, DV, TIn, true>(a, w, rows);
        keyside_load<DK, DELTA>(a, w, ks);
        chunk_stage<kBTG, DK, DV, true>(rows, s, g.v, g.S, g.Yv);
        keyside_stage<DK, DV, DELTA>(ks, s);
    }
    if (tid < kC)
        for (int m = 0; m < 9; ++m) u.red[m][tid] = 0.f;
    __syncthreads();
    grad_phases<DK, DV, DELTA, sizeof(TIn) == 2>(a, s, u, g, pos.tok, pos.h, pos.L, tid);
}

// 128-wide heads: the chunk rows, keyside and the chunk-sized intermediates in LDS (151 KB), the
// start state, its gradient, V and the two T^T products (183 KB) in the workgroup's global scratch
// slot; the workgroups loop over the chunks.  Each chunk's products take a thread id read anew for
// that chunk: with threadIdx.x itself the compiler keeps their addresses live across the loop and
// spills 107 registers (3B-shaped 8K call 3.04 -> 2.75 ms).
template <int DK, int DV, typename TIn, bool DELTA>
__global__ __launch_bounds__(kBTG) void bwd_grad_gs_kernel(BwdArgs a, GradBig<DK, DV> *scratch) {
    __shared__ ChunkLds<DK, DV> s;
    __shared__ GradLds<DK, DV> u;
    GradBig<DK, DV> &g = scratch[blockIdx.x];
    const int tid = threadIdx.x;
    const TIn *q = static_cast<const TIn *>(a.q), *k = static_cast<const TIn *>(a.k), *v = static_cast<const TIn *>(a.v);
    for (int w = blockIdx.x; w < a.BH * a.N; w += gridDim.x) {
        const ChunkPos p = chunk_pos(a, w);
        for (int e = tid; e < kC * DK; e += kBTG) {
            const int r = e / DK, c = e % DK;
            const size_t x = ((p.tok + r) * a.H + p.h) * DK + c;
            s.q[r][c] = r < p.L ? load_in(q, x) : 0.f;
            s.k[r][c] = r < p.L ? load_in(k, x) : 0.f;
        }
        for (int e = tid; e < kC * DV; e += kBTG) {
            const int r = e / DV, c = e % DV;
            const size_t x = ((p.tok + r) * a.H + p.h) * DV + c;
            s.dO[r][c] = r < p.L ? a.d_o[x] : 0.f;
            g.v[r][c] = r < p.L ? load_in(v, x) : 0.f;
        }
        const size_t sx = static_cast<size_t>(w) * DK * DV;
        for (int e = tid; e < DK * DV; e += kBTG) {
            g.S[e / DV][e % DV] = a.states[sx + e];
            g.Yv[e / DV][e % DV] = a.Y[sx + e];
        }
        // the keyside its map pass stored: T, KG, P (C x C each), W (C x DK), G, gam, eps
        const float *ks = a.KS + static_cast<size_t>(w) * ks_floats<DK>();
        for (int e = tid; e < kC * kC; e += kBTG) {
            const int r = e / kC, c = e % kC;
            if (DELTA) {
                s.T[r][c] = ks[e];
                s.KG[r][c] = ks[kC * kC + e];
            }
            s.P[r][c] = ks[2 * kC * kC + e];
        }
        if (DELTA)
            for (int e = tid; e < kC * DK; e += kBTG) s.W[e / DK][e % DK] = ks[3 * kC * kC + e];
        if (tid < kC) {
            const float *gates = ks + 3 * kC * kC + kC * DK;
            s.G[tid] = gates[tid];
            s.gam[tid] = gates[kC + tid];
            s.eps[tid] = gates[2 * kC + tid];
            s.b[tid] = tid < p.L ? a.beta[(p.tok + tid) * a.H + p.h] : 0.f;
            for (int m = 0; m < 9; ++m) u.red[m][tid] = 0.f;
        }
        __syncthreads();
        grad_phases<DK, DV, DELTA, sizeof(TIn) == 2>(a, s, u, g, p.tok, p.h, p.L, thread_id());
        __syncthreads();  // the next chunk restages s and u
    }
}

// Pieces for the reverse scan: none when the heads alone give enough workgroups or the
// sequence is short (the pieces triple the work: their maps run on twice the columns); else
// about sqrt(N) chunks per piece (three short sequential passes).  128-wide heads have twice
// the columns per head and four times the work per step, so the pieces pay later: a 3B-shaped
// 8K call (24 heads, 256 chunks) takes 4.86 ms with one level against 5.39 ms with two.
struct ScanPlan {
    int m, P;  // chunks per piece, pieces per head (P = 1: one range per head)
};
ScanPlan scan_plan(int BH, int N, int dk) {
    if (N < 128 || BH * (64 / kSW) >= 256) return {N, 1};  // heads alone fill the 256 CUs
    if (dk == 128 && N < 1024) return {N, 1};
    int m = 16;
    while (m * m < N) m *= 2;
    return {m, (N + m - 1) / m};
}

// 128-wide heads: the gradient pass keeps its larger matrices in global scratch, one slot per
// workgroup (one workgroup per compute unit: 81 KB of LDS)
template <int DK, int DV> constexpr bool kGradGlobal = DK == 128;
constexpr int kGradSlots = 256;

template <int DK, int DV, bool DELTA>
hipError_t run_backward(BwdArgs &a, gdn_dtype dt, const ScanPlan &plan, float *Gp, float *cp, float *yend,
                        hipStream_t stream) {
    const int items = a.BH * a.N;
    const bool bf = dt == GDN_BF16;
    if (items > 0) {
        if (bf) hipLaunchKernelGGL((bwd_map_kernel<DK, DV, uint16_t, DELTA>), dim3(items), dim3(kBTM), 0, stream, a);
        else hipLaunchKernelGGL((bwd_map_kernel<DK, DV, float, DELTA>), dim3(items), dim3(kBTM), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    auto grid8 = [](int items) { return dim3((items + 7) / 8 * 8); };
    ScanArgs sa{};
    sa.F = a.F; sa.R = a.R; sa.Y = a.Y; sa.steps = a.N;
    if (plan.P == 1) {
        sa.y_end = a.ds_final; sa.y_start = a.ds0; sa.m = a.N; sa.P = 1;
        sa.items = a.BH * (DV / kSW);
        if (bf) hipLaunchKernelGGL((bwd_scan_kernel<DK, DV, kScanAll, true>), grid8(sa.items), dim3(kBT<DK>), 0, stream, sa);
        else hipLaunchKernelGGL((bwd_scan_kernel<DK, DV, kScanAll, false>), grid8(sa.items), dim3(kBT<DK>), 0, stream, sa);
    } else {
        // piece maps, then the chain over pieces (the same scan with piece maps as its steps), then
        // every chunk's Y inside each piece from the piece's end value
        sa.m = plan.m; sa.P = plan.P; sa.Gp = Gp; sa.cp = cp;
        sa.items = a.BH * plan.P * ((DV + DK) / kSW);
        if (bf) hipLaunchKernelGGL((bwd_scan_kernel<DK, DV, kScanMap, true>), grid8(sa.items), dim3(kBT<DK>), 0, stream, sa);
        else hipLaunchKernelGGL((bwd_scan_kernel<DK, DV, kScanMap, false>), grid8(sa.items), dim3(kBT<DK>), 0, stream, sa);
        ScanArgs ch{};
        ch.F = Gp; ch.R = cp; ch.Y = yend; ch.y_end = a.ds_final; ch.y_start = a.ds0;
        ch.steps = plan.P; ch.m = plan.P; ch.P = 1;
        ch.items = a.BH * (DV / kSW);
        if (bf) hipLaunchKernelGGL((bwd_scan_kernel<DK, DV, kScanAll, true>), grid8(ch.items), dim3(kBT<DK>), 0, stream, ch);
        else hipLaunchKernelGGL((bwd_scan_kernel<DK, DV, kScanAll, false>), grid8(ch.items), dim3(kBT<DK>), 0, stream, ch);
        sa.y_end = yend;
        sa.items = a.BH * plan.P * (DV / kSW);
        if (bf) hipLaunchKernelGGL((bwd_scan_kernel<DK, DV, kScanPiece, true>), grid8(sa.items), dim3(kBT<DK>), 0, stream, sa);
        else hipLaunchKernelGGL((bwd_scan_kernel<DK, DV, kScanPiece, false>), grid8(sa.items), dim3(kBT<DK>), 0, stream, sa);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || items == 0) return e;
    if constexpr (kGradGlobal<DK, DV>) {
        auto *slots = static_cast<GradBig<DK, DV> *>(a.gscratch);
        const dim3 grid(items < kGradSlots ? items : kGradSlots);
        if (bf) hipLaunchKernelGGL((bwd_grad_gs_kernel<DK, DV, uint16_t, DELTA>), grid, dim3(kBTG), 0, stream, a, slots);
        else hipLaunchKernelGGL((bwd_grad_gs_kernel<DK, DV, float, DELTA>), grid, dim3(kBTG), 0, stream, a, slots);
    } else {
        if (bf) hipLaunchKernelGGL((bwd_grad_kernel<DK, DV, uint16_t, DELTA>), dim3(items), dim3(kBTG), 0, stream, a);
        else hipLaunchKernelGGL((bwd_grad_kernel<DK, DV, float, DELTA>), dim3(items), dim3(kBTG), 0, stream, a);
    }
    return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

struct BwdLayout {
    size_t fwd, o, sfin, states, F, R, Y, KS, Gp, cp, yend, gs, total;
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
    L.KS = off; off += align256(BH * N * (dk == 128 ? ks_floats<128>() : ks_floats<64>()) * 4);
    const ScanPlan plan = scan_plan(static_cast<int>(BH), static_cast<int>(N), dk);
    const size_t PP = plan.P > 1 ? static_cast<size_t>(plan.P) : 0;
    L.Gp = off; off += align256(BH * PP * dk * dk * 4);
    L.cp = off; off += align256(BH * PP * dk * dv * 4);
    L.yend = off; off += align256(BH * PP * dk * dv * 4);
    L.gs = off; off += dk == 128 ? align256(kGradSlots * sizeof(GradBig<128, 128>)) : 0;
    L.total = off;
    return L;
}

}  // namespace

bool backward_supported(int dk, int dv, gdn_dtype dt) {
    return dk == dv && (dk == 64 || dk == 128) && (dt == GDN_BF16 || dt == GDN_F32);
}

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
    a.KS = reinterpret_cast<float *>(w + L.KS);
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.ds0 = ds0;
    a.T = T; a.H = H; a.BH = B * H; a.N = (T + kC - 1) / kC;
    a.scale = 1.0f / sqrtf(static_cast<float>(d_k));
    a.gscratch = w + L.gs;
    if (T > 0 && dt == GDN_F32) {
        // fp32 q/k/v: the fp32 chunk kernel, again keeping every chunk's start state
        hipError_t e = launch_prefill_valu(q, k, v, g, beta, s0, reinterpret_cast<float *>(w + L.o),
                                           reinterpret_cast<float *>(w + L.sfin), B, T, H, d_k, d_v, kC, dt, delta,
                                           stream, reinterpret_cast<float *>(w + L.states));
        if (e != hipSuccess) return e;
    } else if (T > 0) {
        // forward pass again, keeping the state every chunk starts from
        hipError_t e = launch_prefill_chunk(static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                                            static_cast<const uint16_t *>(v), g, beta, s0,
                                            reinterpret_cast<float *>(w + L.o), reinterpret_cast<float *>(w + L.sfin),
                                            B, T, H, d_k, d_v, kC, delta, w + L.fwd, stream,
                                            reinterpret_cast<float *>(w + L.states));
        if (e != hipSuccess) return e;
    }
    const ScanPlan plan = scan_plan(a.BH, a.N, d_k);
    float *Gp = reinterpret_cast<float *>(w + L.Gp), *cp = reinterpret_cast<float *>(w + L.cp);
    float *yend = reinterpret_cast<float *>(w + L.yend);
    if (d_k == 128)
        return delta ? run_backward<128, 128, true>(a, dt, plan, Gp, cp, yend, stream)
                     : run_backward<128, 128, false>(a, dt, plan, Gp, cp, yend, stream);
    return delta ? run_backward<64, 64, true>(a, dt, plan, Gp, cp, yend, stream)
                 : run_backward<64, 64, false>(a, dt, plan, Gp, cp, yend, stream);
}

}  // namespace gdn
