// gdn_prefill_bf16.hip -- chunked GDN prefill for bf16 q/k/v on MFMA (gfx950).
//
// Chunk form of the gated delta rule (derived from the rule; the pages give
// no chunked algorithm).  For a chunk of C tokens with start state
// St = S0^T (d_k x d_v, fp32) and G_r = sum_{i<=r} g_i (within the chunk):
//   A     = strict_tril(diag(b) (K K^T .* exp(G_r - G_j)))
//   T     = (I + A)^{-1}                       forward substitution
//   W     = T diag(b exp(G)) K,   U = T diag(b) V
//   Delta = U - W St                           (row r = delta_r of the rule)
//   O     = scale (diag(exp(G)) Q St + (Q K^T .* exp(G_r - G_j) .* tril) Delta)
//   St'   = exp(G_C) St + K^T diag(exp(G_C - G)) Delta
//
// Three kernels, queued in order on the caller's stream:
//   prep   (one workgroup per chunk)   G, K K^T, A, T, W, U
//   scan   (one wavefront per 16-column value slice of a head; serial over
//           chunks, state in registers)  Delta, St per chunk
//   output (one workgroup per chunk)   Q K^T, O
// Intermediates pass through the caller's workspace in MFMA fragment order
// (see gdn_mfma.h), so the scan reads every operand with one 16-byte load
// per lane and keeps the state and Delta in registers.
//
// Precision: q/k/v are bf16, so K K^T and Q K^T are exact products with fp32
// accumulation.  Operands derived in fp32 are rounded to bf16 only where the
// result tolerates it -- W and the state in the W St product -- and are split
// into hi + lo bf16 pairs where it does not: T diag(b) in U, the state in
// Q St, P and Delta in P Delta, and the decayed Delta in the state update.
// Decays are exponentials of non-positive differences of cumulative gates,
// masked before exponentiation.
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int kWave = 64;
constexpr int kBlock = 256;
constexpr int kPad = 8;  // bf16 row padding in LDS

template <int DK, int DV, int C>
struct Geo {
    static constexpr int CT = C / 16;   // 16-row tiles over a chunk
    static constexpr int CS = C / 32;   // k-steps over chunk rows
    static constexpr int KT = DK / 16;  // 16-row tiles over d_k
    static constexpr int KS = DK / 32;  // k-steps over d_k
    static constexpr int VT = DV / 16;  // 16-column value slices
    static constexpr int NB = C / 16;   // diagonal blocks of T
    // per-chunk workspace element counts
    static constexpr size_t WF = static_cast<size_t>(C) * DK;   // bf16, W A-fragments
    static constexpr size_t KF = static_cast<size_t>(DK) * C;   // bf16, K^T A-fragments
    static constexpr size_t UF = static_cast<size_t>(C) * DV;   // fp32, U tiles
    static constexpr size_t GW = C;                             // fp32, cumulative gates
    static constexpr size_t SN = static_cast<size_t>(DK) * DV;  // fp32, chunk start state tiles
    static constexpr size_t DF = static_cast<size_t>(C) * DV;   // fp32, Delta tiles
};

struct Ws {
    uint16_t *wf;
    uint16_t *kf;
    float *uf;
    float *gw;
    float *sn;
    float *df;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

template <int DK, int DV, int C>
size_t ws_bytes(size_t chunks) {
    using G = Geo<DK, DV, C>;
    return align256(chunks * G::WF * 2) + align256(chunks * G::KF * 2) + align256(chunks * G::UF * 4) +
           align256(chunks * G::GW * 4) + align256(chunks * G::SN * 4) + align256(chunks * G::DF * 4);
}

template <int DK, int DV, int C>
Ws ws_carve(void *base, size_t chunks) {
    using G = Geo<DK, DV, C>;
    char *p = static_cast<char *>(base);
    Ws w;
    w.wf = reinterpret_cast<uint16_t *>(p); p += align256(chunks * G::WF * 2);
    w.kf = reinterpret_cast<uint16_t *>(p); p += align256(chunks * G::KF * 2);
    w.uf = reinterpret_cast<float *>(p);    p += align256(chunks * G::UF * 4);
    w.gw = reinterpret_cast<float *>(p);    p += align256(chunks * G::GW * 4);
    w.sn = reinterpret_cast<float *>(p);    p += align256(chunks * G::SN * 4);
    w.df = reinterpret_cast<float *>(p);
    return w;
}

// Column fragment of a row-major bf16 LDS matrix M: slots e hold
// M[kmap(s, gq, e)][col], i.e. an operand whose k index runs over M's rows.
__device__ __forceinline__ bf16x8 lds_colfrag(const uint16_t *m, int stride, int col, int s, int gq) {
    u16x8 u;
#pragma unroll
    for (int e = 0; e < 8; ++e) u[e] = m[kmap(s, gq, e) * stride + col];
    return as_bf16x8(u);
}

// Copies rows [t0, t0+L) of a [.., T, H, D] bf16 tensor for head (b, h) into a
// C x (D + kPad) LDS tile, zero-filling rows >= L.
template <int D, int C>
__device__ __forceinline__ void load_rows(uint16_t (*dst)[D + kPad], const uint16_t *src, int b,
                                          int h, int t0, int L, int T, int H) {
    for (int e = threadIdx.x; e < C * D / 8; e += kBlock) {
        const int r = e / (D / 8), c8 = e % (D / 8);
        u16x8 val = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < L)
            val = *reinterpret_cast<const u16x8 *>(
                src + ((static_cast<size_t>(b) * T + t0 + r) * H + h) * D + 8 * c8);
        *reinterpret_cast<u16x8 *>(&dst[r][8 * c8]) = val;
    }
}

// ---------------------------------------------------------------------------
// prep: G, A, T = (I + A)^{-1}, W and U for one chunk.
// ---------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kBlock) void prep_kernel(const uint16_t *__restrict__ k,
                                                      const uint16_t *__restrict__ v,
                                                      const float *__restrict__ g,
                                                      const float *__restrict__ beta, Ws ws, int T,
                                                      int H, int N) {
    using G = Geo<DK, DV, C>;
    __shared__ __align__(16) uint16_t Ks[C][DK + kPad];
    __shared__ __align__(16) float Tm[C][C + 4];   // T = (I + A)^{-1}
    // A (strictly lower) while T is built, then the V rows
    __shared__ __align__(16) char avbuf[(C * (C + 4) * 4 > C * (DV + kPad) * 2) ? C * (C + 4) * 4
                                                                                : C * (DV + kPad) * 2];
    __shared__ __align__(16) float Xs[4][16][16 + 4];  // per-wave block-product scratch
    __shared__ float Gs[C], bs[C], bgs[C];
    float(*As)[C + 4] = reinterpret_cast<float(*)[C + 4]>(avbuf);
    uint16_t(*Vs)[DV + kPad] = reinterpret_cast<uint16_t(*)[DV + kPad]>(avbuf);

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int gq = lane / 16, li = lane % 16;
    const int n = blockIdx.x % N;
    const size_t bh = blockIdx.x / N;
    const int b = static_cast<int>(bh / H), h = static_cast<int>(bh % H);
    const int t0 = n * C;
    const int L = min(C, T - t0);
    const size_t chunk = bh * N + n;

    load_rows<DK, C>(Ks, k, b, h, t0, L, T, H);
    for (int e = tid; e < C * (C + 4); e += kBlock) {
        (&Tm[0][0])[e] = 0.f;
        (&As[0][0])[e] = 0.f;
    }
    if (wave == 0) {
        // inclusive prefix sum of the gates; rows >= L add 0, so they repeat G_{L-1}
        float x = (lane < L) ? g[(static_cast<size_t>(b) * T + t0 + lane) * H + h] : 0.f;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float y = __shfl_up(x, off, kWave);
            if (lane >= off) x += y;
        }
        if (lane < C) {
            const float bb = (lane < L) ? beta[(static_cast<size_t>(b) * T + t0 + lane) * H + h] : 0.f;
            Gs[lane] = x;
            bs[lane] = bb;
            bgs[lane] = bb * __expf(x);
            ws.gw[chunk * G::GW + lane] = x;
        }
    }
    __syncthreads();

    // A = strict_tril(diag(b) (K K^T .* exp(G_r - G_j))), lower 16x16 tiles
    constexpr int LT = G::CT * (G::CT + 1) / 2;
    for (int t = wave; t < LT; t += 4) {
        int mt = 0, rem = t;
        while (rem > mt) rem -= ++mt;
        const int nt = rem;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < G::KS; ++s)
            acc = mfma_bf16(lds_frag_bf16(&Ks[16 * mt + li][0], s, gq),
                            lds_frag_bf16(&Ks[16 * nt + li][0], s, gq), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * gq + r, col = 16 * nt + li;
            As[row][col] = (row > col && row < L) ? bs[row] * acc[r] * __expf(Gs[row] - Gs[col]) : 0.f;
        }
    }
    __syncthreads();

    // T: diagonal 16x16 blocks by forward substitution, one column per lane
    if (wave == 0 && gq < G::NB) {
        const int a = gq, j = li;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) acc += As[16 * a + r][16 * a + m] * t[m];
            t[r] = (r == j) ? 1.f : -acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) Tm[16 * a + r][16 * a + j] = t[r];
    }
    __syncthreads();

    // T: off-diagonal blocks, T_ac = -T_aa sum_{c<=m<a} A_am T_mc, by distance a - c
    for (int dist = 1; dist < G::NB; ++dist) {
        const int c = wave, a = wave + dist;
        const bool active = a < G::NB;
        const int rr = lane / 4, c4 = 4 * (lane % 4);
        if (active) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            for (int m = c; m < a; ++m)
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    x += As[16 * a + rr][16 * m + kk] *
                         *reinterpret_cast<const f32x4 *>(&Tm[16 * m + kk][16 * c + c4]);
            *reinterpret_cast<f32x4 *>(&Xs[wave][rr][c4]) = x;
        }
        __syncthreads();
        if (active) {
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 16; ++kk)
                y += Tm[16 * a + rr][16 * a + kk] * *reinterpret_cast<const f32x4 *>(&Xs[wave][kk][c4]);
            *reinterpret_cast<f32x4 *>(&Tm[16 * a + rr][16 * c + c4]) = -y;
        }
        __syncthreads();
    }

    // V rows replace A
    load_rows<DV, C>(Vs, v, b, h, t0, L, T, H);
    __syncthreads();

    // W^T = K^T diag(b exp(G)) T^T, written as the scan's W A-fragments:
    // fragment (ct, s2) of lane = W^T tiles (2 s2, ct) and (2 s2 + 1, ct).
    for (int p = wave; p < G::CT * G::KS; p += 4) {
        const int ct = p % G::CT, s2 = p / G::CT;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
        for (int s = 0; s < G::CS; ++s) {
            float x[8];
            lds_slots_f32(&Tm[16 * ct + li][0], s, gq, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= bgs[kmap(s, gq, e)];
            const bf16x8 bfr = pack_bf16(x);
            acc0 = mfma_bf16(lds_colfrag(&Ks[0][0], DK + kPad, 16 * (2 * s2) + li, s, gq), bfr, acc0);
            acc1 = mfma_bf16(lds_colfrag(&Ks[0][0], DK + kPad, 16 * (2 * s2 + 1) + li, s, gq), bfr, acc1);
        }
        float x[8];
        acc_pair_to_slots(acc0, acc1, x);
        *reinterpret_cast<bf16x8 *>(ws.wf + chunk * G::WF + ((ct * G::KS + s2) * kWave + lane) * 8) =
            pack_bf16(x);
    }
    // K^T A-fragments for the scan's state update (k runs over chunk rows)
    for (int p = wave; p < G::KT * G::CS; p += 4) {
        const int mt = p / G::CS, s = p % G::CS;
        *reinterpret_cast<bf16x8 *>(ws.kf + chunk * G::KF + ((mt * G::CS + s) * kWave + lane) * 8) =
            lds_colfrag(&Ks[0][0], DK + kPad, 16 * mt + li, s, gq);
    }
    // U = (T diag(b)) V with T diag(b) split into hi + lo bf16
    for (int p = wave; p < G::CT * G::VT; p += 4) {
        const int mt = p % G::CT, nt = p / G::CT;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < G::CS; ++s) {
            float x[8];
            lds_slots_f32(&Tm[16 * mt + li][0], s, gq, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] *= bs[kmap(s, gq, e)];
            bf16x8 hi, lo;
            split_bf16(x, hi, lo);
            const bf16x8 vb = lds_colfrag(&Vs[0][0], DV + kPad, 16 * nt + li, s, gq);
            acc = mfma_bf16(hi, vb, acc);
            acc = mfma_bf16(lo, vb, acc);
        }
        *reinterpret_cast<f32x4 *>(ws.uf + chunk * G::UF + ((nt * G::CT + mt) * kWave + lane) * 4) = acc;
    }
}

// ---------------------------------------------------------------------------
// scan: serial over chunks for one 16-column value slice of one head.
// Lane (gq, li) keeps St[16 mt + 4 gq + r][16 slice + li] in St[mt][r].
// ---------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kWave) void scan_kernel(Ws ws, const float *__restrict__ s0,
                                                     float *__restrict__ s_out, int N) {
    using G = Geo<DK, DV, C>;
    const int lane = threadIdx.x, gq = lane / 16, li = lane % 16;
    const int slice = blockIdx.x % G::VT;
    const size_t bh = blockIdx.x / G::VT;
    const int col = 16 * slice + li;

    f32x4 St[G::KT];
#pragma unroll
    for (int mt = 0; mt < G::KT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            St[mt][r] = s0 ? s0[(bh * DK + 16 * mt + 4 * gq + r) * DV + col] : 0.f;

    for (int n = 0; n < N; ++n) {
        const size_t chunk = bh * N + n;
#pragma unroll
        for (int mt = 0; mt < G::KT; ++mt)
            *reinterpret_cast<f32x4 *>(ws.sn + chunk * G::SN + ((slice * G::KT + mt) * kWave + lane) * 4) =
                St[mt];

        bf16x8 Sb[G::KS];
#pragma unroll
        for (int s = 0; s < G::KS; ++s) {
            float x[8];
            acc_pair_to_slots(St[2 * s], St[2 * s + 1], x);
            Sb[s] = pack_bf16(x);
        }

        const float *Gc = ws.gw + chunk * G::GW;
        const float glast = Gc[C - 1];
        f32x4 D[G::CT];
#pragma unroll
        for (int ct = 0; ct < G::CT; ++ct) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < G::KS; ++s)
                acc = mfma_bf16(*reinterpret_cast<const bf16x8 *>(
                                    ws.wf + chunk * G::WF + ((ct * G::KS + s) * kWave + lane) * 8),
                                Sb[s], acc);
            const f32x4 u = *reinterpret_cast<const f32x4 *>(
                ws.uf + chunk * G::UF + ((slice * G::CT + ct) * kWave + lane) * 4);
            D[ct] = u - acc;
            *reinterpret_cast<f32x4 *>(ws.df + chunk * G::DF + ((slice * G::CT + ct) * kWave + lane) * 4) =
                D[ct];
#pragma unroll
            for (int r = 0; r < 4; ++r) D[ct][r] *= __expf(glast - Gc[16 * ct + 4 * gq + r]);
        }

        bf16x8 Dh[G::CS], Dl[G::CS];
#pragma unroll
        for (int s = 0; s < G::CS; ++s) {
            float x[8];
            acc_pair_to_slots(D[2 * s], D[2 * s + 1], x);
            split_bf16(x, Dh[s], Dl[s]);
        }
        const float gl = __expf(glast);
#pragma unroll
        for (int mt = 0; mt < G::KT; ++mt) {
            f32x4 acc = gl * St[mt];
#pragma unroll
            for (int s = 0; s < G::CS; ++s) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                    ws.kf + chunk * G::KF + ((mt * G::CS + s) * kWave + lane) * 8);
                acc = mfma_bf16(a, Dh[s], acc);
                acc = mfma_bf16(a, Dl[s], acc);
            }
            St[mt] = acc;
        }
    }

#pragma unroll
    for (int mt = 0; mt < G::KT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_out[(bh * DK + 16 * mt + 4 * gq + r) * DV + col] = St[mt][r];
}

// ---------------------------------------------------------------------------
// output: O = scale (diag(exp(G)) Q St + P Delta) for one chunk.
// ---------------------------------------------------------------------------
template <int DK, int DV, int C>
__global__ __launch_bounds__(kBlock) void output_kernel(const uint16_t *__restrict__ q,
                                                        const uint16_t *__restrict__ k, Ws ws,
                                                        float *__restrict__ o, int T, int H, int N,
                                                        float scale) {
    using G = Geo<DK, DV, C>;
    __shared__ __align__(16) uint16_t Qs[C][DK + kPad];
    __shared__ __align__(16) uint16_t Ks[C][DK + kPad];
    __shared__ __align__(16) float P[C][C + 4];
    __shared__ float Gs[C];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int gq = lane / 16, li = lane % 16;
    const int n = blockIdx.x % N;
    const size_t bh = blockIdx.x / N;
    const int b = static_cast<int>(bh / H), h = static_cast<int>(bh % H);
    const int t0 = n * C;
    const int L = min(C, T - t0);
    const size_t chunk = bh * N + n;

    load_rows<DK, C>(Qs, q, b, h, t0, L, T, H);
    load_rows<DK, C>(Ks, k, b, h, t0, L, T, H);
    for (int e = tid; e < C * (C + 4); e += kBlock) (&P[0][0])[e] = 0.f;
    if (tid < C) Gs[tid] = ws.gw[chunk * G::GW + tid];
    __syncthreads();

    // P = Q K^T .* exp(G_r - G_j) on and below the diagonal
    constexpr int LT = G::CT * (G::CT + 1) / 2;
    for (int t = wave; t < LT; t += 4) {
        int mt = 0, rem = t;
        while (rem > mt) rem -= ++mt;
        const int nt = rem;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < G::KS; ++s)
            acc = mfma_bf16(lds_frag_bf16(&Qs[16 * mt + li][0], s, gq),
                            lds_frag_bf16(&Ks[16 * nt + li][0], s, gq), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * gq + r, col = 16 * nt + li;
            P[row][col] = (row >= col) ? acc[r] * __expf(Gs[row] - Gs[col]) : 0.f;
        }
    }
    __syncthreads();

    for (int slice = wave; slice < G::VT; slice += 4) {
        bf16x8 Sh[G::KS], Sl[G::KS];
#pragma unroll
        for (int s = 0; s < G::KS; ++s) {
            const f32x4 *sp = reinterpret_cast<const f32x4 *>(ws.sn + chunk * G::SN) +
                              (slice * G::KT) * kWave + lane;
            float x[8];
            acc_pair_to_slots(sp[(2 * s) * kWave], sp[(2 * s + 1) * kWave], x);
            split_bf16(x, Sh[s], Sl[s]);
        }
        bf16x8 Dh[G::CS], Dl[G::CS];
#pragma unroll
        for (int s = 0; s < G::CS; ++s) {
            const f32x4 *dp = reinterpret_cast<const f32x4 *>(ws.df + chunk * G::DF) +
                              (slice * G::CT) * kWave + lane;
            float x[8];
            acc_pair_to_slots(dp[(2 * s) * kWave], dp[(2 * s + 1) * kWave], x);
            split_bf16(x, Dh[s], Dl[s]);
        }
#pragma unroll
        for (int mt = 0; mt < G::CT; ++mt) {
            f32x4 qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < G::KS; ++s) {
                const bf16x8 a = lds_frag_bf16(&Qs[16 * mt + li][0], s, gq);
                qs = mfma_bf16(a, Sh[s], qs);
                qs = mfma_bf16(a, Sl[s], qs);
            }
            f32x4 pd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < G::CS; ++s) {
                float x[8];
                lds_slots_f32(&P[16 * mt + li][0], s, gq, x);
                bf16x8 ph, pl;
                split_bf16(x, ph, pl);
                pd = mfma_bf16(ph, Dh[s], pd);
                pd = mfma_bf16(ph, Dl[s], pd);
                pd = mfma_bf16(pl, Dh[s], pd);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * mt + 4 * gq + r;
                if (row < L)
                    o[((static_cast<size_t>(b) * T + t0 + row) * H + h) * DV + 16 * slice + li] =
                        scale * (__expf(Gs[row]) * qs[r] + pd[r]);
            }
        }
    }
}

template <int DK, int DV, int C>
hipError_t run_mfma(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                    const float *beta, const float *s0, float *o, float *s_out, int B, int T, int H,
                    void *ws, hipStream_t stream) {
    using G = Geo<DK, DV, C>;
    const int N = (T + C - 1) / C;
    const size_t chunks = static_cast<size_t>(B) * H * N;
    const Ws w = ws_carve<DK, DV, C>(ws, chunks);
    const float scale = 1.0f / sqrtf(static_cast<float>(DK));
    hipLaunchKernelGGL((prep_kernel<DK, DV, C>), dim3(static_cast<unsigned>(chunks)), dim3(kBlock), 0,
                       stream, k, v, g, beta, w, T, H, N);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((scan_kernel<DK, DV, C>), dim3(static_cast<unsigned>(B * H * G::VT)),
                       dim3(kWave), 0, stream, w, s0, s_out, N);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((output_kernel<DK, DV, C>), dim3(static_cast<unsigned>(chunks)), dim3(kBlock),
                       0, stream, q, k, w, o, T, H, N, scale);
    return hipGetLastError();
}

}  // namespace

bool prefill_bf16_uses_mfma(int dk, int dv, int chunk) {
    return (dk == 64 || dk == 128) && (dv == 64 || dv == 128) && (chunk == 32 || chunk == 64);
}

#define GDN_MFMA_CASES(X) \
    X(64, 64, 32) X(64, 64, 64) X(64, 128, 32) X(64, 128, 64) \
    X(128, 64, 32) X(128, 64, 64) X(128, 128, 32) X(128, 128, 64)

size_t prefill_bf16_workspace(int B, int T, int H, int dk, int dv, int chunk) {
    if (!prefill_bf16_uses_mfma(dk, dv, chunk)) return 0;
    const size_t chunks = static_cast<size_t>(B) * H * ((T + chunk - 1) / chunk);
#define GDN_WS(DK_, DV_, C_) \
    if (dk == DK_ && dv == DV_ && chunk == C_) return ws_bytes<DK_, DV_, C_>(chunks);
    GDN_MFMA_CASES(GDN_WS)
#undef GDN_WS
    return 0;
}

hipError_t launch_prefill_bf16(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                               const float *g, const float *beta, const float *s0, float *o,
                               float *s_out, int B, int T, int H, int dk, int dv, int chunk,
                               void *ws, hipStream_t stream) {
    if (!prefill_bf16_uses_mfma(dk, dv, chunk))
        return launch_prefill_valu(q, k, v, g, beta, s0, o, s_out, B, T, H, dk, dv, chunk, GDN_BF16,
                                   stream);
#define GDN_RUN(DK_, DV_, C_)                                                                      \
    if (dk == DK_ && dv == DV_ && chunk == C_)                                                     \
        return run_mfma<DK_, DV_, C_>(q, k, v, g, beta, s0, o, s_out, B, T, H, ws, stream);
    GDN_MFMA_CASES(GDN_RUN)
#undef GDN_RUN
    return hipErrorInvalidValue;
}

}  // namespace gdn
