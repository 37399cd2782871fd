// gdn_prefill_chunk.hip -- fused chunked GDN prefill for bf16 q/k/v (gfx950).
//
// Chunk form of the gated delta rule (derived from the rule; the pages give
// no chunked algorithm).  For a chunk of C tokens with start state
// St = S0^T (d_k x d_v, fp32) and G_r = sum_{i<=r} g_i within the chunk:
//   A     = strict_tril(diag(b) (K K^T .* exp(G_r - G_j)))
//   T     = (I + A)^{-1}
//   W     = T diag(b exp(G)) K,   U = T diag(b) V
//   Delta = U - W St                      (row r is b_r (v_r - a_r S_{r-1} k_r))
//   O     = scale (diag(exp(G)) Q St + (Q K^T .* exp(G_r - G_j) .* tril) Delta)
//   St'   = exp(G_C) St + K^T diag(exp(G_C - G)) Delta
//
// Sequence pieces.  A head's chunks are split into P consecutive pieces so
// that every compute unit has work even for few heads.  The state after a
// piece is an affine function of the state before it:
//   St_out = M_p St_in + N_p
// where N_p is the piece run from a zero state and M_p (d_k x d_k) is the
// same chunk recurrence run on the identity with no values.  Three launches:
//   MAP   (one workgroup per head and piece but the last) runs the recurrence
//         on [values | identity] columns and stores [N_p | M_p];
//   chain (one workgroup per head and 16 value columns) composes the maps
//         serially over pieces and stores every piece's true start state;
//   OUT   (one workgroup per head and piece) reruns each piece from its
//         start state and writes the outputs (and the final state).
// With a single piece only OUT runs, from the caller's start state.
//
// Inside a workgroup (4 wavefronts; 8 for 128 x 128 heads, the keyside still on
// four of them) all per-chunk operands live in LDS:
// K K^T and A, T by blocked substitution (16x16 diagonal blocks one column
// per lane, then 16x16 block products on MFMA with hi/lo bf16 splits), the
// W and K^T fragments of the scan, and P = Q K^T .* decay.  Each wavefront
// owns whole 16-column slices of the state: it keeps them in registers,
// computes U, Delta and the state update for them, and (OUT) their outputs,
// so the serial path never leaves the wavefront.
//
// Precision: K K^T and Q K^T are exact bf16 products with fp32 accumulation.
// Every other MFMA operand that is not an input is a hi + lo bf16 pair: T diag(b exp G)
// in W, W and the state in W St (Delta = U - W St cancels where a slowly decaying state
// already holds what the chunk writes), T diag(b) in U, the state in Q St, P and Delta
// in P Delta, the decayed Delta in the state update, and both factors of the
// inversion's block products.
#include <algorithm>
#include <type_traits>
#include <vector>

#include "gdn_mfma.h"

namespace gdn {

#define GDN_CHUNK_CASES(X) \
    X(64, 64, 32) X(64, 64, 64) X(64, 128, 32) X(64, 128, 64) \
    X(128, 64, 32) X(128, 64, 64) X(128, 128, 32) X(128, 128, 64)

namespace {

constexpr int kWave = 64;
// Wavefronts per workgroup.  The chunk's keyside (K K^T, T, W, P) is dealt over four
// wavefronts; the state's 16-column slices over all of them.  128 x 128 heads use eight,
// so each wavefront carries half the slices it would with four (two wavefronts per SIMD
// instead of one register-bound wavefront).
template <int DK, int DV>
constexpr int kWavesOf = (DK == 128 && DV == 128) ? 8 : 4;
constexpr int kKeyWaves = 4;  // wavefronts that build the keyside
// bf16 row padding in LDS.  Natural column order: row strides of 2 * odd dwords, so the
// 8-byte fragment reads of 16 consecutive rows (one per lane) cover all 32 banks once.
// Permuted order (below): strides of 4 * odd dwords, so the 16-byte fragment reads of 8
// consecutive rows cover the 32 banks once.
constexpr int kPad = 4;
constexpr int kPadPerm = 8;
constexpr int kXcds = 8;  // accelerator dies (each with its own L2) of an MI355X

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

struct FragPair {
    bf16x8 h, l;  // hi and lo bf16 parts of one MFMA operand fragment
};

template <int N>
using IC = std::integral_constant<int, N>;

constexpr float kLog2e = 1.4426950408889634f;
// MAP: the largest element of a piece map's identity slice that may be dropped (2^-32)
constexpr float kFlush = 0x1p-32f;
// 2^x by the hardware instruction (the decays here are 2^(non-positive) in log2 units)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// x from the lane whose index differs in bit 0 (resp. bit 1): DPP quad permutations
__device__ __forceinline__ float quad_xor1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}

// x + (x of the lane selected by a DPP control); lanes without a source, or outside the
// enabled rows, add zero
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}

// Inclusive prefix sum over the 64 lanes of a wavefront, all in DPP: shifts by 1, 2, 4, 8
// within each 16-lane row, then row 0's total broadcast into row 1 (and row 2's into row 3),
// then rows 0-1's total into rows 2 and 3.
__device__ __forceinline__ float wave_prefix_sum(float x) {
    x = dpp_add<0x111>(x);        // row_shr:1
    x = dpp_add<0x112>(x);        // row_shr:2
    x = dpp_add<0x114>(x);        // row_shr:4
    x = dpp_add<0x118>(x);        // row_shr:8
    x = dpp_add<0x142, 0xA>(x);   // row_bcast:15 into rows 1 and 3
    x = dpp_add<0x143, 0xC>(x);   // row_bcast:31 into rows 2 and 3
    return x;
}

__device__ __forceinline__ void split4(f32x4 x, s16x4 &hi, s16x4 &lo) {
    u32x2 h, l;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        h[i] = cvt2_bf16(x[2 * i], x[2 * i + 1]);
        l[i] = cvt2_bf16(x[2 * i] - lo_half_f32(h[i]), x[2 * i + 1] - hi_half_f32(h[i]));
    }
    hi = __builtin_bit_cast(s16x4, h);
    lo = __builtin_bit_cast(s16x4, l);
}

// acc + A B for 16x16 blocks to ~fp32 accuracy: a holds A[i][4 gq + e] of
// lane (gq, i); b holds B[4 gq + e][n] of lane (gq, n) (accumulator layout).
__device__ __forceinline__ f32x4 mm16(f32x4 a, f32x4 b, f32x4 acc) {
    s16x4 ah, al, bh, bl;
    split4(a, ah, al);
    split4(b, bh, bl);
    acc = mfma16(ah, bh, acc);
    acc = mfma16(ah, bl, acc);
    acc = mfma16(al, bh, acc);
    return acc;
}

template <int DK, int DV, int C, bool MAP>
struct Cfg {
    static constexpr int CT = C / 16, CS = C / 32, KT = DK / 16, KS = DK / 32, VT = DV / 16;
    static constexpr int NB = C / 16;
    static constexpr int WAVES = kWavesOf<DK, DV>, BLOCK = WAVES * kWave;
    static constexpr int NS = VT + (MAP ? KT : 0);  // 16-column slices of the carried state
    static constexpr int SPW = NS / WAVES;           // slices per wavefront
    static_assert(NS % WAVES == 0, "slices must divide among the wavefronts");
    static_assert(C == 32 || C == 64, "chunk");
    static constexpr int MAPW = DV + DK;  // row length of a stored piece map
};

// Packed variable-length sequences: a table built on the host and copied to the
// device.  Global piece gp (all sequences' pieces in order) belongs to sequence
// piece_seq[gp], global map gm (every piece but a sequence's last) to map_seq[gm];
// per sequence: first token, length, first global piece, first global map, state
// slot in the pool (-1: start from zeros, final state dropped) and whether to start
// from the slot's stored state.
struct SeqTable {
    const int *piece_seq, *map_seq;
    const int *tok0, *len, *pstart, *mstart, *slot, *init;
    // OUT: the global piece of each work-item slot (kXcds x out_per_xcd slots, -1 = none): the
    // pieces dealt to the XCDs in balanced bins, each bin longest first
    const int *out_order;
};

struct ChunkArgs {
    const uint16_t *q, *k, *v;
    const float *g, *beta;
    const float *s_start;  // OUT: start states, dense (bh * P + piece) or packed (gp * H + h) * DK * DV; NULL = zeros
    float *o;              // OUT: outputs
    float *s_final;        // OUT, dense: final states [BH][DK][DV], written by the last piece
    float *maps;           // MAP: dense [BH][P - 1] or packed [gm][H], each [DK][DV + DK]
    float *chunk_states;   // OUT, dense: start state of every chunk [BH][N][DK][DV], or NULL
    int T, H, BH, P, piece_chunks, N;
    float scale;
    SeqTable sq;           // packed sequences when sq.tok0 != NULL (then work items = pieces * H)
    float *pool;           // packed: state pool [slot][H][DK][DV] receiving final states
    int items;             // work items of this launch
    // PREP (the input preparation in the loads): q, k, v, g, beta above then point at the raw
    // projections and the raw gate / write-strength logits
    const float *conv_w;   // [H (2 DK + DV)][4]: q channels, then k, then v (head-major)
    const float *rate, *bias;  // [H] or NULL (1, 0)
    const float *conv_in;  // [B][H (2 DK + DV)][3]: the three raw inputs before t = 0, or NULL
    // 128 x 128 heads, gated delta rule, dense: the hi/lo A-fragments of T diag(b) of every chunk,
    // [BH][N][hi/lo x 2 row tiles][64 lanes], written by MAP (whose grid then also covers the
    // last piece, keyside only) and read by OUT in place of its own keyside; NULL: OUT forms them
    u16x8 *tfrag;
};

// Inputs of the preparation done in the chunk loads (PREP), beside the raw projections.
struct PrepIn {
    const float *conv_w, *rate, *bias, *conv_in;
};

// Eight bf16 to an 8-byte aligned LDS address (padded rows are not 16-byte aligned).
// Four-wavefront workgroups store the rows of K, Q, K^T and V^T with their columns permuted
// inside each 32-column block, so that the eight k-slots a lane feeds an MFMA lie next to
// each other: logical column 16 h + 4 g + e (h < 2, g < 4, e < 4) sits at 8 g + 4 h + e, and
// a fragment is one 16-byte read instead of two 8-byte ones (64K prefill 0.79 -> 0.78 ms;
// the eight-wavefront 128 x 128 kernel spills with it and keeps the natural order).
__device__ __forceinline__ int perm_col(int c) { return (c & ~31) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1) + (c & 3); }
__device__ __forceinline__ bf16x8 lds_frag_perm(const uint16_t *rowp, int s, int gq) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(rowp + 32 * s + 8 * gq));
}
// logical columns [8 c8, 8 c8 + 8) of a permuted row: two runs of four
__device__ __forceinline__ void lds_store8_perm(uint16_t *row, int c8, u16x8 x) {
    const int m = c8 & 3, off = 32 * (c8 >> 2) + 16 * (m & 1) + 4 * (m >> 1);
    reinterpret_cast<u16x4 *>(row + off)[0] = u16x4{x[0], x[1], x[2], x[3]};
    reinterpret_cast<u16x4 *>(row + off + 8)[0] = u16x4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void lds_store8(uint16_t *p, u16x8 x) {
    reinterpret_cast<u16x4 *>(p)[0] = u16x4{x[0], x[1], x[2], x[3]};
    reinterpret_cast<u16x4 *>(p)[1] = u16x4{x[4], x[5], x[6], x[7]};
}

// Per-thread share of one chunk's rows, loaded from HBM one chunk ahead.
template <int DK, int DV, int C, bool MAP>
struct ChunkRegs {
    // V is loaded (and transposed into LDS in F) by the first VTHREADS threads only: with
    // 64-wide values that is wavefronts 0 and 1, whose share of F is otherwise the smaller
    static constexpr int BLOCK = kWave * kWavesOf<DK, DV>;
    static constexpr int VTHREADS = DV == 64 ? BLOCK / 2 : BLOCK;
    static constexpr int NK = C * DK / 8 / BLOCK, NV = C * DV / 8 / VTHREADS;
    static_assert(C * DK % (8 * BLOCK) == 0 && C * DV % (8 * VTHREADS) == 0, "rows divide among threads");
    u16x8 k[NK], q[MAP ? 1 : NK], v[NV];
    // OUT, 128 x 128 heads: the chunk's T diag(b) fragments from MAP (wavefronts 0 and 1: hi, lo
    // of row tile tid / 64)
    static constexpr bool TB = !MAP && DK == 128 && C == 32;
    u16x8 tb[TB ? 2 : 1];
    float g, beta;
    u16x8 halo;  // PREP: one raw vector of the three rows before the chunk (halo threads only)
};

// PREP: the raw rows before a chunk (the convolution's window) are loaded by the first
// threads, one 8-channel vector each: three rows of K, of Q (not in MAP) and of V.
template <int DK, int DV, bool MAP>
struct Halo {
    static constexpr int NKH = 3 * DK / 8, NQH = MAP ? 0 : 3 * DK / 8, NVH = 3 * DV / 8;
    static constexpr int N = NKH + NQH + NVH;
};

// K and V are loaded one chunk row per lane (so their transposed copies can be
// written to LDS without bank conflicts); Q with consecutive lanes on one row.
// Buffer loads: each tensor's resource starts at the chunk's first row of this
// head and ends after its last valid row, so rows past the sequence end read as
// zeros (the hardware's range check) with no branch, and the lane offsets are 32-bit.
constexpr int kBufWord3 = 0x00020000;  // raw buffer, default data format (gfx9 family)

template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const T *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(base), 0, static_cast<int>(bytes), kBufWord3);
}
__device__ __forceinline__ u16x8 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
    return __builtin_bit_cast(u16x8, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_off), 0, 0));
}
__device__ __forceinline__ float buf_load4(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(byte_off), 0, 0));
}

// A value every lane holds alike, moved to scalar registers (lane 0's copy)
__device__ __forceinline__ size_t uniform_u64(size_t x) {
    const unsigned lo = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(x));
    const unsigned hi = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(x >> 32));
    return (static_cast<size_t>(hi) << 32) | lo;
}

template <int DK, int DV, int C, bool MAP, bool PREP>
__device__ __forceinline__ void load_chunk(ChunkRegs<DK, DV, C, MAP> &r, const ChunkArgs &a, size_t tok_base,
                                           int seq_len, int h, int n, int tid, const u16x8 *tb_src = nullptr) {
    using R = ChunkRegs<DK, DV, C, MAP>;
    // the lane offsets below are cheap to rebuild per chunk; hoisted out of the chunk loop
    // they would hold a dozen registers for its whole length
    __asm__ __volatile__("" : "+v"(tid));
    const int t0 = n * C;
    const int L = min(C, seq_len - t0);  // >= 1
    const size_t row0 = (tok_base + t0) * a.H + h;  // token-head row of t0
    const unsigned rows_k = static_cast<unsigned>((L - 1) * a.H * DK + DK) * 2u;
    const unsigned rows_v = static_cast<unsigned>((L - 1) * a.H * DV + DV) * 2u;
    const auto rk = chunk_rsrc(a.k + row0 * DK, rows_k);
    const auto rv = chunk_rsrc(a.v + row0 * DV, rows_v);
#pragma unroll
    for (int i = 0; i < R::NK; ++i) {
        const int e = tid + i * R::BLOCK;
        const int rr = e % C, c8 = e / C;
        r.k[i] = buf_load16(rk, static_cast<unsigned>(rr * a.H * DK + 8 * c8) * 2u);
        if (!MAP) {
            const auto rq = chunk_rsrc(a.q + row0 * DK, rows_k);
            const int qr = e / (DK / 8), qc = e % (DK / 8);
            r.q[i] = buf_load16(rq, static_cast<unsigned>(qr * a.H * DK + 8 * qc) * 2u);
        }
    }
    if (tid < R::VTHREADS) {
#pragma unroll
        for (int i = 0; i < R::NV; ++i) {
            const int e = tid + i * R::VTHREADS;
            const int rr = e % C, c8 = e / C;
            r.v[i] = buf_load16(rv, static_cast<unsigned>(rr * a.H * DV + 8 * c8) * 2u);
        }
    }
    if constexpr (R::TB) {
        if (tb_src != nullptr && tid < 2 * kWave) {
            const u16x8 *p = tb_src + static_cast<size_t>(n) * (4 * kWave) + 2 * (tid & ~(kWave - 1)) + tid % kWave;
            r.tb[0] = p[0];
            r.tb[1] = p[kWave];
        }
    }
    const unsigned rows_g = __builtin_amdgcn_readfirstlane(static_cast<unsigned>((L - 1) * a.H + 1) * 4u);
    const auto rg = chunk_rsrc(a.g + row0, rows_g);
    const auto rb = chunk_rsrc(a.beta + row0, rows_g);
    if (tid < kWave) {
        const unsigned off = static_cast<unsigned>(tid * a.H) * 4u;
        r.g = buf_load4(rg, off);
        r.beta = buf_load4(rb, off);
    }
    if constexpr (PREP) {
        using HL = Halo<DK, DV, MAP>;
        if (tid < HL::N) {
            // element: tensor (K, Q, V), halo row i (token t0 - 3 + i), 8-channel group c8
            const bool isk = tid < HL::NKH, isq = !isk && tid < HL::NKH + HL::NQH;
            const int e = isk ? tid : isq ? tid - HL::NKH : tid - HL::NKH - HL::NQH;
            const int W = (isk || isq) ? DK : DV;
            const int i = e / (W / 8), c8 = e % (W / 8);
            const uint16_t *x = isk ? a.k : isq ? a.q : a.v;
            if (t0 > 0) {  // chunks start at multiples of C >= 32: three earlier rows exist
                r.halo = *reinterpret_cast<const u16x8 *>(x + ((tok_base + t0 - 3 + i) * a.H + h) * W + 8 * c8);
            } else {
                // the carried window [b][channel][3] (oldest first), read through bf16 (it holds
                // raw inputs); zeros when absent
                const int chan = (isq ? 0 : isk ? a.H * DK : 2 * a.H * DK) + h * W + 8 * c8;
                const int nch = a.H * (2 * DK + DV);
                u16x8 hv;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    hv[j] = a.conv_in ? f32_to_bf16_bits(a.conv_in[(static_cast<size_t>(tok_base / a.T) * nch + chan + j) * 3 + i])
                                      : static_cast<uint16_t>(0);
                r.halo = hv;
            }
        }
    }
}

// Several workgroups per compute unit where registers and LDS allow it (64-wide heads), so
// one workgroup's dependent latencies and barrier waits are filled by the others' work: two
// with chunk 64 (73 KB of LDS each), three with chunk 32 (29 KB; at most 168 registers per
// lane, the occupancy bound of three wavefronts per SIMD).  64K prefill, 64-wide heads: chunk
// 32 with three workgroups per compute unit 0.72 ms, with two 0.81 ms; chunk 64 with two 0.81 ms.
template <int DK, int DV, int C>
constexpr int kBlocksPerCU = (DK == 64 && DV == 64) ? (C == 32 ? 3 : 2) : 1;
// workgroups the chip holds at once (256 compute units), the target of the piece plan
template <int DK, int DV, int C>
constexpr int kPlanSlots = 256 * kBlocksPerCU<DK, DV, C>;
int plan_slots(int dk, int dv, int chunk) { return 256 * ((dk == 64 && dv == 64) ? (chunk == 32 ? 3 : 2) : 1); }

// DELTA selects the rule: the gated delta rule (true) or the same recurrence without the
// erase term (false), S_t = a_t S_{t-1} + b_t v_t k_t^T, whose chunk form has A = 0 and T = I:
// Delta = diag(b) V with no W St term, and a piece map M_p that is a multiple of I.
// STATES (OUT only): write the state every chunk starts from (for the gradients) instead of the
// outputs, which the gradients do not use.
// Sum over aligned groups of N adjacent lanes (N = 8 or 16), left in every lane of the group.
template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
    x = dpp_add<0xB1>(x);                  // quad_perm [1,0,3,2]: lane ^ 1
    x = dpp_add<0x4E>(x);                  // quad_perm [2,3,0,1]: lane ^ 2
    x = dpp_add<0x141>(x);                 // row_half_mirror: the other quad of the eight
    if constexpr (N == 16) x = dpp_add<0x140>(x);  // row_mirror: the other eight of the row
    static_assert(N == 8 || N == 16, "group");
    return x;
}

// SiLU as the preparation kernel evaluates it: c / (1 + e^-c)
__device__ __forceinline__ float silu_f(float c) {
    return c * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-c * kLog2e));
}

// PREP: the input preparation ahead of the mixer done in the chunk loads (the rows loaded are
// the raw projections and logits): causal depthwise convolution of width 4, SiLU, the L2 norm
// of each head's q and k rows (eps 1e-6 under the root), g = -A_h softplus(a + bias_h) and
// beta = sigmoid(b); the prepared q, k, v are rounded once to bf16 (as the preparation kernel
// stores them) and go on exactly like loaded rows.
template <int DK, int DV, int C, bool MAP, bool DELTA, bool STATES = false, bool PREP = false>
__global__ __launch_bounds__((kWave * kWavesOf<DK, DV>), (kBlocksPerCU<DK, DV, C>)) void chunk_kernel(ChunkArgs a) {
    using G = Cfg<DK, DV, C, MAP>;
    using R = ChunkRegs<DK, DV, C, MAP>;
    constexpr bool kPerm = G::WAVES == 4;  // permuted bf16 rows (see perm_col)
    constexpr int kRowPad = kPerm ? kPadPerm : kPad;
    constexpr int KSTR = DK + kRowPad;   // K and Q rows
    constexpr int VSTR = C + kRowPad;    // V^T rows
    constexpr int CSTR = C + 4;       // A and T rows (fp32)
    // Chunk 32 with the erase term: no W.  Delta = U - W St = T diag(b) (V - diag(exp G) K St),
    // formed per slice in G from K's rows, V^T and T, so there is no phase F; V^T and the P
    // fragments get buffers of their own (K's rows stay live through G).
    constexpr bool kNoW = DELTA && C == 32;
    constexpr int KV_ELEMS = (kNoW || C * KSTR > DV * VSTR) ? C * KSTR : DV * VSTR;
    constexpr int KTSTR = C + kRowPad;   // K^T rows
    constexpr int CSTR16 = 20;        // rows of the 16x16 scratch tile (conflict-free f32x4 reads)
    static_assert(2 * G::CT * G::CS * kWave * 16 <= C * CSTR * 4, "P fragments fit in A's buffer");
    // With one 16-row tile of T per wavefront (chunk 64), F builds the hi/lo fragments of
    // T diag(b) once and parks them over that wavefront's own (then dead) T rows.
    constexpr bool kTbFrags = G::CT == kKeyWaves;
    static_assert(!kTbFrags || 2 * G::CS * kWave * 16 <= 16 * CSTR * 4, "T diag(b) fragments fit in 16 T rows");
    __shared__ __align__(16) uint16_t kv_s[KV_ELEMS];              // K rows (then V^T, with W)
    __shared__ __align__(16) uint16_t vt_s[kNoW ? DV * VSTR : 8];  // V^T (no W)
    __shared__ __align__(16) bf16x8 pf2_s[kNoW ? 2 * G::CT * G::CS * kWave : 1];  // P fragments (no W)
    __shared__ __align__(16) uint16_t q_s[MAP ? 8 : C * KSTR];     // Q rows
    __shared__ __align__(16) float a_s[C * CSTR];                  // A, then P fragments
    // T = (I + A)^{-1}; without the erase term (no T) the same buffer holds V^T
    constexpr int TS_FLOATS = (DELTA || C * CSTR * 2 >= DV * VSTR) ? C * CSTR : (DV * VSTR + 1) / 2;
    __shared__ __align__(16) float t_s[TS_FLOATS];
    // W A-fragments as hi + lo bf16 pairs: Delta = U - W St cancels where a slowly decaying state
    // already holds what the chunk writes, so W St needs both factors split
    __shared__ __align__(16) bf16x8 wf_s[(DELTA && !kNoW) ? G::CT * G::KS * kWave : 1];   // W, hi parts
    __shared__ __align__(16) bf16x8 wfl_s[(DELTA && !kNoW) ? G::CT * G::KS * kWave : 1];  // W, lo parts
    __shared__ __align__(16) uint16_t kt_s[DK * KTSTR];            // K^T
    __shared__ __align__(16) float x_s[DELTA ? 16 * CSTR16 : 4];   // one 16x16 fp32 tile (C)
    // Eight wavefronts: two per T row tile build W in F (each half of its tiles), so the
    // T diag(b) fragments get a buffer of their own instead of the T rows both still read.
    constexpr bool kSplitF = kTbFrags && DELTA && G::WAVES == 2 * G::CT;
    // Eight wavefronts, chunk 64: B's tiles below the diagonal and every P tile go to
    // wavefronts 4-7, so 0-3 compute only their diagonal tile and its inverse in B, and the
    // blocks of T in C.
    constexpr bool kSplitKey = kSplitF;
    // Chunk 32: the whole keyside in B, no phase C.  Wavefront 0 forms A's first diagonal tile and
    // inverts it; wavefront 1 the second tile and its inverse, then A10, and after wavefront 0 has
    // published T00 (an LDS flag holding the chunk index), T10 = -T11 A10 T00.  (With eight
    // wavefronts, 128 x 128 heads, wavefronts 4-7 wait in B: 3B-shaped 64K call 1.59 -> 1.56 ms
    // against the A tiles on three wavefronts and T10 after a barrier of its own.)
    constexpr bool kMergeBC = DELTA && C == 32 && (G::WAVES == 4 || G::WAVES == 8);
    __shared__ __align__(16) bf16x8 tbf_s[kSplitF ? G::CT * G::CS * 2 * kWave : 1];
    __shared__ float g_s[C], b_s[C], bg_s[C], dec_s[C], gam_s[C];  // g_s: G * log2(e)
    __shared__ int t00_ready;  // the last chunk whose T00 wavefront 0 has stored (kMergeBC)
    __shared__ int a10_ready;  // the last chunk whose A10 wavefront 2 has stored (kMergeBC)
    // MAP, gated delta rule (the identity slices dropped below kFlush, in G): grow_s, some chunk of
    // the piece so far can expand the map (a log gate above 0, or b |k|^2 > 2); flush_s[n & 1], a
    // wavefront dropped a slice at the end of chunk n (read in chunk n + 1)
    __shared__ int grow_s, flush_s[2];
    // The hi/lo A-fragments of T diag(b) for G, built once per chunk by wavefronts 0 and 1 at the end
    // of B instead of by every slice wavefront (not in the preparation kernels, whose registers are
    // at the occupancy limit already)
    constexpr bool kShareTB = kMergeBC && !PREP;
    __shared__ __align__(16) bf16x8 tbs_s[kShareTB ? 2 * G::CT * kWave : 1];  // (ct * 2 + hi/lo) * 64 + lane
    // 128 x 128 heads (one workgroup per compute unit, so no other workgroup's work hides OUT's
    // keyside): MAP stores those fragments and OUT loads them (3B-shaped 64K call 1.56 -> 1.48 ms).
    // With three workgroups per compute unit the 64 x 64 kernels gain nothing from it (MAP +17 us
    // for the stores, OUT -20 us).
    constexpr bool kTfrag = kShareTB && DK == 128 && C == 32;
    static_assert(!kTfrag || G::CT == 2, "two row tiles of T");
    // PREP: raw rows of the chunk after the three rows before it (row 3 + r holds chunk row r),
    // the per-row partial squares of k, and this head's convolution weights (q, k, v channels)
    constexpr int RKS = DK + 8, RVS = DV + 8;  // raw row strides (16-byte multiples)
    __shared__ __align__(16) uint16_t kraw_s[PREP ? (C + 3) * RKS : 8];
    __shared__ __align__(16) uint16_t qraw_s[(PREP && !MAP) ? (C + 3) * RKS : 8];
    __shared__ __align__(16) uint16_t vraw_s[PREP ? (C + 3) * RVS : 8];
    __shared__ __align__(16) float ksq_s[PREP ? C * (DK / 8) : 4];
    __shared__ __align__(16) float wconv_s[PREP ? (2 * DK + DV) * 4 : 4];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform
    const int tid = threadIdx.x, lane = tid % kWave;
    const int gq = lane / 16, li = lane % 16;
    // Work item w = piece * BH + bh.  Workgroups go to the eight XCDs round-robin by index,
    // so consecutive work items (one piece, consecutive heads: they share every g and beta
    // cache line) are given to indices that land on the same XCD and its L2.  The grid is a
    // multiple of 8; surplus workgroups leave at once.
    const int per_xcd = gridDim.x / kXcds;
    const int w = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (w >= a.items) return;
    // this work item: one head of one piece of one sequence
    int h, n0, n1, seq_len;
    size_t tok_base;                  // first token of the sequence in the [tokens, H, d] layout
    const float *start = nullptr;     // OUT: start state [DK][DV] (NULL = zeros)
    float *map_out = nullptr;         // MAP: piece map [DK][DV + DK]
    float *final_out = nullptr;       // OUT: final state [DK][DV] of the sequence's last piece
    float *states_out = nullptr;      // OUT, dense: this head's chunk start states [N][DK][DV]
    u16x8 *tb_ptr = nullptr;          // kTfrag: this head's T diag(b) fragments, chunk n at n * 4 * 64
    bool key_only = false;            // MAP over the last piece (kTfrag): the fragments, no map
    if (a.sq.tok0 == nullptr) {
        const int piece = w / a.BH;
        const size_t bh = w % a.BH;
        const int b = static_cast<int>(bh / a.H);
        h = static_cast<int>(bh % a.H);
        tok_base = static_cast<size_t>(b) * a.T;
        seq_len = a.T;
        n0 = piece * a.piece_chunks;
        n1 = min(n0 + a.piece_chunks, a.N);
        if constexpr (kTfrag) {
            if (a.tfrag) tb_ptr = a.tfrag + bh * a.N * (4 * kWave);
        }
        key_only = MAP && piece >= a.P - 1;
        if (MAP && !key_only) map_out = a.maps + (bh * (a.P - 1) + piece) * DK * G::MAPW;
        else if (a.s_start) start = a.s_start + (bh * a.P + piece) * DK * DV;
        if (!MAP && piece == a.P - 1) final_out = a.s_final + bh * DK * DV;
        if (!MAP && STATES) states_out = a.chunk_states + bh * a.N * DK * DV;
    } else {
        const int gp = MAP ? w / a.H : a.sq.out_order[w / a.H];  // global map (MAP) or piece (OUT)
        if (gp < 0) return;  // an empty slot of the dealing (uniform over the workgroup)
        h = w % a.H;
        const int s = MAP ? a.sq.map_seq[gp] : a.sq.piece_seq[gp];
        const int piece = gp - (MAP ? a.sq.mstart[s] : a.sq.pstart[s]);
        tok_base = static_cast<size_t>(a.sq.tok0[s]);
        seq_len = a.sq.len[s];
        const int nchunks = (seq_len + C - 1) / C;
        n0 = piece * a.piece_chunks;
        n1 = min(n0 + a.piece_chunks, nchunks);
        if (MAP) {
            map_out = a.maps + (static_cast<size_t>(gp) * a.H + h) * DK * G::MAPW;
        } else {
            start = a.s_start + (static_cast<size_t>(gp) * a.H + h) * DK * DV;
            const int slot = a.sq.slot[s];
            if (n1 == nchunks && slot >= 0) final_out = a.pool + (static_cast<size_t>(slot) * a.H + h) * DK * DV;
        }
    }

    // The work item's indices are the same on every lane, but on the packed-sequence
    // path they come from a table load the compiler cannot prove uniform: without this each
    // chunk's buffer loads would run as a loop over distinct descriptors.
    h = __builtin_amdgcn_readfirstlane(h);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    n1 = __builtin_amdgcn_readfirstlane(n1);
    seq_len = __builtin_amdgcn_readfirstlane(seq_len);
    tok_base = uniform_u64(tok_base);

    // ---- carried state: St[j][mt] holds rows 16 mt + 4 gq + r, column 16 sl + li, sl = wave + 4 j
    f32x4 St[G::SPW][G::KT];
    auto init_state = [&]() {
#pragma unroll
        for (int j = 0; j < G::SPW; ++j) {
            const int sl = wave + G::WAVES * j;
#pragma unroll
            for (int mt = 0; mt < G::KT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * mt + 4 * gq + r;
                    float x = 0.f;
                    if (MAP) {
                        if (sl >= G::VT) x = (row == 16 * (sl - G::VT) + li) ? 1.f : 0.f;
                    } else if (start) {
                        x = start[row * DV + 16 * sl + li];
                    }
                    St[j][mt][r] = x;
                }
        }
    };
    init_state();
    // T's blocks above the diagonal stay zero for the whole kernel
    for (int e = tid; e < TS_FLOATS; e += G::BLOCK) t_s[e] = 0.f;
    if (tid == 0) {
        t00_ready = a10_ready = -1;
        grow_s = flush_s[0] = flush_s[1] = 0;
    }
    float rate_h = 1.f, bias_h = 0.f;
    if constexpr (PREP) {
        for (int c = tid; c < 2 * DK + DV; c += G::BLOCK) {
            const int chan = c < DK ? h * DK + c : c < 2 * DK ? a.H * DK + h * DK + (c - DK)
                                                             : 2 * a.H * DK + h * DV + (c - 2 * DK);
            *reinterpret_cast<f32x4 *>(&wconv_s[4 * c]) = *reinterpret_cast<const f32x4 *>(a.conv_w + 4 * static_cast<size_t>(chan));
        }
        if (a.rate) rate_h = a.rate[h];
        if (a.bias) bias_h = a.bias[h];
    }

    uint16_t(*ks)[KSTR] = reinterpret_cast<uint16_t(*)[KSTR]>(kv_s);
    uint16_t(*vt)[VSTR] = reinterpret_cast<uint16_t(*)[VSTR]>(kNoW ? static_cast<void *>(vt_s)
                                                              : DELTA ? static_cast<void *>(kv_s)
                                                                      : static_cast<void *>(t_s));
    uint16_t(*qs)[KSTR] = reinterpret_cast<uint16_t(*)[KSTR]>(q_s);
    uint16_t(*kt)[KTSTR] = reinterpret_cast<uint16_t(*)[KTSTR]>(kt_s);
    // K^T A-fragment (d tile mt, chunk-row step s): K^T[16 mt + li][kmap(s, gq, e)]
    // fragment reads, row stores and column positions in the chosen column order
    auto frag = [&](const uint16_t *rowp, int s) {
        if constexpr (kPerm) return lds_frag_perm(rowp, s, gq);
        else return lds_frag_bf16(rowp, s, gq);
    };
    auto store8 = [&](uint16_t *row, int c8, u16x8 x) {
        if constexpr (kPerm) lds_store8_perm(row, c8, x);
        else lds_store8(row + 8 * c8, x);
    };
    auto col_of = [&](int c) { return kPerm ? perm_col(c) : c; };
    auto kfrag = [&](int mt, int s) { return frag(&kt[16 * mt + li][0], s); };
    float(*as)[CSTR] = reinterpret_cast<float(*)[CSTR]>(a_s);
    float(*ts)[CSTR] = reinterpret_cast<float(*)[CSTR]>(t_s);
    // P fragments: ((mt * CS + s) * 2 + hi/lo) * 64 + lane
    bf16x8 *pf_s = kNoW ? pf2_s : reinterpret_cast<bf16x8 *>(a_s);

    float(*xs)[CSTR16] = reinterpret_cast<float(*)[CSTR16]>(x_s);
    // 16x16 fp32 blocks of a row-major LDS matrix as MFMA operands
    auto rowfrag = [&](auto m, int r0, int c0) {
        return *reinterpret_cast<const f32x4 *>(&m[r0 + li][c0 + 4 * gq]);
    };
    auto accfrag = [&](auto m, int r0, int c0) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = m[r0 + 4 * gq + e][c0 + li];
        return x;
    };
    auto store_acc = [&](auto m, int r0, int c0, f32x4 x) {
#pragma unroll
        for (int e = 0; e < 4; ++e) m[r0 + 4 * gq + e][c0 + li] = x[e];
    };
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    R cur;
    if (n0 < n1) load_chunk<DK, DV, C, MAP, PREP>(cur, a, tok_base, seq_len, h, n0, tid, tb_ptr);
    // MAP, gated delta rule: identity slice j of this wavefront is zero and skipped for the rest of
    // the piece.  Its columns of the piece map carry no values, so a zero slice stays zero
    // (R = -diag(exp G) K 0 = 0, Delta = 0, St' = 0).  A slice is zero once the decays have taken it
    // below fp32's range, or is set to zero once every element is at most kFlush while every token
    // of the piece so far has a map of norm at most 1 (log gate <= 0 and b |k|^2 <= 2: then each
    // later token can only shrink what was dropped).  Dropping at most kFlush per element over the
    // d_k identity columns changes the map by at most d_k kFlush = 2^-25 in norm (d_k <= 128), under
    // half a unit in the last place of fp32: the piece's end state M_p S_p + N_p moves by less than
    // its own rounding relative to |S_p|.  A chunk that can expand the map turns the drops off for
    // the rest of the piece, and if a slice was already dropped, the piece's map is recomputed
    // from its first chunk without drops.  Gains: 64K workload 0.745 -> 0.705 ms (exact zeros
    // alone: 0.727), literal-gate reading 0.73 -> 0.67 ms, 3B-shaped call 1.49 -> 1.31 ms.
    // (not with the preparation in the loads, whose kernels are at their register limit: there a
    // slice is skipped only once it is exactly zero)
    constexpr bool kDrop = MAP && DELTA && !PREP;
    bool id_zero[G::SPW] = {};
    bool flush_ok = kDrop, any_flush = false;

    for (int n = n0; n < n1; ++n) {
        const int t0 = n * C;
        const int L = min(C, seq_len - t0);
        if (!MAP && STATES) {  // the state this chunk starts from, kept for the gradients
            float *cs = states_out + static_cast<size_t>(n) * DK * DV;
#pragma unroll
            for (int j = 0; j < G::SPW; ++j)
#pragma unroll
                for (int mt = 0; mt < G::KT; ++mt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        cs[(16 * mt + 4 * gq + r) * DV + 16 * (wave + G::WAVES * j) + li] = St[j][mt][r];
        }

        if constexpr (PREP) {
            // ---- the input preparation: raw rows (and the window before the chunk) to LDS
            using HL = Halo<DK, DV, MAP>;
#pragma unroll
            for (int i = 0; i < R::NK; ++i) {
                const int e = tid + i * G::BLOCK;
                *reinterpret_cast<u16x8 *>(&kraw_s[(3 + e % C) * RKS + 8 * (e / C)]) = cur.k[i];
                if constexpr (!MAP)
                    *reinterpret_cast<u16x8 *>(&qraw_s[(3 + e / (DK / 8)) * RKS + 8 * (e % (DK / 8))]) = cur.q[i];
            }
            if (tid < R::VTHREADS) {
#pragma unroll
                for (int i = 0; i < R::NV; ++i) {
                    const int e = tid + i * R::VTHREADS;
                    *reinterpret_cast<u16x8 *>(&vraw_s[(3 + e % C) * RVS + 8 * (e / C)]) = cur.v[i];
                }
            }
            if (tid < HL::N) {
                const bool isk = tid < HL::NKH, isq = !isk && tid < HL::NKH + HL::NQH;
                const int e = isk ? tid : isq ? tid - HL::NKH : tid - HL::NKH - HL::NQH;
                const int W = (isk || isq) ? DK : DV;
                uint16_t *dst = isk ? kraw_s : isq ? qraw_s : vraw_s;
                *reinterpret_cast<u16x8 *>(&dst[(e / (W / 8)) * (W + 8) + 8 * (e % (W / 8))]) = cur.halo;
            }
            if (wave == 0) {
                // gates from the raw logits; rows past the sequence end stay inert (g = beta = 0)
                const float z = cur.g + bias_h;
                const float sp = fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
                cur.g = lane < L ? -rate_h * sp : 0.f;
                cur.beta = lane < L ? 1.f / (1.f + expf(-cur.beta)) : 0.f;
            }
            __syncthreads();
            // convolution over the four rows ending at the lane's row, then SiLU; rows past the
            // sequence end give zeros
            auto conv8 = [&](const uint16_t *raw, int stride, int r, int c0, const float *w, float (&y)[8]) {
                u16x8 x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) x[j] = *reinterpret_cast<const u16x8 *>(&raw[(r + j) * stride + c0]);
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const f32x4 wc = *reinterpret_cast<const f32x4 *>(&w[4 * (c0 + c)]);
                    const float cv = fmaf(wc[3], from_bf16(x[3][c]), fmaf(wc[2], from_bf16(x[2][c]),
                                     fmaf(wc[1], from_bf16(x[1][c]), wc[0] * from_bf16(x[0][c]))));
                    y[c] = r < L ? silu_f(cv) : 0.f;
                }
            };
            // q first (finished here: its row's eight or sixteen lanes sum the squares), then k,
            // whose sums cross wavefronts and wait for the next barrier
            if constexpr (!MAP) {
#pragma unroll
                for (int i = 0; i < R::NK; ++i) {
                    const int e = tid + i * G::BLOCK, rq = e / (DK / 8), cq = e % (DK / 8);
                    float qy[8];
                    conv8(qraw_s, RKS, rq, 8 * cq, wconv_s, qy);
                    float qs2 = 0.f;
#pragma unroll
                    for (int c = 0; c < 8; ++c) qs2 = fmaf(qy[c], qy[c], qs2);
                    const float rn = __builtin_amdgcn_rsqf(lane_group_sum<DK / 8>(qs2) + 1e-6f);
#pragma unroll
                    for (int c = 0; c < 8; ++c) qy[c] *= rn;
                    cur.q[i] = __builtin_bit_cast(u16x8, pack_bf16(qy));
                }
            }
            float ky[R::NK][8];
#pragma unroll
            for (int i = 0; i < R::NK; ++i) {
                const int e = tid + i * G::BLOCK, rr = e % C, c8 = e / C;
                conv8(kraw_s, RKS, rr, 8 * c8, wconv_s + 4 * DK, ky[i]);
                float ss = 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) ss = fmaf(ky[i][c], ky[i][c], ss);
                ksq_s[rr * (DK / 8) + c8] = ss;
            }
            if (tid < R::VTHREADS) {
#pragma unroll
                for (int i = 0; i < R::NV; ++i) {
                    const int e = tid + i * R::VTHREADS;
                    float vy[8];
                    conv8(vraw_s, RVS, e % C, 8 * (e / C), wconv_s + 8 * DK, vy);
                    cur.v[i] = __builtin_bit_cast(u16x8, pack_bf16(vy));
                }
            }
            __syncthreads();
            // k's norm from the partial squares of its row
#pragma unroll
            for (int i = 0; i < R::NK; ++i) {
                const int e = tid + i * G::BLOCK, rr = e % C;
                float ss = 0.f;
#pragma unroll
                for (int c8 = 0; c8 < DK / 8; ++c8) ss += ksq_s[rr * (DK / 8) + c8];
                const float rn = __builtin_amdgcn_rsqf(ss + 1e-6f);
#pragma unroll
                for (int c = 0; c < 8; ++c) ky[i][c] *= rn;
                cur.k[i] = __builtin_bit_cast(u16x8, pack_bf16(ky[i]));
            }
        }

        // ---- A: this chunk's rows into LDS (K both row-major and transposed); gates
#pragma unroll
        for (int i = 0; i < R::NK; ++i) {
            const int e = tid + i * G::BLOCK;
            const int rr = e % C, c8 = e / C;
            store8(&ks[rr][0], c8, cur.k[i]);
            const int rc = col_of(rr);
#pragma unroll
            for (int q8 = 0; q8 < 8; ++q8) kt[8 * c8 + q8][rc] = cur.k[i][q8];
            if (!MAP) {
                const int rq = e / (DK / 8), cq = e % (DK / 8);
                store8(&qs[rq][0], cq, cur.q[i]);
            }
        }
        if (wave == 0) {
            // inclusive prefix sum of the gates; rows >= L add 0 and repeat G_{L-1}
            // G in log2 units: every decay below is then one v_exp_f32 (2^x)
            const float x = wave_prefix_sum(cur.g) * kLog2e;
            const float glast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), C - 1));
            if (lane < C) {
                if (MAP && DELTA && !(cur.g <= 0.f)) grow_s = 1;
                const float ex = exp2_fast(x);
                g_s[lane] = x;
                b_s[lane] = cur.beta;
                gam_s[lane] = ex;
                bg_s[lane] = cur.beta * ex;
                dec_s[lane] = exp2_fast(glast - x);
            }
        }
        if constexpr (!DELTA || kNoW) {
            // V^T goes to its own buffer at once (no phase F to stage it in)
            if (tid < R::VTHREADS) {
#pragma unroll
                for (int i = 0; i < R::NV; ++i) {
                    const int e = tid + i * R::VTHREADS, rr = e % C, c8 = e / C;
#pragma unroll
                    for (int q8 = 0; q8 < 8; ++q8) vt[8 * c8 + q8][col_of(rr)] = cur.v[i][q8];
                }
            }
        }
        __syncthreads();

        // Wave priorities (two workgroups per compute unit): the phases on the chunk's critical
        // path issue first when both workgroups have a wave ready -- B and C (the inversion) at 1,
        // G (the state chain) at 2, A and F (loads, staging, fragment building) at 0.  On the 64K
        // call: 0.84 ms with none, 0.82 with G alone raised, 0.79-0.80 with this order.
        if constexpr (G::WAVES == 4) __builtin_amdgcn_s_setprio(1);
        // ---- B: A = strict_tril(diag(b) (K K^T .* exp(G_r - G_j))) tile by tile, then each
        // wavefront inverts the diagonal block of (I + A) whose A tile it computed itself, so no
        // barrier separates the two.  Tiles (C = 64): w0 (0,0) (1,0) (2,0); w1 (1,1) (2,1) (3,0);
        // w2 (2,2); w3 (3,3) (3,2); (3,1) on w0 (OUT) or w2 (MAP); w2 and w3 also form the
        // two single-product P tiles (OUT).
        auto a_tile = [&](auto mt_c, auto nt_c) {
            constexpr int mt = decltype(mt_c)::value, nt = decltype(nt_c)::value;
            f32x4 acc = zero4;
#pragma unroll
            for (int s = 0; s < G::KS; ++s)
                acc = mfma_bf16(frag(&ks[16 * mt + li][0], s), frag(&ks[16 * nt + li][0], s),
                                acc);
            const f32x4 grow = *reinterpret_cast<const f32x4 *>(&g_s[16 * mt + 4 * gq]);
            const f32x4 brow = *reinterpret_cast<const f32x4 *>(&b_s[16 * mt + 4 * gq]);
            const int col = 16 * nt + li;
            const float gcol = g_s[col];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * mt + 4 * gq + r;
                if constexpr (mt > nt) {
                    as[row][col] = brow[r] * acc[r] * exp2_fast(grow[r] - gcol);
                } else {
                    // diagonal tile: exp of a clamped exponent times a 0/1 mask (no branch)
                    const float ex = exp2_fast(fminf(grow[r] - gcol, 0.f));
                    as[row][col] = ((row > col) ? 1.f : 0.f) * (brow[r] * acc[r] * ex);
                    // the diagonal holds |k_row|^2: the token's map (I - b k k^T) has norm above 1
                    if (MAP && row == col && !(brow[r] * acc[r] <= 2.f)) grow_s = 1;
                }
            }
        };
        // Diagonal block w of T = (I + A)^{-1} by forward substitution down each column j,
        // t_r = delta_rj - sum_{m<r} A[r][m] t_m, four rows at a time.  Lane (j, q) = (lane / 4,
        // lane % 4) keeps t_m for m in [4q, 4q + 4).  For the rows of group g (4g .. 4g + 3) the
        // sums over the earlier groups are independent of each other: each lane adds its four
        // terms and two quad-lane adds complete them, four rows side by side.  The 4 x 4
        // triangle inside the group is then solved on the lane that holds those columns of A
        // (q = g), which also keeps the results.  Per group the chain is one reduction and
        // three dependent fused multiply-adds, instead of one reduction per row.  A is strictly
        // lower and t_m is zero until its group is reached, so nothing needs masking.  Reads
        // only this wavefront's own A tile (LDS keeps a wavefront's accesses in order).
        auto inv_diag = [&](int bb) {
            const int j = lane >> 2, q = lane & 3;
            float tq[4] = {0.f, 0.f, 0.f, 0.f};  // t_m for m = 4q + i
            // this lane's four columns of a group's rows; the next group's are loaded while this one
            // is solved
            f32x4 arow[4], nrow[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) nrow[a] = *reinterpret_cast<const f32x4 *>(&as[bb + a][bb + 4 * q]);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
#pragma unroll
                for (int a = 0; a < 4; ++a) arow[a] = nrow[a];
                if (g + 1 < 4) {
#pragma unroll
                    for (int a = 0; a < 4; ++a)
                        nrow[a] = *reinterpret_cast<const f32x4 *>(&as[bb + 4 * (g + 1) + a][bb + 4 * q]);
                }
                float p[4] = {0.f, 0.f, 0.f, 0.f};
                if (g > 0) {
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        float x = arow[a][0] * tq[0];
#pragma unroll
                        for (int i = 1; i < 4; ++i) x = fmaf(arow[a][i], tq[i], x);
                        p[a] = x;
                    }
#pragma unroll
                    for (int a = 0; a < 4; ++a) p[a] += quad_xor1(p[a]);
#pragma unroll
                    for (int a = 0; a < 4; ++a) p[a] += quad_xor2(p[a]);
                }
                float t[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int r = 4 * g + a;
                    float v = ((r == j) ? 1.f : 0.f) - p[a];
#pragma unroll
                    for (int b = 0; b < a; ++b) v = fmaf(-arow[a][b], t[b], v);
                    t[a] = v;
                }
#pragma unroll
                for (int a = 0; a < 4; ++a) tq[a] = (q == g) ? t[a] : tq[a];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) ts[bb + 4 * q + i][bb + j] = tq[i];
        };
        // P tiles (mt, s): formed into registers (P^T accumulator tiles are P's A-fragment
        // layout, split hi + lo), stored in F once A's buffer is free.  Per wavefront (chunk 64):
        // B: w2 (0,0), w3 (2,1) (single products); C: w0 (3,0), w1 (1,0) (2,0), w2 (3,1).
        auto p_pair = [&](auto mt_c, auto s_c) {
            constexpr int mt = decltype(mt_c)::value, s = decltype(s_c)::value;
            f32x4 acc[2] = {zero4, zero4};
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int jt = 2 * s + half;
                if (jt > mt) continue;
#pragma unroll
                for (int ss = 0; ss < G::KS; ++ss)
                    acc[half] = mfma_bf16(frag(&ks[16 * jt + li][0], ss), frag(&qs[16 * mt + li][0], ss),
                                          acc[half]);
            }
            // lane holds P[r][j] for r = 16 mt + li and j = kmap(s, gq, e)
            const int r = 16 * mt + li;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int jj = kmap(s, gq, e);
                const float qk = acc[e >> 2][e & 3];
                const float ex = exp2_fast(fminf(g_s[r] - g_s[jj], 0.f));
                x[e] = ((jj <= r) ? 1.f : 0.f) * (qk * ex);
            }
            FragPair f;
            split_bf16(x, f.h, f.l);
            return f;
        };
        auto p_store = [&](auto mt_c, auto s_c, FragPair f) {
            constexpr int mt = decltype(mt_c)::value, s = decltype(s_c)::value;
            pf_s[((mt * G::CS + s) * 2 + 0) * kWave + lane] = f.h;
            pf_s[((mt * G::CS + s) * 2 + 1) * kWave + lane] = f.l;
        };
        FragPair pa{}, pb{};
        if constexpr (DELTA) {
            using I0 = IC<0>;
            using I1 = IC<1>;
            if constexpr (kSplitKey) {
                // eight wavefronts: 0-3 their diagonal tile, then its inverse; 4-6 the tiles below
                // the diagonal; 7 the two single-product P tiles
                if (wave == 0) a_tile(I0{}, I0{});
                else if (wave == 1) a_tile(I1{}, I1{});
                else if (wave == 2) a_tile(IC<2>{}, IC<2>{});
                else if (wave == 3) a_tile(IC<3>{}, IC<3>{});
                else if (wave == 4) {
                    a_tile(I1{}, I0{});
                    a_tile(IC<2>{}, I0{});
                } else if (wave == 5) {
                    a_tile(IC<2>{}, I1{});
                    a_tile(IC<3>{}, I0{});
                } else if (wave == 6) {
                    a_tile(IC<3>{}, I1{});
                    a_tile(IC<3>{}, IC<2>{});
                } else if (wave == 7) {
                    if constexpr (!MAP) {
                        pa = p_pair(I0{}, I0{});
                        pb = p_pair(IC<2>{}, I1{});
                    }
                }
            } else if constexpr (G::CT == 4) {
                // (3,1) goes to wavefront 0 where wavefront 2 also forms a P tile
                if (wave == 0) {
                    a_tile(I0{}, I0{});
                    a_tile(I1{}, I0{});
                    a_tile(IC<2>{}, I0{});
                    if constexpr (!MAP) a_tile(IC<3>{}, I1{});
                } else if (wave == 1) {
                    a_tile(I1{}, I1{});
                    a_tile(IC<2>{}, I1{});
                    a_tile(IC<3>{}, I0{});
                } else if (wave == 2) {
                    a_tile(IC<2>{}, IC<2>{});
                    if constexpr (MAP) a_tile(IC<3>{}, I1{});
                } else if (wave == 3) {
                    a_tile(IC<3>{}, IC<3>{});
                    a_tile(IC<3>{}, IC<2>{});
                }
            } else if constexpr (kMergeBC) {
                if (!(kTfrag && !MAP && tb_ptr)) {
                    if (wave == 0) {
                        a_tile(I0{}, I0{});
                    } else if (wave == 1) {
                        a_tile(I1{}, I1{});
                    } else if (wave == 2) {
                        // the tile below the diagonal, for wavefront 1's T10, published like T00
                        a_tile(I1{}, I0{});
                        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                        __hip_atomic_store(&a10_ready, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    }
                }
            } else {
                // chunk 32: wavefronts 0 and 1 compute their diagonal tile and go straight on to its
                // inverse; the tile below the diagonal (needed only in C) goes to wavefront 2
                if (wave == 0) {
                    a_tile(I0{}, I0{});
                } else if (wave == 1) {
                    a_tile(I1{}, I1{});
                } else if (wave == 2) {
                    a_tile(I1{}, I0{});
                }
            }
            if constexpr (!MAP && !kSplitKey) {
                if constexpr (G::CT == 4) {
                    if (wave == 2) pa = p_pair(IC<0>{}, IC<0>{});
                    else if (wave == 3) pa = p_pair(IC<2>{}, IC<1>{});
                } else if constexpr (kNoW) {
                    // P has its own buffer: stored at once, read in G after B's barrier
                    if (wave == 2) p_store(IC<0>{}, IC<0>{}, p_pair(IC<0>{}, IC<0>{}));
                    else if (wave == 3) p_store(IC<1>{}, IC<0>{}, p_pair(IC<1>{}, IC<0>{}));
                } else {
                    if (wave == 2) pa = p_pair(IC<0>{}, IC<0>{});
                    else if (wave == 3) pa = p_pair(IC<1>{}, IC<0>{});
                }
            }
            if constexpr (kMergeBC) {
                // chunk 32: the two diagonal inverses run side by side on wavefronts 0
                // and 1; T10 waits for T00 on wavefront 1 through the flag instead of a barrier.  The
                // wait ends: wavefront 0 publishes every chunk without waiting on anything of wavefront
                // 1, and the chunk's barriers keep the two within one chunk of each other.  64K prefill
                // 0.80 -> 0.78 ms against both inverses and T10 on wavefront 0; with the fragments of
                // T diag(b) built here too, 0.75 ms.
                auto tb_build = [&](int ct) {
                    float x[8];
                    lds_slots_f32(&ts[16 * ct + li][0], 0, gq, x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] *= b_s[kmap(0, gq, e)];
                    bf16x8 hi, lo;
                    split_bf16(x, hi, lo);
                    tbs_s[(2 * ct) * kWave + lane] = hi;
                    tbs_s[(2 * ct + 1) * kWave + lane] = lo;
                    if constexpr (kTfrag && MAP) {
                        if (tb_ptr) {
                            u16x8 *d = tb_ptr + static_cast<size_t>(n) * (4 * kWave) + (2 * ct) * kWave + lane;
                            d[0] = __builtin_bit_cast(u16x8, hi);
                            d[kWave] = __builtin_bit_cast(u16x8, lo);
                        }
                    }
                };
                if (kTfrag && !MAP && tb_ptr) {
                    // the fragments MAP stored for this chunk, loaded with its rows
                    if constexpr (ChunkRegs<DK, DV, C, MAP>::TB) {
                        if (wave < 2) {
                            tbs_s[(2 * wave) * kWave + lane] = __builtin_bit_cast(bf16x8, cur.tb[0]);
                            tbs_s[(2 * wave + 1) * kWave + lane] = __builtin_bit_cast(bf16x8, cur.tb[1]);
                        }
                    }
                } else if (wave == 0) {
                    inv_diag(0);
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
                    __hip_atomic_store(&t00_ready, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    if constexpr (kShareTB) tb_build(0);
                } else if (wave == 1) {
                    inv_diag(16);
                    while (__hip_atomic_load(&a10_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < n ||
                           __hip_atomic_load(&t00_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < n)
                        __builtin_amdgcn_s_sleep(1);
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
                    const f32x4 t10 =
                        -mm16(rowfrag(ts, 16, 16), mm16(rowfrag(as, 16, 0), accfrag(ts, 0, 0), zero4), zero4);
                    store_acc(ts, 16, 0, t10);
                    if constexpr (kShareTB) tb_build(1);
                }
            } else if (wave < G::NB) {
                inv_diag(16 * wave);
            }
            if constexpr (kTbFrags) {
                // T's blocks (0,1) and (2,3) are read as zeros by F; last chunk's T diag(b)
                // fragments (written over T's rows) are dead, so clear them again
                if (wave == 0 || wave == 2) {
                    const int r = 16 * wave + lane / 4, c = 16 * wave + 16 + 4 * (lane % 4);
                    *reinterpret_cast<f32x4 *>(&ts[r][c]) = zero4;
                }
            }
        } else if constexpr (!MAP) {
            // no erase term: only P is needed, and its tiles go straight to LDS (A's buffer is unused)
            if constexpr (G::CT == 4) {
                if (wave == 0) {
                    p_store(IC<1>{}, IC<0>{}, p_pair(IC<1>{}, IC<0>{}));
                    p_store(IC<0>{}, IC<0>{}, p_pair(IC<0>{}, IC<0>{}));
                } else if (wave == 1) {
                    p_store(IC<2>{}, IC<0>{}, p_pair(IC<2>{}, IC<0>{}));
                    p_store(IC<2>{}, IC<1>{}, p_pair(IC<2>{}, IC<1>{}));
                } else if (wave == 2) {
                    p_store(IC<3>{}, IC<0>{}, p_pair(IC<3>{}, IC<0>{}));
                } else if (wave == 3) {
                    p_store(IC<3>{}, IC<1>{}, p_pair(IC<3>{}, IC<1>{}));
                }
            } else {
                if (wave == 0) p_store(IC<0>{}, IC<0>{}, p_pair(IC<0>{}, IC<0>{}));
                else if (wave == 1) p_store(IC<1>{}, IC<0>{}, p_pair(IC<1>{}, IC<0>{}));
            }
        }
        if constexpr (DELTA || !MAP) __syncthreads();

        if constexpr (DELTA && !kMergeBC) {
            if constexpr (G::WAVES == 4) __builtin_amdgcn_s_setprio(1);
            // ---- C: the blocks of T below the diagonal (chunk 64: T10, T32 and the lower-left
            // quarter T_BL = -T_BR A_BL T_TL), one output tile per wavefront:
            //   T10 = -T11 A10 T00, T32 = -T33 A32 T22, X = A_BL T_TL, T_BL = -T_BR X.
            // A wavefront recomputes the level-1 block it needs rather than waiting for it;
            // the remaining P tiles fill the shorter chains.
            if constexpr (G::NB == 4) {
                if (wave == 0) {
                    const f32x4 t10 = -mm16(rowfrag(ts, 16, 16), mm16(rowfrag(as, 16, 0), accfrag(ts, 0, 0), zero4), zero4);
                    store_acc(ts, 16, 0, t10);
                    f32x4 x = mm16(rowfrag(as, 32, 0), accfrag(ts, 0, 0), zero4);
                    x = mm16(rowfrag(as, 32, 16), t10, x);
                    store_acc(ts, 32, 0, -mm16(rowfrag(ts, 32, 32), x, zero4));
                } else if (wave == 1) {
                    const f32x4 x = mm16(rowfrag(as, 32, 16), accfrag(ts, 16, 16), zero4);
                    store_acc(ts, 32, 16, -mm16(rowfrag(ts, 32, 32), x, zero4));
                } else if (wave == 2) {
                    const f32x4 t32 =
                        -mm16(rowfrag(ts, 48, 48), mm16(rowfrag(as, 48, 32), accfrag(ts, 32, 32), zero4), zero4);
                    store_acc(ts, 48, 32, t32);
                    const f32x4 x21 = mm16(rowfrag(as, 32, 16), accfrag(ts, 16, 16), zero4);
                    const f32x4 x31 = mm16(rowfrag(as, 48, 16), accfrag(ts, 16, 16), zero4);
                    f32x4 y = mm16(rowfrag(ts, 48, 48), x31, zero4);
                    y = mm16(rowfrag(ts, 48, 32), x21, y);  // T32 row fragments: this wavefront's store
                    store_acc(ts, 48, 16, -y);
                } else if (wave == 3) {
                    const f32x4 t10 = -mm16(rowfrag(ts, 16, 16), mm16(rowfrag(as, 16, 0), accfrag(ts, 0, 0), zero4), zero4);
                    const f32x4 t32 =
                        -mm16(rowfrag(ts, 48, 48), mm16(rowfrag(as, 48, 32), accfrag(ts, 32, 32), zero4), zero4);
                    store_acc(xs, 0, 0, t32);  // private copy, read back as row fragments
                    f32x4 x20 = mm16(rowfrag(as, 32, 0), accfrag(ts, 0, 0), zero4);
                    x20 = mm16(rowfrag(as, 32, 16), t10, x20);
                    f32x4 x30 = mm16(rowfrag(as, 48, 0), accfrag(ts, 0, 0), zero4);
                    x30 = mm16(rowfrag(as, 48, 16), t10, x30);
                    f32x4 y = mm16(rowfrag(ts, 48, 48), x30, zero4);
                    y = mm16(rowfrag(xs, 0, 0), x20, y);
                    store_acc(ts, 48, 0, -y);
                }
            } else {
                if (wave == 0) {
                    const f32x4 t10 = -mm16(rowfrag(ts, 16, 16), mm16(rowfrag(as, 16, 0), accfrag(ts, 0, 0), zero4), zero4);
                    store_acc(ts, 16, 0, t10);
                }
            }
            if constexpr (!MAP && kSplitKey) {
                if (wave == 4) {
                    pa = p_pair(IC<3>{}, IC<0>{});
                } else if (wave == 5) {
                    pa = p_pair(IC<1>{}, IC<0>{});
                    pb = p_pair(IC<2>{}, IC<0>{});
                } else if (wave == 6) {
                    pa = p_pair(IC<3>{}, IC<1>{});
                }
            } else if constexpr (!MAP && G::CT == 4) {
                if (wave == 0) {
                    pb = p_pair(IC<3>{}, IC<0>{});
                } else if (wave == 1) {
                    pa = p_pair(IC<1>{}, IC<0>{});
                    pb = p_pair(IC<2>{}, IC<0>{});
                } else if (wave == 2) {
                    pb = p_pair(IC<3>{}, IC<1>{});
                }
            }
            __syncthreads();
        }

        auto tb_frag = [&](int ct, int s, int hl) -> bf16x8 * {
            if constexpr (kSplitF) return &tbf_s[((ct * G::CS + s) * 2 + hl) * kWave + lane];
            return reinterpret_cast<bf16x8 *>(&ts[16 * ct][0]) + (s * 2 + hl) * kWave + lane;
        };
        if constexpr (DELTA && !kNoW) {
            if constexpr (G::WAVES == 4) __builtin_amdgcn_s_setprio(0);
            // ---- F: P fragments and V^T into LDS (A and K are dead); W A-fragments = W^T tiles
            // (2 s2, ct) and (2 s2 + 1, ct), W = T diag(b exp G) K
            if constexpr (!MAP && kSplitKey) {
                if (wave == 4) {
                    p_store(IC<3>{}, IC<0>{}, pa);
                } else if (wave == 5) {
                    p_store(IC<1>{}, IC<0>{}, pa);
                    p_store(IC<2>{}, IC<0>{}, pb);
                } else if (wave == 6) {
                    p_store(IC<3>{}, IC<1>{}, pa);
                } else if (wave == 7) {
                    p_store(IC<0>{}, IC<0>{}, pa);
                    p_store(IC<2>{}, IC<1>{}, pb);
                }
            } else if constexpr (!MAP) {
                if constexpr (G::CT == 4) {
                    if (wave == 0) {
                        p_store(IC<3>{}, IC<0>{}, pb);
                    } else if (wave == 1) {
                        p_store(IC<1>{}, IC<0>{}, pa);
                        p_store(IC<2>{}, IC<0>{}, pb);
                    } else if (wave == 2) {
                        p_store(IC<0>{}, IC<0>{}, pa);
                        p_store(IC<3>{}, IC<1>{}, pb);
                    } else if (wave == 3) {
                        p_store(IC<2>{}, IC<1>{}, pa);
                    }
                } else {
                    if (wave == 2) p_store(IC<0>{}, IC<0>{}, pa);
                    else if (wave == 3) p_store(IC<1>{}, IC<0>{}, pa);
                }
            }
            if (tid < R::VTHREADS) {
    #pragma unroll
                for (int i = 0; i < R::NV; ++i) {
                    const int e = tid + i * R::VTHREADS, rr = e % C, c8 = e / C;
    #pragma unroll
                    for (int q8 = 0; q8 < 8; ++q8) vt[8 * c8 + q8][col_of(rr)] = cur.v[i][q8];
                }
            }
            if (kTbFrags && (kSplitF || wave < G::CT)) {
                // wavefront ct owns T's row tile ct: one pass over it gives T diag(b exp G) for
                // every W tile of that row and the T diag(b) fragments of U.  With eight
                // wavefronts, wavefronts ct and ct + 4 each build half of the row's W tiles.
                constexpr int MTN = kSplitF ? G::KT / 2 : G::KT;  // W tiles of this wavefront
                const int ct = kSplitF ? wave % G::CT : wave;
                const int half = kSplitF ? wave / G::CT : 0;
                f32x4 accw[MTN];
    #pragma unroll
                for (int mt = 0; mt < MTN; ++mt) accw[mt] = zero4;
                bf16x8 tbh[G::CS], tbl[G::CS];
    #pragma unroll
                for (int s = 0; s < G::CS; ++s) {
                    if (32 * s > 16 * ct + 15) continue;  // T is lower triangular
                    float x[8], xg[8], xb[8];
                    lds_slots_f32(&ts[16 * ct + li][0], s, gq, x);
                    const f32x4 bg0 = *reinterpret_cast<const f32x4 *>(&bg_s[32 * s + 4 * gq]);
                    const f32x4 bg1 = *reinterpret_cast<const f32x4 *>(&bg_s[32 * s + 16 + 4 * gq]);
                    const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&b_s[32 * s + 4 * gq]);
                    const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&b_s[32 * s + 16 + 4 * gq]);
    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        xg[e] = x[e] * bg0[e];
                        xg[4 + e] = x[4 + e] * bg1[e];
                        xb[e] = x[e] * b0[e];
                        xb[4 + e] = x[4 + e] * b1[e];
                    }
                    bf16x8 bgh, bgl;
                    split_bf16(xg, bgh, bgl);
                    split_bf16(xb, tbh[s], tbl[s]);
    #pragma unroll
                    for (int mt = 0; mt < MTN; ++mt) {
                        accw[mt] = mfma_bf16(kfrag(half * MTN + mt, s), bgh, accw[mt]);
                        accw[mt] = mfma_bf16(kfrag(half * MTN + mt, s), bgl, accw[mt]);
                    }
                }
    #pragma unroll
                for (int s2 = 0; s2 < MTN / 2; ++s2) {
                    float x[8];
                    acc_pair_to_slots(accw[2 * s2], accw[2 * s2 + 1], x);
                    const int wi = (ct * G::KS + half * (MTN / 2) + s2) * kWave + lane;
                    split_bf16(x, wf_s[wi], wfl_s[wi]);
                }
                // this wavefront's T rows have all been read (LDS keeps a wavefront's accesses in
                // order); keep the compiler from moving the stores above the loads
                __asm__ __volatile__("" ::: "memory");
                if (half == 0) {
    #pragma unroll
                    for (int s = 0; s < G::CS; ++s) {
                        if (32 * s > 16 * ct + 15) continue;
                        *tb_frag(ct, s, 0) = tbh[s];
                        *tb_frag(ct, s, 1) = tbl[s];
                    }
                }
            } else if (!kTbFrags) {
    #pragma unroll
                for (int p = 0; p < G::CT * G::KS; ++p) {
                    if (p % G::WAVES != wave) continue;
                    const int ct = p % G::CT, s2 = p / G::CT;
                    f32x4 acc0 = zero4, acc1 = zero4;
    #pragma unroll
                    for (int s = 0; s < G::CS; ++s) {
                        if (32 * s > 16 * ct + 15) continue;  // T is lower triangular
                        float x[8];
                        lds_slots_f32(&ts[16 * ct + li][0], s, gq, x);
    #pragma unroll
                        for (int e = 0; e < 8; ++e) x[e] *= bg_s[kmap(s, gq, e)];
                        bf16x8 bgh, bgl;
                        split_bf16(x, bgh, bgl);
                        acc0 = mfma_bf16(kfrag(2 * s2, s), bgh, acc0);
                        acc0 = mfma_bf16(kfrag(2 * s2, s), bgl, acc0);
                        acc1 = mfma_bf16(kfrag(2 * s2 + 1, s), bgh, acc1);
                        acc1 = mfma_bf16(kfrag(2 * s2 + 1, s), bgl, acc1);
                    }
                    float x[8];
                    acc_pair_to_slots(acc0, acc1, x);
                    const int wi = (ct * G::KS + s2) * kWave + lane;
                    split_bf16(x, wf_s[wi], wfl_s[wi]);
                }
            }
            __syncthreads();
        }

        // next chunk's rows: loads in flight during this chunk's slice work
        // MAP: drops in earlier chunks, and whether this chunk ends them (uniform: neither flag is
        // written again before the barrier that ends the chunk).  A restart loads the piece's first
        // chunk next instead of chunk n + 1.
        bool restart = false;
        if constexpr (kDrop) {
            any_flush = any_flush || __builtin_amdgcn_readfirstlane(flush_s[(n - 1) & 1]) != 0;
            if (flush_ok && __builtin_amdgcn_readfirstlane(grow_s) != 0) {
                flush_ok = false;
                restart = any_flush;
            }
        }
        const int next = restart ? n0 : n + 1;
        if (next < n1) load_chunk<DK, DV, C, MAP, PREP>(cur, a, tok_base, seq_len, h, next, tid, tb_ptr);
        if (MAP && key_only) continue;

        // ---- G: per slice: U = (T diag b) V, Delta = U - W St (chunk 32: Delta = T diag(b) R,
        // R = V - diag(exp G) K St), outputs, state update
        if constexpr (G::WAVES == 4) __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int j = 0; j < G::SPW; ++j) {
            const int sl = wave + G::WAVES * j;
            // sl < VT, known per j: VT is a multiple of the wavefront count
            static_assert(G::VT % G::WAVES == 0, "value slices");
            const bool value_slice = j < G::VT / G::WAVES;
            if constexpr (MAP && DELTA) {
                if (restart || (!value_slice && id_zero[j])) continue;
            }
            if constexpr (!DELTA) {
                if (!value_slice) {
                    // identity columns of a piece map: with no erase term only the decay acts
                    const float gl = gam_s[C - 1];
#pragma unroll
                    for (int mt = 0; mt < G::KT; ++mt) St[j][mt] = gl * St[j][mt];
                    continue;
                }
            }
            f32x4 D[G::CT];
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct) D[ct] = zero4;
            bf16x8 Sh[G::KS], Sl[G::KS];  // the chunk's start state as hi + lo pairs
            if constexpr (DELTA || !MAP) {
#pragma unroll
                for (int s = 0; s < G::KS; ++s) {
                    float x[8];
                    acc_pair_to_slots(St[j][2 * s], St[j][2 * s + 1], x);
                    split_bf16(x, Sh[s], Sl[s]);
                }
            }
            if constexpr (kNoW) {
                // R = V - diag(exp G) K St in fp32 (V = 0 on a map's identity columns): where the
                // state already holds what the chunk writes the two nearly cancel, so K St takes
                // the state as hi + lo and R is split again before Delta = T diag(b) R
                f32x4 Rr[G::CT];
#pragma unroll
                for (int ct = 0; ct < G::CT; ++ct) {
                    f32x4 acc = zero4;
#pragma unroll
                    for (int s = 0; s < G::KS; ++s) {
                        const bf16x8 kr = frag(&ks[16 * ct + li][0], s);
                        acc = mfma_bf16(kr, Sh[s], acc);
                        acc = mfma_bf16(kr, Sl[s], acc);
                    }
                    const f32x4 g4 = *reinterpret_cast<const f32x4 *>(&gam_s[16 * ct + 4 * gq]);
                    if (value_slice) {
                        const u16x4 v4 = *reinterpret_cast<const u16x4 *>(&vt[16 * sl + li][col_of(16 * ct + 4 * gq)]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) Rr[ct][r] = fmaf(-g4[r], acc[r], from_bf16(v4[r]));
                    } else {
                        Rr[ct] = -(g4 * acc);
                    }
                }
                bf16x8 Rh[G::CS], Rl[G::CS];
#pragma unroll
                for (int s = 0; s < G::CS; ++s) {
                    float x[8];
                    acc_pair_to_slots(Rr[2 * s], Rr[2 * s + 1], x);
                    split_bf16(x, Rh[s], Rl[s]);
                }
#pragma unroll
                for (int ct = 0; ct < G::CT; ++ct) {
#pragma unroll
                    for (int s = 0; s < G::CS; ++s) {
                        if (32 * s > 16 * ct + 15) continue;  // T is lower triangular
                        bf16x8 th, tl;
                        if constexpr (kShareTB) {
                            th = tbs_s[(2 * ct) * kWave + lane];
                            tl = tbs_s[(2 * ct + 1) * kWave + lane];
                        } else {
                            float x[8];
                            lds_slots_f32(&ts[16 * ct + li][0], s, gq, x);
#pragma unroll
                            for (int e = 0; e < 8; ++e) x[e] *= b_s[kmap(s, gq, e)];
                            split_bf16(x, th, tl);
                        }
                        D[ct] = mfma_bf16(th, Rh[s], D[ct]);
                        D[ct] = mfma_bf16(th, Rl[s], D[ct]);
                        D[ct] = mfma_bf16(tl, Rh[s], D[ct]);
                    }
                }
            } else if (!DELTA) {
                // no erase term: Delta = diag(b) V, four consecutive chunk rows per lane from V^T
#pragma unroll
                for (int ct = 0; ct < G::CT; ++ct) {
                    const u16x4 v4 = *reinterpret_cast<const u16x4 *>(&vt[16 * sl + li][col_of(16 * ct + 4 * gq)]);
                    const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&b_s[16 * ct + 4 * gq]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) D[ct][r] = b4[r] * from_bf16(v4[r]);
                }
            } else if (value_slice) {
#pragma unroll
                for (int s = 0; s < G::CS; ++s) {
                    const bf16x8 vb = frag(&vt[16 * sl + li][0], s);
#pragma unroll
                    for (int ct = 0; ct < G::CT; ++ct) {
                        if (32 * s > 16 * ct + 15) continue;  // T is lower triangular
                        bf16x8 th, tl;
                        if constexpr (kTbFrags) {
                            th = *tb_frag(ct, s, 0);
                            tl = *tb_frag(ct, s, 1);
                        } else {
                            float x[8];
                            lds_slots_f32(&ts[16 * ct + li][0], s, gq, x);
#pragma unroll
                            for (int e = 0; e < 8; ++e) x[e] *= b_s[kmap(s, gq, e)];
                            split_bf16(x, th, tl);
                        }
                        D[ct] = mfma_bf16(th, vb, D[ct]);
                        D[ct] = mfma_bf16(tl, vb, D[ct]);
                    }
                }
            }
            if constexpr (DELTA && !kNoW) {
#pragma unroll
                for (int ct = 0; ct < G::CT; ++ct) {
                    f32x4 acc = zero4;
#pragma unroll
                    for (int s = 0; s < G::KS; ++s) {
                        const bf16x8 wh = wf_s[(ct * G::KS + s) * kWave + lane];
                        acc = mfma_bf16(wh, Sh[s], acc);
                        acc = mfma_bf16(wh, Sl[s], acc);
                        acc = mfma_bf16(wfl_s[(ct * G::KS + s) * kWave + lane], Sh[s], acc);
                    }
                    D[ct] -= acc;  // Delta = U - W St
                }
            }

            if (!MAP && !STATES && value_slice) {
                // O = scale (diag(exp G) Q St + P Delta) with the chunk's start state
                bf16x8 Dh[G::CS], Dl[G::CS];
#pragma unroll
                for (int s = 0; s < G::CS; ++s) {
                    float x[8];
                    acc_pair_to_slots(D[2 * s], D[2 * s + 1], x);
                    split_bf16(x, Dh[s], Dl[s]);
                }
                // O^T tiles: with the operands swapped, lane (gq, li) holds O[16 mt + li][16 sl + 4 gq + r]
                // for r = 0..3, i.e. four consecutive columns of one row -- one 16-byte store
                float *obase = a.o + ((tok_base + t0) * a.H + h) * DV;  // uniform
#pragma unroll
                for (int mt = 0; mt < G::CT; ++mt) {
                    f32x4 qsa = zero4, pd = zero4;
#pragma unroll
                    for (int s = 0; s < G::KS; ++s) {
                        const bf16x8 qa = frag(&qs[16 * mt + li][0], s);
                        qsa = mfma_bf16(Sh[s], qa, qsa);
                        qsa = mfma_bf16(Sl[s], qa, qsa);
                    }
#pragma unroll
                    for (int s = 0; s < G::CS; ++s) {
                        if (32 * s > 16 * mt + 15) continue;
                        const bf16x8 ph = pf_s[((mt * G::CS + s) * 2 + 0) * kWave + lane];
                        const bf16x8 pl = pf_s[((mt * G::CS + s) * 2 + 1) * kWave + lane];
                        pd = mfma_bf16(Dh[s], ph, pd);
                        pd = mfma_bf16(Dl[s], ph, pd);
                        pd = mfma_bf16(Dh[s], pl, pd);
                    }
                    const int row = 16 * mt + li;
                    if (row < L)
                        *reinterpret_cast<f32x4 *>(obase + static_cast<unsigned>(row * a.H * DV + 16 * sl + 4 * gq)) =
                            a.scale * (gam_s[row] * qsa + pd);
                }
            }

            // St' = exp(G_C) St + K^T diag(exp(G_C - G)) Delta
#pragma unroll
            for (int ct = 0; ct < G::CT; ++ct) {
                const f32x4 dec = *reinterpret_cast<const f32x4 *>(&dec_s[16 * ct + 4 * gq]);
                D[ct] *= dec;
            }
            bf16x8 Eh[G::CS], El[G::CS];
#pragma unroll
            for (int s = 0; s < G::CS; ++s) {
                float x[8];
                acc_pair_to_slots(D[2 * s], D[2 * s + 1], x);
                split_bf16(x, Eh[s], El[s]);
            }
            const float gl = gam_s[C - 1];
#pragma unroll
            for (int mt = 0; mt < G::KT; ++mt) {
                f32x4 acc = gl * St[j][mt];
#pragma unroll
                for (int s = 0; s < G::CS; ++s) {
                    const bf16x8 kfr = kfrag(mt, s);
                    acc = mfma_bf16(kfr, Eh[s], acc);
                    acc = mfma_bf16(kfr, El[s], acc);
                }
                St[j][mt] = acc;
            }
            if constexpr (MAP && DELTA) {
                if (!value_slice) {
                    // (a NaN counts as large)
                    const float lim = (kDrop && flush_ok) ? kFlush : 0.f;
                    bool big = false;
#pragma unroll
                    for (int mt = 0; mt < G::KT; ++mt)
#pragma unroll
                        for (int r = 0; r < 4; ++r) big = big || !(fabsf(St[j][mt][r]) <= lim);
                    id_zero[j] = __builtin_amdgcn_ballot_w64(big) == 0;  // uniform over the wavefront
                    if (kDrop && id_zero[j] && flush_ok) {
#pragma unroll
                        for (int mt = 0; mt < G::KT; ++mt) St[j][mt] = zero4;
                        if (lane == 0) flush_s[n & 1] = 1;
                    }
                }
            }
            // 128 x 128 maps: two slices per wavefront, one after the other.  Interleaved, their
            // products need twice the temporaries and spill (85 registers; MAP 0.90 -> 0.68 ms on
            // a 24-head 64K call with this barrier).  The 64 x 64 maps interleave them in
            // registers they have, and are faster that way (0.36 vs 0.38 ms).
            // Chunk 32 (three workgroups per compute unit, 168 registers): the same, else the two
            // slices' hi/lo state pairs spill.
            if constexpr (G::SPW > 1 && (G::WAVES == 8 || C == 32)) __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (G::WAVES == 4) __builtin_amdgcn_s_setprio(0);
        __syncthreads();
        if constexpr (kDrop) {
            if (restart) {
                // the piece's map again from its first chunk (its rows loaded above), with no
                // drops; wavefront 1 waits for T00 and A10 of chunk n0 again
                init_state();
#pragma unroll
                for (int j = 0; j < G::SPW; ++j) id_zero[j] = false;
                if (tid == 0) t00_ready = a10_ready = n0 - 1;
                n = n0 - 1;
            }
        }
    }

    // ---- results
    if (MAP && key_only) return;
#pragma unroll
    for (int j = 0; j < G::SPW; ++j) {
        const int sl = wave + G::WAVES * j;
#pragma unroll
        for (int mt = 0; mt < G::KT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * mt + 4 * gq + r;
                if (MAP)
                    map_out[row * G::MAPW + 16 * sl + li] = St[j][mt][r];
                else if (final_out)
                    final_out[row * DV + 16 * sl + li] = St[j][mt][r];
            }
    }
}

// ---------------------------------------------------------------------------
// chain: start states of every piece, St_in(p+1) = M_p St_in(p) + N_p.  Packed
// sequences: one wavefront per 16-column slice of one head and sequence (state in
// registers, M_p rows loaded as A fragments and split hi + lo, the state split
// hi + lo; the maps do not depend on the state, so (64-wide keys) piece p + 1's are
// loaded while piece p's product runs).  The dense chain splits each slice's rows
// over several wavefronts (chain_kernel below).
// ---------------------------------------------------------------------------
template <int DK, int DV>
struct ChainMap {
    static constexpr int KT = DK / 16, KS = DK / 32;
    float n[KT][4];     // N_p rows 16 mt + 4 gq + r, this lane's column
    float m[KT][KS][8];  // M_p row 16 mt + li, k-slots of step s
};

template <int DK, int DV>
__device__ __forceinline__ void chain_load(ChainMap<DK, DV> &c, const float *mp, int gq, int li, int col) {
    constexpr int KT = DK / 16, KS = DK / 32, MAPW = DV + DK;
#pragma unroll
    for (int mt = 0; mt < KT; ++mt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) c.n[mt][r] = mp[(16 * mt + 4 * gq + r) * MAPW + col];
#pragma unroll
        for (int s = 0; s < KS; ++s) lds_slots_f32(mp + (16 * mt + li) * MAPW + DV, s, gq, c.m[mt][s]);
    }
}

template <int DK, int DV>
__device__ __forceinline__ void chain_step(f32x4 (&St)[DK / 16], const ChainMap<DK, DV> &c) {
    constexpr int KT = DK / 16, KS = DK / 32;
    // M_p = 0 (every identity slice of the map dropped or decayed to zero): St = N_p, no product
    bool nz = false;
#pragma unroll
    for (int mt = 0; mt < KT; ++mt)
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int e = 0; e < 8; ++e) nz = nz || c.m[mt][s][e] != 0.f;
    if (__builtin_amdgcn_ballot_w64(nz) == 0) {
#pragma unroll
        for (int mt = 0; mt < KT; ++mt) St[mt] = f32x4{c.n[mt][0], c.n[mt][1], c.n[mt][2], c.n[mt][3]};
        return;
    }
    bf16x8 Sh[KS], Sl[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        float x[8];
        acc_pair_to_slots(St[2 * s], St[2 * s + 1], x);
        split_bf16(x, Sh[s], Sl[s]);
    }
#pragma unroll
    for (int mt = 0; mt < KT; ++mt) {
        f32x4 acc = {c.n[mt][0], c.n[mt][1], c.n[mt][2], c.n[mt][3]};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            bf16x8 mh, ml;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = c.m[mt][s][e];
            split_bf16(x, mh, ml);
            acc = mfma_bf16(mh, Sh[s], acc);
            acc = mfma_bf16(mh, Sl[s], acc);
            acc = mfma_bf16(ml, Sh[s], acc);
        }
        St[mt] = acc;
    }
}

// The serial part shared by both layouts: start states of P pieces from St (the first
// piece's), St <- M_p St + N_p.  map_at(p) points at piece p's map [DK][DV + DK];
// store_at(St, p) records piece p's start state.
template <int DK, int DV, typename MapAt, typename StoreAt>
__device__ __forceinline__ void chain_run(f32x4 (&St)[DK / 16], int P, MapAt map_at, StoreAt store_at,
                                          int gq, int li, int col) {
    if constexpr (DK == 64) {
        // two map buffers used in turn, so piece p + 1's loads overlap piece p's product
        ChainMap<DK, DV> ma, mb;
        if (P > 1) chain_load<DK, DV>(ma, map_at(0), gq, li, col);
        for (int p = 0; p < P; p += 2) {
            store_at(St, p);
            if (p + 1 >= P) break;
            if (p + 1 < P - 1) chain_load<DK, DV>(mb, map_at(p + 1), gq, li, col);
            chain_step<DK, DV>(St, ma);
            store_at(St, p + 1);
            if (p + 2 >= P) break;
            if (p + 2 < P - 1) chain_load<DK, DV>(ma, map_at(p + 2), gq, li, col);
            chain_step<DK, DV>(St, mb);
        }
    } else {
        // 128-wide maps would not fit twice in registers: load each in place
        for (int p = 0; p < P; ++p) {
            store_at(St, p);
            if (p == P - 1) break;
            ChainMap<DK, DV> mc;
            chain_load<DK, DV>(mc, map_at(p), gq, li, col);
            chain_step<DK, DV>(St, mc);
        }
    }
}

// Dense chain: one workgroup per head and 16-column slice, DK / 32 wavefronts, each owning
// 32 rows (two row tiles) of the slice.  A wavefront multiplies its rows of M_p with the
// whole slice and adds its rows of N_p; the slice is exchanged through LDS once per piece
// (two buffers used in turn, so one barrier per piece).  Each wavefront loads only its rows of
// the maps, a piece ahead, so the loads of piece p + 1 overlap piece p's product (loading two
// pieces ahead was tried: no faster).  Per piece: 2.7 us at 128 x 128, 1.0 us at 64 x 64.
template <int DK>
struct ChainRows {
    static constexpr int KS = DK / 32;
    float n[2][4];      // N_p rows 16 mt + 4 gq + r of this wavefront's two row tiles, this lane's column
    float m[2][KS][8];  // M_p row 16 mt + li, k-slots of step s
};

template <int DK, int DV>
__device__ __forceinline__ void chain_rows_load(ChainRows<DK> &c, const float *mp, int mt0, int gq, int li,
                                                int col) {
    constexpr int KS = DK / 32, MAPW = DV + DK;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int mt = mt0 + rt;
#pragma unroll
        for (int r = 0; r < 4; ++r) c.n[rt][r] = mp[(16 * mt + 4 * gq + r) * MAPW + col];
#pragma unroll
        for (int s = 0; s < KS; ++s) lds_slots_f32(mp + (16 * mt + li) * MAPW + DV, s, gq, c.m[rt][s]);
    }
}

template <int DK, int DV>
__global__ __launch_bounds__(kWave * (DK / 32)) void chain_kernel(const float *__restrict__ maps,
                                                                  const float *__restrict__ s0,
                                                                  float *__restrict__ starts, int P) {
    constexpr int KT = DK / 16, KS = DK / 32, VT = DV / 16, MAPW = DV + DK;
    __shared__ f32x4 sbuf[2][KT][kWave];  // the slice in accumulator layout, tile mt, lane
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave, gq = lane / 16, li = lane % 16;
    const int sl = blockIdx.x % VT;
    const size_t bh = blockIdx.x / VT;
    const int col = 16 * sl + li;
    const int mt0 = 2 * wave;  // this wavefront's row tiles: mt0, mt0 + 1
    const float *mbase = maps + bh * (P - 1) * DK * MAPW;
    auto map_at = [&](int p) { return mbase + static_cast<size_t>(p) * DK * MAPW; };

    f32x4 own[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            own[rt][r] = s0 ? s0[(bh * DK + 16 * (mt0 + rt) + 4 * gq + r) * DV + col] : 0.f;
    auto publish = [&](int p) {  // piece p's start state: into LDS buffer p & 1 and to HBM
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            sbuf[p & 1][mt0 + rt][lane] = own[rt];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                starts[((bh * P + p) * DK + 16 * (mt0 + rt) + 4 * gq + r) * DV + col] = own[rt][r];
        }
    };
    // own rows of piece p + 1's start state from piece p's: M_p St + N_p (just N_p where this
    // wavefront's rows of M_p are all zero, as the map pass leaves them once every identity slice is
    // dropped or has decayed to zero: then no product and no read of the slice)
    auto step = [&](int p, const ChainRows<DK> &c) {
        bool nz = false;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ss = 0; ss < KS; ++ss)
#pragma unroll
                for (int e = 0; e < 8; ++e) nz = nz || c.m[rt][ss][e] != 0.f;
        if (__builtin_amdgcn_ballot_w64(nz) == 0) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) own[rt] = f32x4{c.n[rt][0], c.n[rt][1], c.n[rt][2], c.n[rt][3]};
            return;
        }
        bf16x8 Sh[KS], Sl[KS];
#pragma unroll
        for (int ss = 0; ss < KS; ++ss) {
            float x[8];
            acc_pair_to_slots(sbuf[p & 1][2 * ss][lane], sbuf[p & 1][2 * ss + 1][lane], x);
            split_bf16(x, Sh[ss], Sl[ss]);
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            f32x4 acc = {c.n[rt][0], c.n[rt][1], c.n[rt][2], c.n[rt][3]};
#pragma unroll
            for (int ss = 0; ss < KS; ++ss) {
                bf16x8 mh, ml;
                split_bf16(c.m[rt][ss], mh, ml);
                acc = mfma_bf16(mh, Sh[ss], acc);
                acc = mfma_bf16(mh, Sl[ss], acc);
                acc = mfma_bf16(ml, Sh[ss], acc);
            }
            own[rt] = acc;
        }
    };
    ChainRows<DK> ma, mb;
    if (P > 1) chain_rows_load<DK, DV>(ma, map_at(0), mt0, gq, li, col);
    publish(0);
    __syncthreads();
    for (int p = 0; p + 1 < P; p += 2) {
        if (p + 1 < P - 1) chain_rows_load<DK, DV>(mb, map_at(p + 1), mt0, gq, li, col);
        step(p, ma);
        publish(p + 1);
        __syncthreads();
        if (p + 2 >= P) break;
        if (p + 2 < P - 1) chain_rows_load<DK, DV>(ma, map_at(p + 2), mt0, gq, li, col);
        step(p + 1, mb);
        publish(p + 2);
        __syncthreads();
    }
}

// Packed sequences: one wavefront per (sequence, head, 16 value columns).  The first
// piece starts from the sequence's pool slot (or zeros); an empty sequence that is to
// start from zeros gets a zero final state in its slot.
template <int DK, int DV>
__global__ __launch_bounds__(kWave) void chain_varlen_kernel(SeqTable sq, const float *__restrict__ maps,
                                                             float *__restrict__ starts,
                                                             float *__restrict__ pool, int H) {
    constexpr int KT = DK / 16, VT = DV / 16, MAPW = DV + DK;
    const int lane = threadIdx.x, gq = lane / 16, li = lane % 16;
    const int sl = blockIdx.x % VT;
    const int h = (blockIdx.x / VT) % H;
    const int s = blockIdx.x / (VT * H);
    const int col = 16 * sl + li;
    const int P = sq.pstart[s + 1] - sq.pstart[s];
    const int slot = sq.slot[s];
    float *st = slot >= 0 ? pool + (static_cast<size_t>(slot) * H + h) * DK * DV : nullptr;
    f32x4 St[KT];
    if (st && sq.init[s]) {
#pragma unroll
        for (int mt = 0; mt < KT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) St[mt][r] = st[(16 * mt + 4 * gq + r) * DV + col];
    } else {
#pragma unroll
        for (int mt = 0; mt < KT; ++mt) St[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (P == 0) {
        if (st && !sq.init[s]) {
#pragma unroll
            for (int mt = 0; mt < KT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) st[(16 * mt + 4 * gq + r) * DV + col] = 0.f;
        }
        return;
    }
    const int p0 = sq.pstart[s], m0 = sq.mstart[s];
    chain_run<DK, DV>(
        St, P, [&](int p) { return maps + (static_cast<size_t>(m0 + p) * H + h) * DK * MAPW; },
        [&](const f32x4 (&S)[KT], int p) {
#pragma unroll
            for (int mt = 0; mt < KT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    starts[((static_cast<size_t>(p0 + p) * H + h) * DK + 16 * mt + 4 * gq + r) * DV + col] =
                        S[mt][r];
        },
        gq, li, col);
}

// Piece plan: one round of workgroups (slots = 256 compute units x the workgroups
// one unit holds: 512 for 64 x 64 heads, 256 otherwise), at least eight chunks per
// piece, and no empty pieces.  Rounding the piece count down keeps the grid within
// the slots: a workgroup over them would run alone in a further round.  (128 x 128,
// 24 heads: 10 pieces in one round 1.49 ms against 21 pieces in two rounds 1.52 ms;
// rounding up to 22 pieces and a third round of 16 workgroups took 2.57 ms.)
struct PiecePlan {
    int P, piece_chunks;
};
PiecePlan piece_plan(int BH, int N, int slots) {
    int P = slots / BH;
    P = max(1, min(P, N / 8));
    const int pc = (N + P - 1) / P;
    return {(N + pc - 1) / pc, pc};
}

// Workspace of a dense call: the piece maps, the piece start states and (tfrag: 128 x 128 heads,
// gated delta rule) the T diag(b) fragments of every chunk, 4 KiB each.
template <int DK, int DV, int C>
constexpr bool kTfragPlan = DK == 128 && DV == 128 && C == 32;
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
template <int DK, int DV, int C>
size_t chunk_ws_bytes(int B, int T, int H, bool tfrag) {
    const int N = (T + C - 1) / C;
    const int BH = B * H;
    const int P = piece_plan(BH, N, kPlanSlots<DK, DV, C>).P;
    if (P == 1) return 0;
    const size_t maps = static_cast<size_t>(BH) * (P - 1) * DK * (DV + DK) * 4;
    const size_t starts = static_cast<size_t>(BH) * P * DK * DV * 4;
    if (tfrag && kTfragPlan<DK, DV, C>) return align256(maps) + align256(starts) + static_cast<size_t>(BH) * N * 4096;
    return align256(maps) + starts;
}

template <int DK, int DV, int C, bool DELTA, bool PREP = false>
hipError_t run_chunk(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                     const float *beta, const float *s0, float *o, float *s_out, int B, int T, int H,
                     void *ws, hipStream_t stream, float *chunk_states = nullptr, const PrepIn *pin = nullptr,
                     bool tfrag = false) {
    const int N = (T + C - 1) / C;
    const int BH = B * H;
    const PiecePlan plan = piece_plan(BH, N, kPlanSlots<DK, DV, C>);
    const int P = plan.P;
    ChunkArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o; a.s_final = s_out;
    a.chunk_states = chunk_states;
    if constexpr (PREP) {
        a.conv_w = pin->conv_w;
        a.rate = pin->rate;
        a.bias = pin->bias;
        a.conv_in = pin->conv_in;
    }
    a.T = T; a.H = H; a.BH = BH; a.P = P; a.N = N;
    a.sq = SeqTable{};
    auto grid = [](int items) { return dim3((items + kXcds - 1) / kXcds * kXcds); };
    a.piece_chunks = plan.piece_chunks;
    a.scale = 1.0f / sqrtf(static_cast<float>(DK));
    // the OUT pass, with chunk start states written only where the gradients need them
    auto launch_out = [&](int items) {
        if constexpr (DK == DV && (DK == 64 || DK == 128) && C == 32 && !PREP) {
            if (chunk_states) {
                hipLaunchKernelGGL((chunk_kernel<DK, DV, C, false, DELTA, true>), grid(items), dim3(kWave * kWavesOf<DK, DV>), 0, stream, a);
                return hipGetLastError();
            }
        }
        if (chunk_states) return hipErrorInvalidValue;
        hipLaunchKernelGGL((chunk_kernel<DK, DV, C, false, DELTA, false, PREP>), grid(items), dim3(kWave * kWavesOf<DK, DV>), 0, stream, a);
        return hipGetLastError();
    };
    if (P == 1) {
        a.s_start = s0;
        a.items = BH;
        return launch_out(BH);
    }
    const size_t maps_bytes = static_cast<size_t>(BH) * (P - 1) * DK * (DV + DK) * 4;
    const size_t starts_bytes = static_cast<size_t>(BH) * P * DK * DV * 4;
    float *maps = static_cast<float *>(ws);
    float *starts = reinterpret_cast<float *>(static_cast<char *>(ws) + align256(maps_bytes));
    a.maps = maps;
    a.items = BH * (P - 1);
    if (tfrag && DELTA && !PREP && kTfragPlan<DK, DV, C> && !chunk_states) {
        // MAP also covers the last piece, keyside only, so OUT finds every chunk's fragments
        a.tfrag = reinterpret_cast<u16x8 *>(static_cast<char *>(ws) + align256(maps_bytes) + align256(starts_bytes));
        a.items = BH * P;
    }
    hipLaunchKernelGGL((chunk_kernel<DK, DV, C, true, DELTA, false, PREP>), grid(a.items), dim3(kWave * kWavesOf<DK, DV>), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((chain_kernel<DK, DV>), dim3(BH * (DV / 16)), dim3(kWave * (DK / 32)), 0, stream,
                       static_cast<const float *>(maps), s0, starts, P);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    a.s_start = starts;
    a.items = BH * P;
    return launch_out(BH * P);
}

template <int DK, int DV, int C, bool DELTA>
hipError_t run_chunk_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v, const float *g,
                            const float *beta, const VarlenLayout &L, const int *table_dev, float *pool,
                            float *o, int S, int H, void *ws, hipStream_t stream) {
    const int *t = table_dev;
    SeqTable sq;
    sq.piece_seq = t;
    sq.map_seq = t + L.NP;
    sq.tok0 = t + L.NP + L.NM;
    sq.len = sq.tok0 + S;
    sq.pstart = sq.len + S;
    sq.mstart = sq.pstart + S + 1;
    sq.slot = sq.mstart + S + 1;
    sq.init = sq.slot + S;
    sq.out_order = sq.init + S;
    float *maps = reinterpret_cast<float *>(static_cast<char *>(ws) + L.maps_off);
    float *starts = reinterpret_cast<float *>(static_cast<char *>(ws) + L.starts_off);
    ChunkArgs a{};
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.o = o;
    a.H = H; a.piece_chunks = L.pc;
    a.scale = 1.0f / sqrtf(static_cast<float>(DK));
    a.sq = sq;
    a.pool = pool;
    auto grid = [](int items) { return dim3((items + kXcds - 1) / kXcds * kXcds); };
    if (L.NM > 0) {
        a.maps = maps;
        a.items = L.NM * H;
        hipLaunchKernelGGL((chunk_kernel<DK, DV, C, true, DELTA>), grid(a.items), dim3(kWave * kWavesOf<DK, DV>), 0, stream, a);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((chain_varlen_kernel<DK, DV>), dim3(S * H * (DV / 16)), dim3(kWave), 0, stream, sq,
                       static_cast<const float *>(maps), starts, pool, H);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || L.NP == 0) return err;
    a.s_start = starts;
    a.items = kXcds * L.out_per_xcd * H;  // a multiple of kXcds: each XCD's range holds whole piece slots
    hipLaunchKernelGGL((chunk_kernel<DK, DV, C, false, DELTA>), grid(a.items), dim3(kWave * kWavesOf<DK, DV>), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// Plan for packed sequences: pieces of pc chunks (at least 8, and enough to give about
// one round of workgroups over all heads), the host table and the workspace layout.
bool varlen_layout(const int *cu, int S, int H, int dk, int dv, int chunk, VarlenLayout *L) {
    long long chunk_heads = 0;
    for (int s = 0; s < S; ++s) chunk_heads += static_cast<long long>((cu[s + 1] - cu[s] + chunk - 1) / chunk) * H;
    const long long slots = plan_slots(dk, dv, chunk);
    long long pc = (chunk_heads + slots - 1) / slots;
    if (pc < 8) pc = 8;
    long long NP = 0, NM = 0;
    for (int s = 0; s < S; ++s) {
        const long long n = (cu[s + 1] - cu[s] + chunk - 1) / chunk;
        const long long P = (n + pc - 1) / pc;
        NP += P;
        NM += P > 1 ? P - 1 : 0;
    }
    if ((NP + kXcds) * H > 0x7fffffffLL || static_cast<long long>(S) * H * (dv / 16) > 0x7fffffffLL) return false;
    L->chunk = chunk;
    L->pc = static_cast<int>(pc);
    L->NP = static_cast<int>(NP);
    L->NM = static_cast<int>(NM);
    L->out_per_xcd = static_cast<int>((NP + kXcds - 1) / kXcds);
    L->table_ints = static_cast<size_t>(NP + NM) + 6 * static_cast<size_t>(S) + 2 +
                    static_cast<size_t>(kXcds) * L->out_per_xcd;
    auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
    L->maps_off = up(L->table_ints * 4);
    L->starts_off = L->maps_off + up(static_cast<size_t>(NM) * H * dk * (dv + dk) * 4);
    L->bytes = L->starts_off + static_cast<size_t>(NP) * H * dk * dv * 4;
    return true;
}

void varlen_table(const int *cu, int S, const int *slots, const int *init, const VarlenLayout &L, int *t) {
    int *piece_seq = t, *map_seq = t + L.NP, *tok0 = t + L.NP + L.NM, *len = tok0 + S;
    int *pstart = len + S, *mstart = pstart + S + 1, *slot = mstart + S + 1, *ini = slot + S;
    int gp = 0, gm = 0;
    for (int s = 0; s < S; ++s) {
        const int n = cu[s + 1] - cu[s];  // tokens
        tok0[s] = cu[s];
        len[s] = n;
        pstart[s] = gp;
        mstart[s] = gm;
        slot[s] = slots ? slots[s] : s;
        ini[s] = init ? (init[s] != 0) : 1;
        const int nchunks = (n + L.chunk - 1) / L.chunk;
        const int P = (nchunks + L.pc - 1) / L.pc;
        for (int p = 0; p < P; ++p) piece_seq[gp++] = s;
        for (int p = 0; p + 1 < P; ++p) map_seq[gm++] = s;
    }
    pstart[S] = gp;
    mstart[S] = gm;
    // OUT's dealing: work items go to the XCDs in contiguous ranges of out_per_xcd piece slots, and
    // the dispatcher starts them in index order.  Pieces by length (chunks), longest first, each to
    // the XCD with the least work so far that has a free slot; inside an XCD longest first, so no long
    // prompt starts last and no XCD gets all the long ones.
    int *order = ini + S;
    const int ppx = L.out_per_xcd;
    std::vector<int> chunks(static_cast<size_t>(L.NP)), byLen(static_cast<size_t>(L.NP));
    for (int s = 0; s < S; ++s) {
        const int nchunks = (len[s] + L.chunk - 1) / L.chunk;
        for (int p = pstart[s]; p < pstart[s + 1]; ++p) {
            const int left = nchunks - (p - pstart[s]) * L.pc;
            chunks[p] = left < L.pc ? left : L.pc;
        }
    }
    for (int p = 0; p < L.NP; ++p) byLen[p] = p;
    std::stable_sort(byLen.begin(), byLen.end(), [&](int x, int y) { return chunks[x] > chunks[y]; });
    long long load[kXcds] = {};
    int used[kXcds] = {};
    for (int i = 0; i < kXcds * ppx; ++i) order[i] = -1;
    for (int p : byLen) {
        int best = -1;
        for (int x = 0; x < kXcds; ++x)
            if (used[x] < ppx && (best < 0 || load[x] < load[best])) best = x;
        order[best * ppx + used[best]++] = p;
        load[best] += chunks[p];
    }
}

hipError_t launch_prefill_chunk_varlen(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                       const float *g, const float *beta, const int *cu, int S,
                                       const int *slots, const int *init, float *pool, float *o,
                                       int H, int dk, int dv, int chunk, bool delta, void *ws,
                                       hipStream_t stream) {
    VarlenLayout L;
    if (!varlen_layout(cu, S, H, dk, dv, chunk, &L)) return hipErrorInvalidValue;
    std::vector<int> table(L.table_ints);
    varlen_table(cu, S, slots, init, L, table.data());
    // the table is pageable host memory: the copy has read it by the time the call returns
    hipError_t err = hipMemcpyAsync(ws, table.data(), L.table_ints * 4, hipMemcpyHostToDevice, stream);
    if (err != hipSuccess) return err;
    const int *tdev = static_cast<const int *>(ws);
#define GDN_RUNV(DK_, DV_, C_)                                                                           \
    if (dk == DK_ && dv == DV_ && chunk == C_)                                                           \
        return delta ? run_chunk_varlen<DK_, DV_, C_, true>(q, k, v, g, beta, L, tdev, pool, o, S, H, ws, stream) \
                     : run_chunk_varlen<DK_, DV_, C_, false>(q, k, v, g, beta, L, tdev, pool, o, S, H, ws, stream);
    GDN_CHUNK_CASES(GDN_RUNV)
#undef GDN_RUNV
    return hipErrorInvalidValue;
}

namespace {
}  // namespace


namespace {

// The carried convolution window after a call: the last three raw inputs of [window before the
// call, the call's tokens], oldest first, one thread per (sequence, channel).  Each thread reads
// its three old entries before writing any, so the window may be updated in place; it runs
// after the chunk kernels, which read the old window at the first chunk.
template <int DK, int DV>
__global__ __launch_bounds__(256) void conv_window_kernel(const uint16_t *__restrict__ xq, const uint16_t *__restrict__ xk,
                                                          const uint16_t *__restrict__ xv, const float *cin, float *cout,
                                                          int B, int T, int H) {
    const int nch = H * (2 * DK + DV);
    const long long idx = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= static_cast<long long>(B) * nch) return;
    const int b = static_cast<int>(idx / nch), c = static_cast<int>(idx % nch);
    const uint16_t *x;
    int W, cc;  // the channel's tensor, its row width and the channel inside it
    if (c < H * DK) { x = xq; W = H * DK; cc = c; }
    else if (c < 2 * H * DK) { x = xk; W = H * DK; cc = c - H * DK; }
    else { x = xv; W = H * DV; cc = c - 2 * H * DK; }
    float w[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        const int p = T - 3 + i;  // the token at window entry i (negative: an entry of the old window)
        w[i] = p >= 0 ? from_bf16(x[(static_cast<size_t>(b) * T + p) * W + cc])
                      : (cin ? cin[static_cast<size_t>(idx) * 3 + 3 + p] : 0.f);
    }
#pragma unroll
    for (int i = 0; i < 3; ++i) cout[static_cast<size_t>(idx) * 3 + i] = w[i];
}

}  // namespace

bool prepare_prefill_supported(int dk, int dv) { return dk == dv && (dk == 64 || dk == 128); }

// Fused preparation + prefill: always 32-token chunks (the preparation's raw rows must fit
// beside three workgroups' LDS per compute unit for 64-wide heads)
size_t prepare_prefill_workspace(int B, int T, int H, int dk, int dv) {
    return prefill_chunk_workspace(B, T, H, dk, dv, 32);
}

hipError_t launch_prepare_prefill(const uint16_t *xq, const uint16_t *xk, const uint16_t *xv, const float *conv_w,
                                  const float *a_raw, const float *b_raw, const float *rate, const float *bias,
                                  const float *conv_in, float *conv_out, const float *s0, float *o, float *s_out,
                                  int B, int T, int H, int dk, int dv, bool delta, void *ws, hipStream_t stream) {
    if (!prepare_prefill_supported(dk, dv)) return hipErrorInvalidValue;
    const PrepIn pin{conv_w, rate, bias, conv_in};
    hipError_t err = hipSuccess;
    if (T > 0) {
        if (dk == 64)
            err = delta ? run_chunk<64, 64, 32, true, true>(xq, xk, xv, a_raw, b_raw, s0, o, s_out, B, T, H, ws, stream, nullptr, &pin)
                        : run_chunk<64, 64, 32, false, true>(xq, xk, xv, a_raw, b_raw, s0, o, s_out, B, T, H, ws, stream, nullptr, &pin);
        else
            err = delta ? run_chunk<128, 128, 32, true, true>(xq, xk, xv, a_raw, b_raw, s0, o, s_out, B, T, H, ws, stream, nullptr, &pin)
                        : run_chunk<128, 128, 32, false, true>(xq, xk, xv, a_raw, b_raw, s0, o, s_out, B, T, H, ws, stream, nullptr, &pin);
        if (err != hipSuccess) return err;
    }
    if (conv_out) {
        const long long n = static_cast<long long>(B) * H * (2 * dk + dv);
        const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
        if (dk == 64)
            hipLaunchKernelGGL((conv_window_kernel<64, 64>), dim3(blocks), dim3(256), 0, stream, xq, xk, xv, conv_in, conv_out, B, T, H);
        else
            hipLaunchKernelGGL((conv_window_kernel<128, 128>), dim3(blocks), dim3(256), 0, stream, xq, xk, xv, conv_in, conv_out, B, T, H);
        err = hipGetLastError();
    }
    return err;
}

size_t prefill_chunk_workspace(int B, int T, int H, int dk, int dv, int chunk, bool tfrag) {
#define GDN_WS(DK_, DV_, C_) \
    if (dk == DK_ && dv == DV_ && chunk == C_) return chunk_ws_bytes<DK_, DV_, C_>(B, T, H, tfrag);
    GDN_CHUNK_CASES(GDN_WS)
#undef GDN_WS
    return 0;
}

hipError_t launch_prefill_chunk(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                const float *g, const float *beta, const float *s0, float *o,
                                float *s_out, int B, int T, int H, int dk, int dv, int chunk,
                                bool delta, void *ws, hipStream_t stream, float *chunk_states, bool tfrag) {
#define GDN_RUN(DK_, DV_, C_)                                                                      \
    if (dk == DK_ && dv == DV_ && chunk == C_)                                                     \
        return delta ? run_chunk<DK_, DV_, C_, true>(q, k, v, g, beta, s0, o, s_out, B, T, H, ws, stream,  \
                                                     chunk_states, nullptr, tfrag)                         \
                     : run_chunk<DK_, DV_, C_, false>(q, k, v, g, beta, s0, o, s_out, B, T, H, ws, stream, \
                                                      chunk_states);
    GDN_CHUNK_CASES(GDN_RUN)
#undef GDN_RUN
    return hipErrorInvalidValue;
}

}  // namespace gdn
