// TTT-Linear forward on gfx950: segment-parallel chunked gradient descent,
// walked in super-blocks of up to 64 tokens.
//
// What is computed ("Test-Time Training (TTT)" summary page: "TTT definition",
// examples 1 and 2, "TTT-Linear", "Mini-batch gradient descent"; the parallel
// formulation of "Test-Time Training with KV Binding Is Secretly Linear
// Attention"): per (batch, head), with chunk-start state W_c and per-token eta,
//   U_c     = V_c - K_c W_c (MSE)  or  V_c (inner product)
//   O_c     = Q_c W_c + ((Q_c K_c^T) * M_incl * eta^T) U_c
//   W_{c+1} = W_c + K_c^T diag(eta_c) U_c.
//
// How it is laid out on the chip (not on the pages):
//  * Column separability.  Column j of W only ever meets column j of V, U
//    and O, so one wave owns a 16-column block of the state and keeps it in
//    MFMA accumulators (fp32) for a whole segment.  A workgroup = one wave
//    per column block, sharing the token tiles it stages in LDS.
//  * Super-blocks.  Tokens are walked in super-blocks of up to 64 tokens (four
//    16-token tiles), placed so that every token of a super-block takes its
//    residual from the same state:
//      b <= 64: a super-block is floor(64/b) whole chunks.  With R the running
//        state at its start and, for tiles j < i in different chunks,
//        L_ij = K_i K_j^T diag(eta_j), the chunk rule reads (I + L) U = V - K R.
//        Block forward substitution applies T = (I + L)^-1 to K and V, which
//        do not depend on the state: U = Vt - Kt R with Kt = T K, Vt = T V.
//        (Exact up to rounding; it is the chunk recurrence written for four
//        tiles at once.)
//      b > 64: a super-block lies inside one chunk and every residual uses the
//        chunk-start snapshot S: U = V - K S.
//    Either way O = Q R + (Q K^T * M_incl * eta^T) U over the super-block (the
//    running state is the sum of all earlier updates) and R <- R + K^T diag(eta) U.
//    One super-block is one step of the serial chain, and every product in it
//    has four independent 16-token tiles.
//  * Segments.  The chunk update is affine in the state,
//    W_{c+1} = (I - K_c^T H_c K_c) W_c + K_c^T H_c V_c, so a run of whole
//    chunks (a segment) is one affine map W -> W - P W + B.  Two kernels:
//      summary : every segment (but the last, causal) computes P and B from
//                its keys/values alone, all segments in parallel;
//      replay  : every segment first builds its start state by applying the
//                maps of the segments before it to w_init (the chain),
//                W_start(s+1) = W_s - P_s W_s + B_s, then replays its
//                super-blocks and writes its outputs; the last segment writes
//                the final state.
//    For the inner-product loss P = 0 and the chain is a running sum.
//  * Non-causal order: summary over all segments, the chain to W_final (one
//    workgroup per head), then an apply kernel O = Q W_final.
//  * bf16 with d = 64 and b <= 64 runs producer/consumer versions of summary
//    and replay (eight waves; see the section that defines them); the other
//    shapes run the four-wave versions.
#include "ttt_device.h"
#include "ttt_internal.h"

#include <stdlib.h>

namespace tttk {

struct LinParams {
    const void *q, *k, *v;
    const float *eta, *w_init;
    void *out;
    float *w_final;
    void *wsP;      // [NH][Ssum][d][d] element type (MSE only)
    float *wsB;     // [NH][Ssum][d/16 col blocks][d/16 row blocks][64 lanes][4] fp32
    float *wsW0;    // [NH][d][d]: copy of w_init for the replay (causal, S > 1,
                    // w_final == w_init); null otherwise
    int NH, Tq, Tkv, chunk, seg_tokens, S, Ssum, seg_q, Sq;
};

constexpr int SB = 64;  // tokens per super-block tile (four 16-token tiles)

// Which tensors a kernel stages; STAGE_SWZ: bf16 tiles use the swizzled
// layout below instead of padded rows; STAGE_PERM: padded bf16 rows whose
// 4-column groups are permuted (pcol below) so that the two 16-column halves a
// 32-deep row fragment pairs are one 16-byte read.
enum { STAGE_Q = 1, STAGE_K = 2, STAGE_V = 4, STAGE_E = 8, STAGE_SWZ = 16, STAGE_PERM = 32 };

// Swizzled position of the 4-column group starting at column col (a multiple
// of 4) in row row of an unpadded bf16 tile: inside each 64-column group the
// 8-column chunk index is XORed with a 3-bit function of row bits 0-2 and the
// two 4-column halves are exchanged on row bit 3.  The row fragments (16 rows,
// 4 columns each), the transposing reads (4 rows x 16 columns per 16 lanes)
// and the 16-byte stores then spread over the banks.  A 4-column group is
// never split, so every 8-byte access stays contiguous.
__device__ __forceinline__ int swz(int row, int col)
{
    const int v = ((row & 3) << 1) | ((row >> 2) & 1), hs = (row >> 3) & 1;
    return (col & ~63) | ((((col >> 3) & 7) ^ v) << 3) | ((((col >> 2) & 1) ^ hs) << 2);
}

// Permuted position of the 4-column group starting at column col (a multiple
// of 4): inside each 32-column block, group g of the first 16 columns goes to
// 8g and group g of the second 16 to 8g + 4.  A 32-deep row fragment pairs
// columns 32s + 4g + (0..3) with 32s + 16 + 4g + (0..3) (the state's
// accumulator order), which then lie side by side.
__device__ __forceinline__ bf16x8 as_bf8x(const __bf16 *p)
{
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ int pcol(int col)
{
    return (col & ~31) | (((col >> 2) & 3) << 3) | (((col >> 4) & 1) << 2) | (col & 3);
}

// LDS image of one 64-token super-block.  bf16: token-major tiles; fragments
// that need four consecutive tokens of one feature come from the transposing
// read.  fp32: queries token-major, keys and values feature-major (rows
// padded), so both fragment kinds are plain 16-byte or scalar reads.
template <typename E, int D, int ST> struct alignas(16) SbTile {
    static constexpr bool TR = sizeof(E) == 2;
    static constexpr bool LQ = (ST & STAGE_Q) != 0, LK = (ST & STAGE_K) != 0, LV = (ST & STAGE_V) != 0;
    static constexpr bool SW = TR && (ST & STAGE_SWZ) != 0;
    static constexpr bool PM = TR && !SW && (ST & STAGE_PERM) != 0;
    static constexpr int RP = SW ? D : D + (TR ? 8 : 4);  // token-major row pitch
    static constexpr int FP = SB + 4;            // feature-major row pitch (fp32)
    E qs[LQ ? SB : 1][RP];
    E ks[(LK && TR) ? SB : 1][RP];
    E vs[(LV && TR) ? SB : 1][RP];
    E kt[(LK && !TR) ? D : 1][FP];
    E vt[(LV && !TR) ? D : 1][FP];
    float eta[SB];
};

// Row fragment (rows = tokens of tile i, contraction over features 16r..16r+15):
// lane (m, g) gets X[16i + m][16r + 4g + j].
// column of the 4-column group at col in row row of a token-major tile
template <bool SW, bool PM = false> __device__ __forceinline__ int tcol(int row, int col)
{
    return SW ? swz(row, col) : PM ? pcol(col) : col;
}

template <typename E, int D, int ST>
__device__ __forceinline__ typename Frag<E>::type q_row(const SbTile<E, D, ST> &t, int i, int r, int m, int g)
{
    constexpr bool SW = SbTile<E, D, ST>::SW, PM = SbTile<E, D, ST>::PM;
    return load4<E>(&t.qs[16 * i + m][tcol<SW, PM>(16 * i + m, 16 * r + 4 * g)]);
}
template <typename E, int D, int ST>
__device__ __forceinline__ typename Frag<E>::type k_row(const SbTile<E, D, ST> &t, int i, int r, int m, int g)
{
    constexpr bool SW = SbTile<E, D, ST>::SW, PM = SbTile<E, D, ST>::PM;
    if constexpr (SbTile<E, D, ST>::TR) {
        return load4<E>(&t.ks[16 * i + m][tcol<SW, PM>(16 * i + m, 16 * r + 4 * g)]);
    } else {
        f32x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = t.kt[16 * r + 4 * g + j][16 * i + m];
        return x;
    }
}
// Token fragment (contraction over the tokens of tile i, features 16c..16c+15):
// lane (m, g) gets X[16i + 4g + j][16c + m].  As an A operand it is the
// transposed tile, as a B operand the tile itself, as an accumulator the C layout.
template <typename E, int D, int ST>
__device__ __forceinline__ typename Frag<E>::type k_tok(const SbTile<E, D, ST> &t, int i, int c, int m, int g)
{
    constexpr bool SW = SbTile<E, D, ST>::SW, PM = SbTile<E, D, ST>::PM;
    const int row = 16 * i + 4 * g + (m >> 2);
    if constexpr (SbTile<E, D, ST>::TR)
        return lds_read_tr(&t.ks[row][tcol<SW, PM>(row, 16 * c + 4 * (m & 3))]);
    else
        return load4<E>(&t.kt[16 * c + m][16 * i + 4 * g]);
}
template <typename E, int D, int ST>
__device__ __forceinline__ typename Frag<E>::type v_tok(const SbTile<E, D, ST> &t, int i, int c, int m, int g)
{
    constexpr bool SW = SbTile<E, D, ST>::SW, PM = SbTile<E, D, ST>::PM;
    const int row = 16 * i + 4 * g + (m >> 2);
    if constexpr (SbTile<E, D, ST>::TR)
        return lds_read_tr(&t.vs[row][tcol<SW, PM>(row, 16 * c + 4 * (m & 3))]);
    else
        return load4<E>(&t.vt[16 * c + m][16 * i + 4 * g]);
}

// Row fragments r and r + 1 (r even) of tile i: with the permuted layout one
// 16-byte read, otherwise two 8-byte ones.
template <typename E, int D, int ST>
__device__ __forceinline__ void q_row2(const SbTile<E, D, ST> &t, int i, int r, int m, int g,
                                       typename Frag<E>::type &a, typename Frag<E>::type &b)
{
    if constexpr (SbTile<E, D, ST>::PM) {
        const bf16x8 x = as_bf8x(&t.qs[16 * i + m][pcol(16 * r + 4 * g)]);
        a = __builtin_shufflevector(x, x, 0, 1, 2, 3);
        b = __builtin_shufflevector(x, x, 4, 5, 6, 7);
    } else {
        a = q_row(t, i, r, m, g);
        b = q_row(t, i, r + 1, m, g);
    }
}
template <typename E, int D, int ST>
__device__ __forceinline__ void k_row2(const SbTile<E, D, ST> &t, int i, int r, int m, int g,
                                       typename Frag<E>::type &a, typename Frag<E>::type &b)
{
    if constexpr (SbTile<E, D, ST>::PM) {
        const bf16x8 x = as_bf8x(&t.ks[16 * i + m][pcol(16 * r + 4 * g)]);
        a = __builtin_shufflevector(x, x, 0, 1, 2, 3);
        b = __builtin_shufflevector(x, x, 4, 5, 6, 7);
    } else {
        a = k_row(t, i, r, m, g);
        b = k_row(t, i, r + 1, m, g);
    }
}

// Transformed keys Kt = T K of one super-block, shared by the waves: each wave
// writes its column block (accumulator layout), every wave reads row
// fragments.  bf16: feature-major, 8-byte writes, transposing reads.
template <typename E, int D, bool SW = false> struct alignas(16) KtTile;
template <int D, bool SW> struct alignas(16) KtTile<__bf16, D, SW> {
    __bf16 fm[D][SW ? SB : SB + 8];
    __device__ __forceinline__ void put(int c, int i, f32x4 x, int m, int g)
    {
        const int row = 16 * c + m;
        store4<__bf16>(&fm[row][tcol<SW>(row, 16 * i + 4 * g)], to_bf16x4(x));
    }
    __device__ __forceinline__ bf16x4 row(int i, int r, int m, int g) const
    {
        const int rr = 16 * r + 4 * g + (m >> 2);
        return lds_read_tr(&fm[rr][tcol<SW>(rr, 16 * i + 4 * (m & 3))]);
    }
};
template <int D, bool SW> struct alignas(16) KtTile<float, D, SW> {
    float tm[SB][D + 4];
    __device__ __forceinline__ void put(int c, int i, f32x4 x, int m, int g)
    {
#pragma unroll
        for (int j = 0; j < 4; ++j) tm[16 * i + 4 * g + j][16 * c + m] = x[j];
    }
    __device__ __forceinline__ f32x4 row(int i, int r, int m, int g) const
    {
        return load4<float>(&tm[16 * i + m][16 * r + 4 * g]);
    }
};

// Cooperative global -> register -> LDS loader with a ring of PD register
// slots.  Every thread moves CPT 16-byte pieces of each staged tensor per
// super-block and one eta value, with buffer loads: the per-thread byte
// offset is fixed, the super-block's first token is the scalar offset, and the
// buffer's extent ends at the segment's last token, so rows past it read as
// zero in hardware.
template <typename E, int D, int ST, int PD, int NT> struct SbLoader {
    typedef SbTile<E, D, ST> Tile;
    static constexpr bool TR = Tile::TR, LQ = Tile::LQ, LK = Tile::LK, LV = Tile::LV;
    static constexpr bool LE = (ST & STAGE_E) != 0;
    static constexpr int PE = 16 / (int)sizeof(E);  // elements per piece
    static constexpr int PPR = D / PE;              // pieces per token row
    static constexpr int CPT = SB * PPR / NT;       // pieces per thread per tensor
    static_assert(CPT >= 1 && CPT * NT == SB * PPR, "loader shape");
    int row[CPT], col[CPT], voff[CPT];
    __amdgpu_buffer_rsrc_t rq, rk, rv, re;
    u32x4 vq[PD][CPT], vk[PD][CPT], vv[PD][CPT];
    float ve[PD];

    __device__ void init(int tid, const void *q, const void *k, const void *v, const float *eta, int h,
                         int T, int tend)
    {
        const size_t hoff = (size_t)h * T * D;
        const int bytes = tend * D * (int)sizeof(E);
        rq = __builtin_amdgcn_make_buffer_rsrc((void *)((const E *)q + (LQ ? hoff : 0)), (short)0,
                                               LQ ? bytes : 0, 0x00020000);
        rk = __builtin_amdgcn_make_buffer_rsrc((void *)((const E *)k + (LK ? hoff : 0)), (short)0,
                                               LK ? bytes : 0, 0x00020000);
        rv = __builtin_amdgcn_make_buffer_rsrc((void *)((const E *)v + (LV ? hoff : 0)), (short)0,
                                               LV ? bytes : 0, 0x00020000);
        re = __builtin_amdgcn_make_buffer_rsrc((void *)(eta + (LE ? (size_t)h * T : 0)), (short)0,
                                               LE ? tend * 4 : 0, 0x00020000);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int piece = tid + i * NT;
            row[i] = piece / PPR;
            col[i] = piece % PPR;
            voff[i] = (row[i] * D + PE * col[i]) * (int)sizeof(E);
        }
    }

    __device__ __forceinline__ void issue(int s, int tb0)
    {
        const int so = tb0 * D * (int)sizeof(E);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            if (LQ) vq[s][i] = __builtin_amdgcn_raw_buffer_load_b128(rq, voff[i], so, 0);
            if (LK) vk[s][i] = __builtin_amdgcn_raw_buffer_load_b128(rk, voff[i], so, 0);
            if (LV) vv[s][i] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[i], so, 0);
        }
        if (LE)
            ve[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  re, (int)(threadIdx.x & (SB - 1)) * 4, tb0 * 4, 0));
    }

    // A 16-byte piece (8 columns) in the swizzled layout: its chunk moves and
    // its two 4-column halves swap on row bit 3.
    static __device__ __forceinline__ u32x4 halves(u32x4 x, int r)
    {
        return ((r >> 3) & 1) ? u32x4{x[2], x[3], x[0], x[1]} : x;
    }
    // The two 8-byte halves of a piece, to their own places.
    static __device__ __forceinline__ void put_halves(E *a, E *b, u32x4 x)
    {
        typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
        *reinterpret_cast<u32x2v *>(a) = u32x2v{x[0], x[1]};
        *reinterpret_cast<u32x2v *>(b) = u32x2v{x[2], x[3]};
    }
    // Write slot s to LDS.
    __device__ __forceinline__ void commit(int s, Tile &tl)
    {
        constexpr bool SW = Tile::SW, PM = Tile::PM;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int r = row[i], c0 = PE * col[i];
            const int c = SW ? (swz(r, c0) & ~7) : c0;
            if constexpr (PM) {
                // the piece's two 4-column groups land at their own permuted places
                const int ca = pcol(c0), cb = pcol(c0 + 4);
                if (LQ) put_halves(&tl.qs[r][ca], &tl.qs[r][cb], vq[s][i]);
                if (LK) put_halves(&tl.ks[r][ca], &tl.ks[r][cb], vk[s][i]);
                if (LV) put_halves(&tl.vs[r][ca], &tl.vs[r][cb], vv[s][i]);
                continue;
            }
            if (LQ) *reinterpret_cast<u32x4 *>(&tl.qs[r][c]) = SW ? halves(vq[s][i], r) : vq[s][i];
            if (LK) {
                if constexpr (TR) {
                    *reinterpret_cast<u32x4 *>(&tl.ks[r][c]) = SW ? halves(vk[s][i], r) : vk[s][i];
                } else {
                    const f32x4 x = __builtin_bit_cast(f32x4, vk[s][i]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) tl.kt[c + j][r] = x[j];
                }
            }
            if (LV) {
                if constexpr (TR) {
                    *reinterpret_cast<u32x4 *>(&tl.vs[r][c]) = SW ? halves(vv[s][i], r) : vv[s][i];
                } else {
                    const f32x4 x = __builtin_bit_cast(f32x4, vv[s][i]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) tl.vt[c + j][r] = x[j];
                }
            }
        }
        if (LE) tl.eta[threadIdx.x & (SB - 1)] = ve[s];
    }
};

// Super-block schedule inside a segment (the segment starts on a chunk
// boundary).  b <= 64: super-block n covers floor(64/b) whole chunks.  b > 64:
// each chunk is cut into 64-token pieces plus a shorter last piece.
struct SbSched {
    int b, L, per;
    __device__ explicit SbSched(int chunk) : b(chunk)
    {
        if (chunk <= SB) {
            L = (SB / chunk) * chunk;
            per = 1;
        } else {
            L = SB;
            per = (chunk + SB - 1) / SB;
        }
    }
    __device__ int start(int n) const { return b <= SB ? n * L : (n / per) * b + SB * (n % per); }
    __device__ int len(int n) const { return b <= SB ? L : min(SB, b - SB * (n % per)); }
    __device__ int count(int rem) const
    {
        return b <= SB ? (rem + L - 1) / L : (rem / b) * per + (rem % b + SB - 1) / SB;
    }
    __device__ bool chunk_start(int n) const { return b <= SB || (n % per) == 0; }
};

// Drive the staged loop over the super-blocks of [t0, tend); `body(tile, n)`
// runs once per super-block.  The count is padded up to a multiple of PD so
// the ring runs without branches: padded super-blocks start past tend, read
// as zero (eta = 0) and change nothing; bodies mask their stores.
// NBUF = 2: the next tile is written while the current one is read (one
// barrier per super-block); NBUF = 1 (large fp32 tiles): write after a barrier.
template <typename E, int D, int ST, int PD, int NT, int NBUF, typename Body>
__device__ __forceinline__ void run_sb(SbTile<E, D, ST> *tiles, SbLoader<E, D, ST, PD, NT> &ld,
                                       const SbSched &sc, int t0, int tend, Body &&body)
{
    static_assert(NBUF == 1 || PD % 2 == 0, "double buffering needs an even ring");
    const int nsb = sc.count(tend - t0);
    const int ngroups = (nsb + PD - 1) / PD;
#pragma unroll
    for (int s = 0; s < PD; ++s) {
        ld.issue(s, t0 + sc.start(s));
        __builtin_amdgcn_sched_barrier(0);  // same load order as the loop body
    }
    ld.commit(0, tiles[0]);
    lds_barrier();
    for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
        for (int j = 0; j < PD; ++j) {
            const int n = gi * PD + j;
            ld.issue(j, t0 + sc.start(n + PD));
            if constexpr (NBUF == 2) {
                ld.commit((j + 1) % PD, tiles[(j + 1) & 1]);
                body(tiles[j & 1], n);
                lds_barrier();
            } else {
                body(tiles[0], n);
                lds_barrier();
                ld.commit((j + 1) % PD, tiles[0]);
                lds_barrier();
            }
        }
    }
}

// A state tile as MFMA operand.  bf16: hi = x truncated to bf16, lo =
// bf16(x - hi), so products with exact bf16 inputs keep ~16 mantissa bits of
// the state (the state sits near the identity, where a single bf16 would lose
// the update).  fp32: hi = x, lo unused.
template <typename E> struct SplitFrag {
    typedef typename Frag<E>::type F;
    static constexpr bool SPLIT = sizeof(E) == 2;
    F hi, lo;
    __device__ __forceinline__ void set(f32x4 x) { set_impl(x, *this); }
    template <typename S> static __device__ __forceinline__ void set_impl(f32x4 x, S &s);
};

template <> template <>
__device__ __forceinline__ void SplitFrag<__bf16>::set_impl(f32x4 x, SplitFrag<__bf16> &s)
{
    split_bf16x4(x, s.hi, s.lo);
}
template <> template <>
__device__ __forceinline__ void SplitFrag<float>::set_impl(f32x4 x, SplitFrag<float> &s)
{
    s.hi = x;
}

// acc += A(16 x D) * state(D x 16), state as split fragments (B side).
template <typename E, int ND>
__device__ __forceinline__ f32x4 mma_state_b(f32x4 acc, const typename Frag<E>::type *A,
                                             const SplitFrag<E> *S)
{
#pragma unroll
    for (int r = 0; r < ND; r += 2) acc = mma32(acc, A[r], A[r + 1], S[r].hi, S[r + 1].hi);
    if (SplitFrag<E>::SPLIT) {
#pragma unroll
        for (int r = 0; r < ND; r += 2) acc = mma32(acc, A[r], A[r + 1], S[r].lo, S[r + 1].lo);
    }
    return acc;
}
// acc += state^T(16 x D) * B(D x 16), state as split fragments (A side).
template <typename E, int ND>
__device__ __forceinline__ f32x4 mma_state_a(f32x4 acc, const SplitFrag<E> *S,
                                             const typename Frag<E>::type *B)
{
#pragma unroll
    for (int r = 0; r < ND; r += 2) acc = mma32(acc, S[r].hi, S[r + 1].hi, B[r], B[r + 1]);
    if (SplitFrag<E>::SPLIT) {
#pragma unroll
        for (int r = 0; r < ND; r += 2) acc = mma32(acc, S[r].lo, S[r + 1].lo, B[r], B[r + 1]);
    }
    return acc;
}

// acc += A(16 x D) * B(D x 16) with both operands as D/16 fragments.
template <typename F, int ND>
__device__ __forceinline__ f32x4 mma_b(f32x4 acc, const F *A, const F *B)
{
#pragma unroll
    for (int r = 0; r < ND; r += 2) acc = mma32(acc, A[r], A[r + 1], B[r], B[r + 1]);
    return acc;
}

// ---------------------------------------------------------------------------
// Tile-pair blocks of a super-block, computed once per workgroup and shared
// in fragment-native layout (lane l keeps lane l's fragment).
//   index 0..5  : -L_ij, (i, j) = (1,0) (2,0) (2,1) (3,0) (3,1) (3,2), as the
//                 A operand of L_ij X_j: lane (m, g) holds
//                 -(k_{16i+m} . k_{16j+4g+x}) eta_{16j+4g+x}, zero unless tile
//                 j lies in an earlier chunk than tile i;
//   index 6..15 : A_ij = (Q_i K_j^T * M * eta_j^T), j <= i, in the layout that
//                 is the B operand of U_j^T A_ij^T: lane (m, g) holds
//                 (q_{16i+m} . k_{16j+4g+x}) eta_{16j+4g+x}, causal (key <=
//                 query) on the diagonal.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int lblk(int i, int j) { return i * (i - 1) / 2 + j; }
__host__ __device__ constexpr int ablk(int i, int j) { return 6 + i * (i + 1) / 2 + j; }
__host__ __device__ constexpr int blk_i(int b) { return b < 6 ? (b < 1 ? 1 : b < 3 ? 2 : 3) : (b < 7 ? 0 : b < 9 ? 1 : b < 12 ? 2 : 3); }
__host__ __device__ constexpr int blk_j(int b) { return b < 6 ? b - lblk(blk_i(b), 0) : b - ablk(blk_i(b), 0); }

template <typename E, int D, int ST, int NW, bool WANT_L, bool WANT_A>
__device__ __forceinline__ void pair_blocks(const SbTile<E, D, ST> &t, typename Frag<E>::type (*gb)[64],
                                            const f32x4 *et, int chunk, int wave, int lane, int m, int g)
{
    typedef typename Frag<E>::type F;
    constexpr int ND = D / 16;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
        const bool isL = b < 6;
        if (isL && !WANT_L) continue;
        if (!isL && !WANT_A) continue;
        if (b % NW != wave) continue;
        const int i = blk_i(b), j = blk_j(b);
        if (isL && !((16 * j) / chunk < (16 * i) / chunk)) {
            gb[b][lane] = to_frag<E>(zero4());
            continue;
        }
        F Kj[ND], Xi[ND];
#pragma unroll
        for (int r = 0; r < ND; r += 2) {
            k_row2(t, j, r, m, g, Kj[r], Kj[r + 1]);
            if constexpr (SbTile<E, D, ST>::LQ) {
                if (isL)
                    k_row2(t, i, r, m, g, Xi[r], Xi[r + 1]);
                else
                    q_row2(t, i, r, m, g, Xi[r], Xi[r + 1]);
            } else {
                k_row2(t, i, r, m, g, Xi[r], Xi[r + 1]);
            }
        }
        f32x4 acc = mma_b<F, ND>(zero4(), Kj, Xi);
        if (isL) {
            acc = acc * (-et[j]);
        } else {
            acc = acc * et[j];
            if (i == j) {
#pragma unroll
                for (int x = 0; x < 4; ++x) acc[x] = (4 * g + x <= m) ? acc[x] : 0.f;
            }
        }
        gb[b][lane] = to_frag<E>(acc);
    }
}

// Kt = T K and Vt = T V for one column block c by block forward substitution:
// X~_i = X_i - sum_{j<i} L_ij X~_j (the -L_ij are the shared blocks 0..5).
template <typename E>
__device__ __forceinline__ void substitute(f32x4 *X, const typename Frag<E>::type *Ln)
{
    typedef typename Frag<E>::type F;
    const F x0 = to_frag<E>(X[0]);
    X[1] = mma32z(X[1], Ln[lblk(1, 0)], x0);
    const F x1 = to_frag<E>(X[1]);
    X[2] = mma32(X[2], Ln[lblk(2, 0)], Ln[lblk(2, 1)], x0, x1);
    const F x2 = to_frag<E>(X[2]);
    X[3] = mma32(X[3], Ln[lblk(3, 0)], Ln[lblk(3, 1)], x0, x1);
    X[3] = mma32z(X[3], Ln[lblk(3, 2)], x2);
}

// eta of the tokens a lane's accumulator rows cover, masked to the super-block.
template <typename E, int D, int ST>
__device__ __forceinline__ void load_eta(const SbTile<E, D, ST> &t, int len, int g, f32x4 *et)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) et[i] = *reinterpret_cast<const f32x4 *>(&t.eta[16 * i + 4 * g]);
    if (len < SB) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int x = 0; x < 4; ++x) et[i][x] = (16 * i + 4 * g + x < len) ? et[i][x] : 0.f;
    }
}

// ---------------------------------------------------------------------------
// summary: P_s (MSE) and B_s of a segment.  The state X = [P | B] starts at 0
// and follows the chunk rule with residual R - K X_c, R = [K | V] (MSE; A = I -
// P is the product of the chunk transitions) or R = V (inner product, where
// X_c does not enter).  Wave c owns column block c of P and of B.
// LT: b < 64 (transform by T); SNAP: b > 64 (chunk-start snapshots).
// ---------------------------------------------------------------------------
template <typename E, int D, bool MSE, bool LT, bool SNAP, int PD>
__global__ __launch_bounds__((D / 16) * 64) void lin_summary(LinParams p)
{
    typedef typename Frag<E>::type F;
    constexpr int ND = D / 16;
    constexpr int NT = ND * 64;
    constexpr int NBUF = sizeof(E) == 2 ? 2 : 1;
    constexpr int ST = STAGE_K | STAGE_V | STAGE_E | STAGE_PERM;
    __shared__ SbTile<E, D, ST> tiles[NBUF];
    __shared__ KtTile<E, LT ? D : 16> kts;
    __shared__ F gb[LT ? 16 : 1][64];
    const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
    const int c = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // column block
    // a head's segments on one XCD: the replay's chain then reads the
    // summaries from the L2 they were written to
    const int bid = xcd_block(blockIdx.x, gridDim.x);
    const int seg = bid % p.Ssum, h = bid / p.Ssum;
    const int T = p.Tkv;
    const int t0 = seg * p.seg_tokens;
    const int tend = min(T, t0 + p.seg_tokens);
    const SbSched sc(p.chunk);

    if (seg == 0 && p.wsW0) {
        // copy of w_init for the replay (w_final may alias w_init)
        const f32x4 *src = reinterpret_cast<const f32x4 *>(p.w_init + (size_t)h * D * D);
        f32x4 *dst = reinterpret_cast<f32x4 *>(p.wsW0 + (size_t)h * D * D);
        for (int i = threadIdx.x; i < D * D / 4; i += NT) dst[i] = src[i];
    }

    SbLoader<E, D, ST, PD, NT> ld;
    ld.init(threadIdx.x, nullptr, p.k, p.v, p.eta, h, T, tend);

    // X starts at 0 and stays moderate, so one bf16 rounding per element is
    // enough for the residual product.
    f32x4 Xp[ND], Xb[ND];
    F Xpr[ND], Xbr[ND], Xps[SNAP ? ND : 1], Xbs[SNAP ? ND : 1];
#pragma unroll
    for (int r = 0; r < ND; ++r) {
        Xp[r] = zero4();
        Xb[r] = zero4();
        Xpr[r] = to_frag<E>(zero4());
        Xbr[r] = Xpr[r];
    }

    run_sb<E, D, ST, PD, NT, NBUF>(tiles, ld, sc, t0, tend, [&](SbTile<E, D, ST> &t, int n) {
        f32x4 et[4];
        load_eta(t, sc.len(n), g, et);
        if (!MSE) {
            // B += K^T diag(eta) V
            F EV[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) EV[i] = to_frag<E>(frag_to_f32(v_tok(t, i, c, m, g)) * et[i]);
#pragma unroll
            for (int r = 0; r < ND; ++r)
#pragma unroll
                for (int i = 0; i < 4; i += 2)
                    Xb[r] = mma32(Xb[r], k_tok(t, i, r, m, g), k_tok(t, i + 1, r, m, g), EV[i], EV[i + 1]);
            return;
        }
        if (SNAP && sc.chunk_start(n)) {
#pragma unroll
            for (int r = 0; r < ND; ++r) {
                Xps[r] = Xpr[r];
                Xbs[r] = Xbr[r];
            }
        }
        f32x4 Kc[4], Vc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Kc[i] = frag_to_f32(k_tok(t, i, c, m, g));
            Vc[i] = frag_to_f32(v_tok(t, i, c, m, g));
        }
        if constexpr (LT) {
            pair_blocks<E, D, ST, ND, true, false>(t, gb, et, p.chunk, c, lane, m, g);
            lds_barrier();
            F Ln[6];
#pragma unroll
            for (int x = 0; x < 6; ++x) Ln[x] = gb[x][lane];
            substitute<E>(Kc, Ln);
            substitute<E>(Vc, Ln);
#pragma unroll
            for (int i = 0; i < 4; ++i) kts.put(c, i, Kc[i], m, g);
            lds_barrier();
        }
        // U = [Kt | Vt] - Kt X_base, then X += K^T diag(eta) U
        F EUp[4], EUb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            F Ka[ND];
#pragma unroll
            for (int r = 0; r < ND; r += 2) {
                if constexpr (LT) {
                    Ka[r] = kts.row(i, r, m, g);
                    Ka[r + 1] = kts.row(i, r + 1, m, g);
                } else {
                    k_row2(t, i, r, m, g, Ka[r], Ka[r + 1]);
                }
            }
            const f32x4 Up = Kc[i] - mma_b<F, ND>(zero4(), Ka, SNAP ? Xps : Xpr);
            const f32x4 Ub = Vc[i] - mma_b<F, ND>(zero4(), Ka, SNAP ? Xbs : Xbr);
            EUp[i] = to_frag<E>(Up * et[i]);
            EUb[i] = to_frag<E>(Ub * et[i]);
        }
#pragma unroll
        for (int r = 0; r < ND; ++r) {
            const F k0 = k_tok(t, 0, r, m, g), k1 = k_tok(t, 1, r, m, g);
            const F k2 = k_tok(t, 2, r, m, g), k3 = k_tok(t, 3, r, m, g);
            Xp[r] = mma32(Xp[r], k0, k1, EUp[0], EUp[1]);
            Xp[r] = mma32(Xp[r], k2, k3, EUp[2], EUp[3]);
            Xb[r] = mma32(Xb[r], k0, k1, EUb[0], EUb[1]);
            Xb[r] = mma32(Xb[r], k2, k3, EUb[2], EUb[3]);
            Xpr[r] = to_frag<E>(Xp[r]);
            Xbr[r] = to_frag<E>(Xb[r]);
        }
    });

    const size_t base = ((size_t)h * p.Ssum + seg) * D * D;
    if (MSE) {
        E *dst = (E *)p.wsP + base;
#pragma unroll
        for (int r = 0; r < ND; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[(size_t)(16 * r + 4 * g + j) * D + 16 * c + m] = (E)Xp[r][j];
    }
    f32x4 *dst = reinterpret_cast<f32x4 *>(p.wsB + base) + c * ND * 64;
#pragma unroll
    for (int r = 0; r < ND; ++r) dst[r * 64 + lane] = Xb[r];
}

// ---------------------------------------------------------------------------
// Segment-start chain.  R holds column block c of a state (accumulator
// layout); apply the affine maps of segments 0..nsteps-1 of head h to it:
// R <- R - P_s R + B_s.  P_s (D x D row-major, element type) is staged
// through LDS by the whole workgroup, two steps ahead in registers; each wave
// reads the P rows it needs as A fragments.  B_s is stored in accumulator
// order (column block, row block, lane, 4 rows), so a wave's column block is
// one 16-byte read per row block.  NPB = 2: double-buffered LDS (one barrier a
// step).
// ---------------------------------------------------------------------------
template <typename E, int D> struct alignas(16) PStage {
    E m[D][D + (sizeof(E) == 2 ? 8 : 4)];
};

template <typename E, int D, int NT> struct PLoader {
    static constexpr int PE = 16 / (int)sizeof(E);
    static constexpr int PPR = D / PE;
    static constexpr int CPT = D * PPR / NT;
    static_assert(CPT >= 1 && CPT * NT == D * PPR, "P loader shape");
    int row[CPT], col[CPT];
    u32x4 v[2][CPT];
    const E *base;
    __device__ void init(int tid, const E *b)
    {
        base = b;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int piece = tid + i * NT;
            row[i] = piece / PPR;
            col[i] = piece % PPR;
        }
    }
    __device__ __forceinline__ void issue(int slot, int step)
    {
        const E *P = base + (size_t)step * D * D;
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            v[slot][i] = *reinterpret_cast<const u32x4 *>(P + (size_t)row[i] * D + PE * col[i]);
    }
    __device__ __forceinline__ void commit(int slot, PStage<E, D> &st)
    {
#pragma unroll
        for (int i = 0; i < CPT; ++i) *reinterpret_cast<u32x4 *>(&st.m[row[i]][PE * col[i]]) = v[slot][i];
    }
};

template <typename E, int D, bool MSE, int NT, int NPB>
__device__ __forceinline__ void chain_maps(f32x4 *R, const LinParams &p, int h, int nsteps,
                                           PStage<E, D> *pst, int c, int m, int g)
{
    typedef typename Frag<E>::type F;
    constexpr int ND = D / 16;
    const size_t hb = (size_t)h * p.Ssum * D * D;
    const float *Bh = p.wsB + hb;
    f32x4 Bt[2][ND];
    const int lane = 16 * g + m;
    auto loadB = [&](int slot, int step) {
        const f32x4 *Bs = reinterpret_cast<const f32x4 *>(Bh + (size_t)step * D * D) + c * ND * 64;
#pragma unroll
        for (int r = 0; r < ND; ++r) Bt[slot][r] = Bs[r * 64 + lane];
    };
    const int last = nsteps - 1;
    PLoader<E, D, NT> pl;
    if (MSE) {
        pl.init(threadIdx.x, (const E *)p.wsP + hb);
        pl.issue(0, 0);
        pl.issue(1, min(1, last));
    }
    loadB(0, 0);
    loadB(1, min(1, last));
    if (MSE) {
        pl.commit(0, pst[0]);
        pl.issue(0, min(2, last));
        lds_barrier();
    }
    // Steps run in pairs so ring slots are compile-time; a padded last step
    // changes nothing.  Step s: register slot s%2 holds B_s and, after the
    // commit of step s-1, the P of step s+2; LDS buffer s%NPB holds P_s.
    const int npairs = (nsteps + 1) / 2;
    for (int pi = 0; pi < npairs; ++pi) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int s = 2 * pi + j;
            if (s < nsteps) {
                if (MSE) {
                    SplitFrag<E> Ws[ND];
#pragma unroll
                    for (int r = 0; r < ND; ++r) Ws[r].set(R[r]);
                    const PStage<E, D> &P = pst[NPB == 2 ? j : 0];
#pragma unroll
                    for (int r = 0; r < ND; ++r) {
                        F PA[ND];
#pragma unroll
                        for (int q = 0; q < ND; ++q) PA[q] = load4<E>(&P.m[16 * r + m][16 * q + 4 * g]);
                        R[r] = R[r] + Bt[j][r] - mma_state_b<E, ND>(zero4(), PA, Ws);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < ND; ++r) R[r] = R[r] + Bt[j][r];
                }
            }
            loadB(j, min(s + 2, last));
            if (MSE) {
                if (NPB == 1) lds_barrier();
                pl.commit(1 - j, pst[NPB == 2 ? 1 - j : 0]);
                pl.issue(1 - j, min(s + 3, last));
                lds_barrier();
            }
        }
    }
}

// ---------------------------------------------------------------------------
// final state (non-causal): W_final = the maps of all segments applied to
// w_init, one workgroup per head (wave c owns column block c).  Reads all of
// w_init before writing w_final (they may alias).
// ---------------------------------------------------------------------------
template <typename E, int D, bool MSE>
__global__ __launch_bounds__((D / 16) * 64) void lin_final(LinParams p)
{
    constexpr int ND = D / 16;
    constexpr int NT = ND * 64;
    constexpr int NPB = (sizeof(E) == 4 && D == 128) ? 1 : 2;
    __shared__ PStage<E, D> pst[MSE ? NPB : 1];
    const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
    const int c = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int h = blockIdx.x;
    (void)lane;
    const float *w0 = p.w_init + (size_t)h * D * D;
    f32x4 R[ND];
#pragma unroll
    for (int r = 0; r < ND; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) R[r][j] = w0[(size_t)(16 * r + 4 * g + j) * D + 16 * c + m];
    chain_maps<E, D, MSE, NT, NPB>(R, p, h, p.Ssum, pst, c, m, g);
    float *wf = p.w_final + (size_t)h * D * D;
#pragma unroll
    for (int r = 0; r < ND; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) wf[(size_t)(16 * r + 4 * g + j) * D + 16 * c + m] = R[r][j];
}

// ---------------------------------------------------------------------------
// replay (causal): outputs of one segment.  The workgroup first builds its
// start state from w_init and the summaries of the segments before it, then
// walks its super-blocks.  Wave c owns column block c of the running state R
// (fp32 accumulators, re-split into hi/lo operands after every update) and of
// the outputs.
// ---------------------------------------------------------------------------
template <typename E, int D, bool MSE, bool LT, bool SNAP, int PD>
__global__ __launch_bounds__((D / 16) * 64) void lin_replay(LinParams p)
{
    typedef typename Frag<E>::type F;
    constexpr int ND = D / 16;
    constexpr int NT = ND * 64;
    constexpr int NBUF = sizeof(E) == 2 ? 2 : 1;
    constexpr int ST = STAGE_Q | STAGE_K | STAGE_V | STAGE_E | STAGE_PERM;
    constexpr int NPB = (sizeof(E) == 4 && D == 128) ? 1 : 2;
    // The super-block tiles and the staged P of the segment-start chain are
    // never live at the same time.
    __shared__ union {
        SbTile<E, D, ST> tiles[NBUF];
        PStage<E, D> pst[MSE ? NPB : 1];
    } lds;
    SbTile<E, D, ST> *tiles = lds.tiles;
    __shared__ KtTile<E, LT ? D : 16> kts;
    __shared__ F gb[16][64];
    const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
    const int c = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // column block
    const int bid = xcd_block(blockIdx.x, gridDim.x);  // a head's segments on one XCD
    const int seg = bid % p.S, h = bid / p.S;
    const int T = p.Tkv;
    const int t0 = seg * p.seg_tokens;
    const int tend = min(T, t0 + p.seg_tokens);
    const SbSched sc(p.chunk);

    // w_init itself, or the summary's copy of it when w_final is the same
    // buffer (the last segment writes it while earlier ones may still read).
    const float *ws = (p.wsW0 ? p.wsW0 : p.w_init) + (size_t)h * D * D;
    // Only R (and, for chunks longer than a super-block, the chunk-start
    // snapshot Ss) is carried from one super-block to the next; the bf16
    // split of R is formed where a super-block starts, so it is not live
    // across the tile loads.
    f32x4 R[ND];
    SplitFrag<E> Ss[SNAP ? ND : 1];
#pragma unroll
    for (int r = 0; r < ND; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j) R[r][j] = ws[(size_t)(16 * r + 4 * g + j) * D + 16 * c + m];
    if (seg > 0) chain_maps<E, D, MSE, NT, NPB>(R, p, h, seg, lds.pst, c, m, g);

    SbLoader<E, D, ST, PD, NT> ld;
    ld.init(threadIdx.x, p.q, p.k, p.v, p.eta, h, T, tend);
    E *out_h = (E *)p.out + (size_t)h * T * D;

    run_sb<E, D, ST, PD, NT, NBUF>(tiles, ld, sc, t0, tend, [&](SbTile<E, D, ST> &t, int n) {
        const int s = t0 + sc.start(n), len = sc.len(n);
        const int lim = min(tend, s + len);
        f32x4 et[4];
        load_eta(t, len, g, et);
        SplitFrag<E> Rs[ND];
#pragma unroll
        for (int r = 0; r < ND; ++r) Rs[r].set(R[r]);
        if (SNAP && sc.chunk_start(n)) {
#pragma unroll
            for (int r = 0; r < ND; ++r) Ss[r] = Rs[r];
        }
        pair_blocks<E, D, ST, ND, LT, true>(t, gb, et, p.chunk, c, lane, m, g);
        lds_barrier();
        // residuals U of the four tiles (column block c)
        f32x4 U[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) U[i] = frag_to_f32(v_tok(t, i, c, m, g));
        if (MSE) {
            if constexpr (LT) {
                F Ln[6];
#pragma unroll
                for (int x = 0; x < 6; ++x) Ln[x] = gb[x][lane];
                f32x4 Kc[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) Kc[i] = frag_to_f32(k_tok(t, i, c, m, g));
                substitute<E>(Kc, Ln);
                substitute<E>(U, Ln);
#pragma unroll
                for (int i = 0; i < 4; ++i) kts.put(c, i, Kc[i], m, g);
                lds_barrier();
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                F Ka[ND];
#pragma unroll
                for (int r = 0; r < ND; r += 2) {
                    if constexpr (LT) {
                        Ka[r] = kts.row(i, r, m, g);
                        Ka[r + 1] = kts.row(i, r + 1, m, g);
                    } else {
                        k_row2(t, i, r, m, g, Ka[r], Ka[r + 1]);
                    }
                }
                U[i] = U[i] - mma_state_b<E, ND>(zero4(), Ka, SNAP ? Ss : Rs);
            }
        }
        F Uf[4], EU[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Uf[i] = to_frag<E>(U[i]);
            EU[i] = to_frag<E>(U[i] * et[i]);
        }
        // O^T_i = R^T Q_i^T + sum_{j<=i} U_j^T A_ij^T (transposed so each lane
        // stores four consecutive columns of one token); key tiles are paired
        // into 32-deep products.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (16 * i >= len) break;
            F Qa[ND];
#pragma unroll
            for (int r = 0; r < ND; r += 2) q_row2(t, i, r, m, g, Qa[r], Qa[r + 1]);
            f32x4 O = mma_state_a<E, ND>(zero4(), Rs, Qa);
#pragma unroll
            for (int j = 0; j <= i; j += 2) {
                if (j + 1 <= i)
                    O = mma32(O, Uf[j], Uf[j + 1], gb[ablk(i, j)][lane], gb[ablk(i, j + 1)][lane]);
                else
                    O = mma32z(O, Uf[j], gb[ablk(i, j)][lane]);
            }
            const int tk = s + 16 * i + m;
            if (tk < lim) store4<E>(out_h + (size_t)tk * D + 16 * c + 4 * g, out4<E>(O));
        }
        // R += K^T diag(eta) U
#pragma unroll
        for (int r = 0; r < ND; ++r) {
            R[r] = mma32(R[r], k_tok(t, 0, r, m, g), k_tok(t, 1, r, m, g), EU[0], EU[1]);
            R[r] = mma32(R[r], k_tok(t, 2, r, m, g), k_tok(t, 3, r, m, g), EU[2], EU[3]);
        }
    });

    if (seg == p.S - 1) {
        float *wf = p.w_final + (size_t)h * D * D;
#pragma unroll
        for (int r = 0; r < ND; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) wf[(size_t)(16 * r + 4 * g + j) * D + 16 * c + m] = R[r][j];
    }
}

// ---------------------------------------------------------------------------
// Producer/consumer kernels (bf16, d = 64, b <= 64).  Eight waves per
// workgroup.  Waves 0-3 (consumers) own column block c of the running state
// (replay) or of [P | B] (summary) exactly as above.  Waves 4-7 (producers)
// move the token tiles from HBM into a three-deep LDS ring and compute, one
// super-block ahead, everything that does not depend on the state: the
// transformed keys and values (T K, T V, each producer one column block) and,
// for the replay, the query-key blocks A_ij.  Each SIMD then runs one wave of
// each kind, so the serial state chain issues beside the independent work
// instead of after it.  One workgroup barrier per super-block.
// ---------------------------------------------------------------------------
constexpr int PC_NR = 3;  // LDS ring of raw super-block tiles
// Producer waves 2p and 2p + 1 (p = k >> 1) load super-blocks n = p (mod 2),
// half the rows each, and producer wave k alone stages chain steps
// s = k (mod 4): when a wave commits one, the only loads it has in flight are
// that item's, issued two (super-blocks) or four (chain steps) iterations
// earlier, so the wait before the commit (which the compiler places
// conservatively inside loops) costs nothing.
template <int ST> using PcLoader = SbLoader<__bf16, 64, ST, 1, 128>;

// Producer results for one super-block (replay).
template <bool LT> struct alignas(16) PcRepDer {
    KtTile<__bf16, LT ? 64 : 16, true> kt;  // T K, feature-major (swizzled)
    bf16x4 ab[10][64];                // A_ij (pair-block indices 6..15)
};
// Producer results for one super-block (summary, b < 64 only).
template <bool LT> struct alignas(16) PcSumDer {
    KtTile<__bf16, LT ? 64 : 16, true> kt;
    f32x4 kc[LT ? 4 : 1][4][64];  // T K by column block, accumulator order
};

// Tokens per super-block for chunk CH <= 64, and whether T is needed: only
// when the super-block holds several chunks (b = 48 holds one chunk of three
// tiles; its fourth tile is masked).
template <int CH> struct PcCfg {
    static constexpr int L = (SB / CH) * CH;
    static constexpr bool MULTI = (SB / CH) > 1;
};

template <int ST>
__device__ __forceinline__ void pc_krows(const SbTile<__bf16, 64, ST> &t, bf16x4 (&Kr)[4][4], int m, int g)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) Kr[i][r] = k_row(t, i, r, m, g);
}

// Producer wave owning A_ij block b (6..15).  Blocks of one row block i go
// to one wave where possible, so its query rows are read once; with the six
// shared L_ij blocks of b = 16 (waves 0 and 1 compute two of them, waves 2
// and 3 one) every wave ends up with four blocks, otherwise with three or two.
template <bool ALL_L> __host__ __device__ constexpr int a_owner(int b)
{
    if (ALL_L) return (b == 7 || b == 8) ? 0 : (b == 6 || b == 15) ? 1 : (b >= 12) ? 2 : 3;
    return (b >= 12 && b <= 14) ? 0 : (b >= 9 && b <= 11) ? 1 : (b == 6 || b == 15) ? 2 : 3;
}

template <int PC, bool ALL_L, int ST, typename Der>
__device__ __forceinline__ void pc_ablocks(const SbTile<__bf16, 64, ST> &t, const bf16x4 (&Kr)[4][4],
                                           const f32x4 *et, Der &dv, int lane, int m, int g)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        bool any = false;
#pragma unroll
        for (int j = 0; j <= i; ++j) any |= a_owner<ALL_L>(ablk(i, j)) == PC;
        if (!any) continue;
        bf16x4 Qi[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) Qi[r] = q_row(t, i, r, m, g);
#pragma unroll
        for (int j = 0; j <= i; ++j) {
            const int b = ablk(i, j);
            if (a_owner<ALL_L>(b) != PC) continue;
            f32x4 acc = mma_b<bf16x4, 4>(zero4(), Kr[j], Qi) * et[j];
            if (i == j) {
#pragma unroll
                for (int x = 0; x < 4; ++x) acc[x] = (4 * g + x <= m) ? acc[x] : 0.f;
            }
            dv.ab[b - 6][lane] = to_bf16x4(acc);
        }
    }
}

// -L_ij blocks (b < 64 with several chunks per super-block).  Every producer
// wave computes all nonzero blocks in registers for its own substitution (a
// few extra MFMAs instead of an exchange through LDS and a wait on the other
// producers), and wave K writes blocks K and K + 4 to LDS for the consumers,
// which apply them to V (T V).  Two buffers by super-block parity: the
// consumers read the blocks of their super-block while the producers write
// the next one's.
struct alignas(16) PcLShare {
    bf16x4 blk[2][6][64];
};

template <int CH> __host__ __device__ constexpr bool l_nonzero(int b)
{
    return (16 * blk_j(b)) / CH < (16 * blk_i(b)) / CH;
}

template <int K, int CH>
__device__ __forceinline__ void pc_lblocks(const bf16x4 (&Kr)[4][4], const f32x4 *et, PcLShare &ls, int n,
                                           bf16x4 *Ln, int lane)
{
#pragma unroll
    for (int b = 0; b < 6; ++b) {
        if (!l_nonzero<CH>(b)) continue;
        const int i = blk_i(b), j = blk_j(b);
        Ln[b] = to_bf16x4(mma_b<bf16x4, 4>(zero4(), Kr[j], Kr[i]) * (-et[j]));
        if ((b & 3) == K) ls.blk[n & 1][b][lane] = Ln[b];
    }
}

template <int CH>
__device__ __forceinline__ void pc_lshare_read(const PcLShare &ls, int n, bf16x4 *Ln, int lane)
{
#pragma unroll
    for (int b = 0; b < 6; ++b)
        if (l_nonzero<CH>(b)) Ln[b] = ls.blk[n & 1][b][lane];
}

// Block forward substitution with the blocks that are zero for CH skipped.
template <int CH>
__device__ __forceinline__ void substitute_ch(f32x4 *X, const bf16x4 *Ln)
{
    static_assert(l_nonzero<CH>(1) && l_nonzero<CH>(2) && l_nonzero<CH>(3) && l_nonzero<CH>(4), "chunk shape");
    const bf16x4 x0 = to_bf16x4(X[0]);
    if constexpr (l_nonzero<CH>(0)) X[1] = mma32z(X[1], Ln[lblk(1, 0)], x0);
    const bf16x4 x1 = to_bf16x4(X[1]);
    X[2] = mma32(X[2], Ln[lblk(2, 0)], Ln[lblk(2, 1)], x0, x1);
    const bf16x4 x2 = to_bf16x4(X[2]);
    X[3] = mma32(X[3], Ln[lblk(3, 0)], Ln[lblk(3, 1)], x0, x1);
    if constexpr (l_nonzero<CH>(5)) X[3] = mma32z(X[3], Ln[lblk(3, 2)], x2);
}

// Producer wave K's share of one super-block (replay): its A_ij blocks and,
// for b < 64 with several chunks, its column block of T K.
template <int K, bool LT, int CH, int ST, typename Der>
__device__ __forceinline__ void pc_derive_rep(const SbTile<__bf16, 64, ST> &t, Der &dv, PcLShare &ls, int n,
                                              int len, int lane, int m, int g)
{
    f32x4 et[4];
    load_eta(t, len, g, et);
    bf16x4 Kr[4][4];
    pc_krows(t, Kr, m, g);
    f32x4 Kc[4];
    bf16x4 Ln[6];
    if constexpr (LT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) Kc[i] = to_f32x4(k_tok(t, i, K, m, g));
        pc_lblocks<K, CH>(Kr, et, ls, n, Ln, lane);
    }
    pc_ablocks<K, LT && l_nonzero<CH>(0) && l_nonzero<CH>(5)>(t, Kr, et, dv, lane, m, g);
    if constexpr (LT) {
        substitute_ch<CH>(Kc, Ln);
#pragma unroll
        for (int i = 0; i < 4; ++i) dv.kt.put(K, i, Kc[i], m, g);
    }
}

// Producer wave K's share of one super-block (summary, b < 64 with several
// chunks): its column block of T K (bf16 feature-major and fp32).
template <int K, int CH, int ST, typename Der>
__device__ __forceinline__ void pc_derive_sum(const SbTile<__bf16, 64, ST> &t, Der &dv, PcLShare &ls, int n,
                                              int len, int lane, int m, int g)
{
    f32x4 et[4];
    load_eta(t, len, g, et);
    bf16x4 Kr[4][4];
    pc_krows(t, Kr, m, g);
    f32x4 Kc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) Kc[i] = to_f32x4(k_tok(t, i, K, m, g));
    bf16x4 Ln[6];
    pc_lblocks<K, CH>(Kr, et, ls, n, Ln, lane);
    substitute_ch<CH>(Kc, Ln);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        dv.kt.put(K, i, Kc[i], m, g);
        dv.kc[K][i][lane] = Kc[i];
    }
}

// Segment-start chain for consumer wave c, reading the summaries from global
// memory two steps ahead (no LDS, no barrier): R <- R - P_s R + B_s.
template <bool MSE, typename Step>
__device__ __forceinline__ void pc_chain(f32x4 (&R)[4], const LinParams &p, int h, int nsteps, int c, int lane,
                                         int m, int g, Step &&step)
{
    const size_t hb = (size_t)h * p.Ssum * 64 * 64;
    const __bf16 *Ph = (const __bf16 *)p.wsP + hb + m * 64 + 4 * g;
    const f32x4 *Bh = reinterpret_cast<const f32x4 *>(p.wsB + hb) + c * 4 * 64 + lane;
    bf16x4 PA[2][4][4];
    f32x4 Bt[2][4];
    auto load = [&](int slot, int step) {
        if (MSE) {
            const __bf16 *P = Ph + (size_t)step * 64 * 64;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int q = 0; q < 4; ++q) PA[slot][r][q] = load4<__bf16>(P + 16 * r * 64 + 16 * q);
        }
        const f32x4 *B = Bh + (size_t)step * 1024;
#pragma unroll
        for (int r = 0; r < 4; ++r) Bt[slot][r] = B[r * 64];
    };
    const int last = nsteps - 1;
    load(0, 0);
    load(1, min(1, last));
    for (int s0 = 0; s0 < nsteps; s0 += 2) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int s = s0 + j;
            if (s >= nsteps) break;
            if (MSE) {
                SplitFrag<__bf16> Ws[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) Ws[r].set(R[r]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    R[r] = R[r] + Bt[j][r] - mma_state_b<__bf16, 4>(zero4(), PA[j][r], Ws);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) R[r] = R[r] + Bt[j][r];
            }
            step(s);
            load(j, min(s + 2, last));
        }
    }
}

// Segment-start chain staged through LDS (MSE): producer wave k loads P_s
// (row-major) and B_s (accumulator order) of the steps s = k (mod 4), four
// steps ahead in registers, and commits each into a four-entry LDS ring as
// soon as the consumers are done with that entry's previous step; the
// consumers apply R <- R - P_s R + B_s.  The two sides meet through LDS
// counters, not workgroup barriers: ready[e] holds 1 + the step last
// committed into entry e, done[e] counts the consumer waves' reads of that
// entry.  Entry e only ever holds the steps s = e (mod 4), so the commit of
// step s waits for 4 * (s / 4) reads of its entry, which are the reads of
// the steps before it in that entry; those steps were fed by the same wave's
// earlier commits, and a consumer step waits only on its own commit, so
// every wait ends.
struct alignas(16) PcChainStage {
    __bf16 P[4][64][64];  // swizzled rows
    f32x4 B[4][4][4][64];
    unsigned ready[4];
    unsigned done[4];
};

__device__ __forceinline__ void pc_chain_init(PcChainStage &cs)
{
    if (threadIdx.x < 4) {
        cs.ready[threadIdx.x] = 0u;
        cs.done[threadIdx.x] = 0u;
    }
}

template <typename Mid>
__device__ __forceinline__ void pc_chain_stage(const LinParams &p, int h, int nsteps, PcChainStage &cs, int k,
                                               int lane, Mid &&mid)
{
    const size_t hb = (size_t)h * p.Ssum * 64 * 64;
    const __bf16 *Ph = (const __bf16 *)p.wsP + hb;
    const f32x4 *Bh = reinterpret_cast<const f32x4 *>(p.wsB + hb);
    u32x4 vp[8];
    f32x4 vb[16];
    auto issue = [&](int step) {
        const __bf16 *P = Ph + (size_t)step * 64 * 64;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int piece = lane + 64 * i;
            vp[i] = *reinterpret_cast<const u32x4 *>(P + (piece >> 3) * 64 + (piece & 7) * 8);
        }
        const f32x4 *B = Bh + (size_t)step * 1024;
#pragma unroll
        for (int i = 0; i < 16; ++i) vb[i] = B[lane + 64 * i];
    };
    auto commit = [&](int e) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int piece = lane + 64 * i, r = piece >> 3;
            const u32x4 x = vp[i];
            *reinterpret_cast<u32x4 *>(&cs.P[e][r][swz(r, (piece & 7) * 8) & ~7]) =
                ((r >> 3) & 1) ? u32x4{x[2], x[3], x[0], x[1]} : x;
        }
        f32x4 *Bd = &cs.B[e][0][0][0];
#pragma unroll
        for (int i = 0; i < 16; ++i) Bd[lane + 64 * i] = vb[i];
    };
    lds_barrier();  // counters initialised
    // mid() (the wave's first super-block load) follows the wave's last chain
    // commit: the chain's loads are not queued behind super-block loads, the
    // wave has no chain wait left that would cover it, and the super-blocks
    // are requested during the chain's last steps, when they are next needed
    if (k < nsteps)
        issue(k);
    else
        mid();
    for (int s = k; s < nsteps; s += 4) {
        // entry s % 4 is free once all four consumers are done with step s - 4
        if (s >= 4)
            while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&cs.done[s & 3], __ATOMIC_RELAXED,
                                                                    __HIP_MEMORY_SCOPE_WORKGROUP)) <
                   4u * (unsigned)(s >> 2))
                __builtin_amdgcn_s_sleep(1);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        commit(s & 3);
        if (lane == 0)
            __hip_atomic_store(&cs.ready[s & 3], (unsigned)(s + 1), __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (s + 4 < nsteps)
            issue(s + 4);
        else
            mid();
    }
}

template <typename Step>
__device__ __forceinline__ void pc_chain_lds(f32x4 (&R)[4], int nsteps, PcChainStage &cs, int c, int lane,
                                             int m, int g, Step &&step)
{
    lds_barrier();  // counters initialised
    for (int s = 0; s < nsteps; ++s) {
        const int e = s & 3;
        while (__builtin_amdgcn_readfirstlane(
                   __hip_atomic_load(&cs.ready[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) !=
               (unsigned)(s + 1))
            __builtin_amdgcn_s_sleep(1);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // the four row blocks side by side: consecutive MFMAs are independent
        bf16x4 PA[4][4];
        f32x4 Bs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int q = 0; q < 4; ++q) PA[r][q] = load4<__bf16>(&cs.P[e][16 * r + m][swz(16 * r + m, 16 * q + 4 * g)]);
            Bs[r] = cs.B[e][c][r][lane];
        }
        SplitFrag<__bf16> Ws[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) Ws[r].set(R[r]);
        f32x4 PR[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int q = 0; q < 4; q += 2)
#pragma unroll
            for (int r = 0; r < 4; ++r) PR[r] = mma32(PR[r], PA[r][q], PA[r][q + 1], Ws[q].hi, Ws[q + 1].hi);
#pragma unroll
        for (int q = 0; q < 4; q += 2)
#pragma unroll
            for (int r = 0; r < 4; ++r) PR[r] = mma32(PR[r], PA[r][q], PA[r][q + 1], Ws[q].lo, Ws[q + 1].lo);
        // this wave's reads of entry e are complete: release it
        if (lane == 0) __hip_atomic_fetch_add(&cs.done[e], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int r = 0; r < 4; ++r) R[r] = R[r] + Bs[r] - PR[r];
        step(s);
    }
}

// Producer pair p commits super-block p before the walk; the loads of 2 and
// 3 start with the walk (pc_walk), so that the first two are not queued
// behind them.
template <int ST, int L>
__device__ __forceinline__ void pc_first_commit(SbTile<__bf16, 64, ST> *raw, PcLoader<ST> &ld, int k)
{
    ld.commit(0, raw[k >> 1]);
}

// Main walk: iteration n, consumers run super-block n, producers prepare n + 1
// and producer pair (n + 2) mod 2 commits super-block n + 2 into the ring and
// loads n + 4.  The caller has committed super-blocks 0 and 1 and made them
// visible with a barrier.  The two roles run separate loops with the same
// barrier count, so neither keeps the other's registers.
template <int ST, int L, typename Cons, typename Prod>
__device__ __forceinline__ void pc_walk(SbTile<__bf16, 64, ST> *raw, PcLoader<ST> &ld, bool producer, int k,
                                        int t0, int nsb, Cons &&cons, Prod &&prod)
{
    const int ngroups = (nsb + PC_NR - 1) / PC_NR;
    if (producer) {
        ld.issue(0, t0 + ((k >> 1) + 2) * L);
        if (nsb > 0) prod(raw[0], 0);
        lds_barrier();
        for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
            for (int j = 0; j < PC_NR; ++j) {
                const int n = PC_NR * gi + j;
                if (n >= nsb) break;  // uniform: every wave leaves at the same n
                if (n + 1 < nsb) prod(raw[(j + 1) % PC_NR], n + 1);
                if ((n & 1) == (k >> 1)) {
                    ld.commit(0, raw[(j + 2) % PC_NR]);
                    ld.issue(0, t0 + (n + 4) * L);
                }
                lds_barrier();
            }
        }
    } else {
        lds_barrier();
        for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
            for (int j = 0; j < PC_NR; ++j) {
                const int n = PC_NR * gi + j;
                if (n >= nsb) break;
                cons(raw[j], n);
                lds_barrier();
            }
        }
    }
}

template <bool MSE, int CH>
__global__ __launch_bounds__(512) void lin_summary_pc(LinParams p)
{
    typedef __bf16 E;
    typedef bf16x4 F;
    constexpr int D = 64, ND = 4, L = PcCfg<CH>::L;
    constexpr bool LT = MSE && PcCfg<CH>::MULTI;
    constexpr int ST = STAGE_K | STAGE_V | STAGE_E | STAGE_SWZ;
    __shared__ SbTile<E, D, ST> raw[PC_NR];
    __shared__ PcSumDer<LT> der[LT ? 2 : 1];
    __shared__ PcLShare ls;
    const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const bool producer = wave >= 4;
    const int c = wave & 3;  // consumer column block / producer column block
    // a head's segments on one XCD: the replay's chain then reads the
    // summaries from the L2 they were written to
    const int bid = xcd_block(blockIdx.x, gridDim.x);
    const int seg = bid % p.Ssum, h = bid / p.Ssum;
    const int T = p.Tkv;
    const int t0 = seg * p.seg_tokens;
    const int tend = min(T, t0 + p.seg_tokens);
    const int nsb = (tend - t0 + L - 1) / L;

    PcLoader<ST> ld;
    if (producer) {
        ld.init((c & 1) * 64 + lane, nullptr, p.k, p.v, p.eta, h, T, tend);
        ld.issue(0, t0 + (c >> 1) * L);
        pc_first_commit<ST, L>(raw, ld, c);
    }
    lds_barrier();

    f32x4 Xp[ND], Xb[ND];
    F Xpr[ND], Xbr[ND];
#pragma unroll
    for (int r = 0; r < ND; ++r) {
        Xp[r] = zero4();
        Xb[r] = zero4();
        Xpr[r] = to_frag<E>(zero4());
        Xbr[r] = Xpr[r];
    }
    auto prod = [&](const SbTile<E, D, ST> &t, int n) {
        if constexpr (LT) {
            PcSumDer<LT> &dv = der[n & 1];
            switch (c) {
            case 0: pc_derive_sum<0, CH>(t, dv, ls, n, L, lane, m, g); break;
            case 1: pc_derive_sum<1, CH>(t, dv, ls, n, L, lane, m, g); break;
            case 2: pc_derive_sum<2, CH>(t, dv, ls, n, L, lane, m, g); break;
            default: pc_derive_sum<3, CH>(t, dv, ls, n, L, lane, m, g); break;
            }
        }
    };
    auto cons = [&](const SbTile<E, D, ST> &t, int n) {
        f32x4 et[4];
        load_eta(t, L, g, et);
        if (!MSE) {
            F EV[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) EV[i] = to_bf16x4(to_f32x4(v_tok(t, i, c, m, g)) * et[i]);
#pragma unroll
            for (int r = 0; r < ND; ++r)
#pragma unroll
                for (int i = 0; i < 4; i += 2)
                    Xb[r] = mma32(Xb[r], k_tok(t, i, r, m, g), k_tok(t, i + 1, r, m, g), EV[i], EV[i + 1]);
            return;
        }
        // tiles (and the P and B halves) side by side: consecutive MFMAs are
        // independent
        f32x4 Kc[4], Vc[4];
        F Ka[4][ND];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (LT) {
                const PcSumDer<LT> &dv = der[n & 1];
                Kc[i] = dv.kc[c][i][lane];
                Vc[i] = to_f32x4(v_tok(t, i, c, m, g));
#pragma unroll
                for (int r = 0; r < ND; ++r) Ka[i][r] = dv.kt.row(i, r, m, g);
            } else {
                Kc[i] = to_f32x4(k_tok(t, i, c, m, g));
                Vc[i] = to_f32x4(v_tok(t, i, c, m, g));
#pragma unroll
                for (int r = 0; r < ND; ++r) Ka[i][r] = k_row(t, i, r, m, g);
            }
        }
        if constexpr (LT) {
            // T V for this column block, from the super-block's shared blocks
            bf16x4 Ln[6];
            pc_lshare_read<CH>(ls, n, Ln, lane);
            substitute_ch<CH>(Vc, Ln);
        }
        f32x4 Ap[4] = {zero4(), zero4(), zero4(), zero4()}, Ab[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int r = 0; r < ND; r += 2)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Ap[i] = mma32(Ap[i], Ka[i][r], Ka[i][r + 1], Xpr[r], Xpr[r + 1]);
                Ab[i] = mma32(Ab[i], Ka[i][r], Ka[i][r + 1], Xbr[r], Xbr[r + 1]);
            }
        F EUp[4], EUb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            EUp[i] = to_bf16x4((Kc[i] - Ap[i]) * et[i]);
            EUb[i] = to_bf16x4((Vc[i] - Ab[i]) * et[i]);
        }
        F kt[4][ND];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < ND; ++r) kt[i][r] = k_tok(t, i, r, m, g);
#pragma unroll
        for (int r = 0; r < ND; ++r) {
            Xp[r] = mma32(Xp[r], kt[0][r], kt[1][r], EUp[0], EUp[1]);
            Xb[r] = mma32(Xb[r], kt[0][r], kt[1][r], EUb[0], EUb[1]);
        }
#pragma unroll
        for (int r = 0; r < ND; ++r) {
            Xp[r] = mma32(Xp[r], kt[2][r], kt[3][r], EUp[2], EUp[3]);
            Xb[r] = mma32(Xb[r], kt[2][r], kt[3][r], EUb[2], EUb[3]);
            Xpr[r] = to_bf16x4(Xp[r]);
            Xbr[r] = to_bf16x4(Xb[r]);
        }
    };
    pc_walk<ST, L>(raw, ld, producer, c, t0, nsb, cons, prod);

    const size_t base = ((size_t)h * p.Ssum + seg) * D * D;
    if (!producer) {
        if (MSE) {
            E *dst = (E *)p.wsP + base;
#pragma unroll
            for (int r = 0; r < ND; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[(size_t)(16 * r + 4 * g + j) * D + 16 * c + m] = (E)Xp[r][j];
        }
        f32x4 *dst = reinterpret_cast<f32x4 *>(p.wsB + base) + c * ND * 64;
#pragma unroll
        for (int r = 0; r < ND; ++r) dst[r * 64 + lane] = Xb[r];
    } else if (seg == 0 && p.wsW0) {
        // copy of w_init for the replay when w_final is the same buffer
        const f32x4 *src = reinterpret_cast<const f32x4 *>(p.w_init + (size_t)h * D * D);
        f32x4 *dst = reinterpret_cast<f32x4 *>(p.wsW0 + (size_t)h * D * D);
        for (int i = threadIdx.x - 256; i < D * D / 4; i += 256) dst[i] = src[i];
    }
}

template <bool MSE, int CH>
__global__ __launch_bounds__(512) void lin_replay_pc(LinParams p)
{
    typedef __bf16 E;
    typedef bf16x4 F;
    constexpr int D = 64, ND = 4, L = PcCfg<CH>::L;
    constexpr bool LT = MSE && PcCfg<CH>::MULTI;
    constexpr int ST = STAGE_Q | STAGE_K | STAGE_V | STAGE_E | STAGE_SWZ;
    // the chain's staging and the walk's tiles are never live together
    __shared__ union {
        struct {
            SbTile<E, D, ST> raw[PC_NR];
            PcRepDer<LT> der[2];
        } w;
        PcChainStage cs;
    } u;
    __shared__ PcLShare ls;
    SbTile<E, D, ST> *raw = u.w.raw;
    PcRepDer<LT> *der = u.w.der;
    const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const bool producer = wave >= 4;
    const int c = wave & 3;
    const int bid = xcd_block(blockIdx.x, gridDim.x);  // a head's segments on one XCD
    const int seg = bid % p.S, h = bid / p.S;
    const int T = p.Tkv;
    const int t0 = seg * p.seg_tokens;
    const int tend = min(T, t0 + p.seg_tokens);
    const int nsb = (tend - t0 + L - 1) / L;

    PcLoader<ST> ld;
    f32x4 R[ND];
    SplitFrag<E> Rs[ND];
    const bool chain_lds = MSE && seg > 0;
    if (chain_lds) pc_chain_init(u.cs);
    if (producer) {
        ld.init((c & 1) * 64 + lane, p.q, p.k, p.v, p.eta, h, T, tend);
        // the chain's loads go first; each wave's first super-block load
        // follows its last chain commit
        if (chain_lds) {
            pc_chain_stage(p, h, seg, u.cs, c, lane, [&] { ld.issue(0, t0 + (c >> 1) * L); });
            lds_barrier();  // the consumers are done with the staging, which the tiles overlay
        } else {
            ld.issue(0, t0 + (c >> 1) * L);
        }
        pc_first_commit<ST, L>(raw, ld, c);
    } else {
        // w_init itself, or the summary's copy of it when w_final is the same
        // buffer (the last segment writes it while earlier ones may still read)
        const float *ws = (p.wsW0 ? p.wsW0 : p.w_init) + (size_t)h * D * D;
#pragma unroll
        for (int r = 0; r < ND; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) R[r][j] = ws[(size_t)(16 * r + 4 * g + j) * D + 16 * c + m];
        if (seg > 0) {
            if (MSE) {
                pc_chain_lds(R, seg, u.cs, c, lane, m, g, [](int) {});
                lds_barrier();  // pairs with the producers' barrier after their staging
            } else {
                pc_chain<false>(R, p, h, seg, c, lane, m, g, [](int) {});
            }
        }
#pragma unroll
        for (int r = 0; r < ND; ++r) Rs[r].set(R[r]);
    }
    lds_barrier();

    E *out_h = (E *)p.out + (size_t)h * T * D;
    auto prod = [&](const SbTile<E, D, ST> &t, int n) {
        PcRepDer<LT> &dv = der[n & 1];
        switch (c) {
        case 0: pc_derive_rep<0, LT, CH>(t, dv, ls, n, L, lane, m, g); break;
        case 1: pc_derive_rep<1, LT, CH>(t, dv, ls, n, L, lane, m, g); break;
        case 2: pc_derive_rep<2, LT, CH>(t, dv, ls, n, L, lane, m, g); break;
        default: pc_derive_rep<3, LT, CH>(t, dv, ls, n, L, lane, m, g); break;
        }
    };
    auto cons = [&](const SbTile<E, D, ST> &t, int n) {
        const PcRepDer<LT> &dv = der[n & 1];
        const int s = t0 + n * L;
        const int lim = min(tend, s + L);
        f32x4 et[4];
        load_eta(t, L, g, et);
        // The four tiles' products are issued side by side (tile index
        // innermost) so that consecutive MFMAs are independent.
        f32x4 U[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) U[i] = to_f32x4(v_tok(t, i, c, m, g));
        if constexpr (LT) {
            // T V for this column block, from the super-block's shared blocks
            bf16x4 Ln[6];
            pc_lshare_read<CH>(ls, n, Ln, lane);
            substitute_ch<CH>(U, Ln);
        }
        if (MSE) {
            F Ka[4][ND];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < ND; ++r) {
                    if constexpr (LT)
                        Ka[i][r] = dv.kt.row(i, r, m, g);
                    else
                        Ka[i][r] = k_row(t, i, r, m, g);
                }
            f32x4 KR[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
            for (int r = 0; r < ND; r += 2)
#pragma unroll
                for (int i = 0; i < 4; ++i) KR[i] = mma32(KR[i], Ka[i][r], Ka[i][r + 1], Rs[r].hi, Rs[r + 1].hi);
#pragma unroll
            for (int r = 0; r < ND; r += 2)
#pragma unroll
                for (int i = 0; i < 4; ++i) KR[i] = mma32(KR[i], Ka[i][r], Ka[i][r + 1], Rs[r].lo, Rs[r + 1].lo);
#pragma unroll
            for (int i = 0; i < 4; ++i) U[i] = U[i] - KR[i];
        }
        F Uf[4], EU[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Uf[i] = to_bf16x4(U[i]);
            EU[i] = to_bf16x4(U[i] * et[i]);
        }
        // O^T_i = R^T Q_i^T + sum_{j<=i} U_j^T A_ij^T (transposed so each lane
        // stores four consecutive columns of one token)
        constexpr int NTI = (L + 15) / 16;  // tiles holding outputs
        F Qa[4][ND];
#pragma unroll
        for (int i = 0; i < NTI; ++i)
#pragma unroll
            for (int r = 0; r < ND; ++r) Qa[i][r] = q_row(t, i, r, m, g);
        f32x4 O[4] = {zero4(), zero4(), zero4(), zero4()};
#pragma unroll
        for (int r = 0; r < ND; r += 2)
#pragma unroll
            for (int i = 0; i < NTI; ++i) O[i] = mma32(O[i], Rs[r].hi, Rs[r + 1].hi, Qa[i][r], Qa[i][r + 1]);
#pragma unroll
        for (int r = 0; r < ND; r += 2)
#pragma unroll
            for (int i = 0; i < NTI; ++i) O[i] = mma32(O[i], Rs[r].lo, Rs[r + 1].lo, Qa[i][r], Qa[i][r + 1]);
#pragma unroll
        for (int j = 0; j < 4; j += 2)
#pragma unroll
            for (int i = j; i < NTI; ++i) {
                if (j + 1 <= i)
                    O[i] = mma32(O[i], Uf[j], Uf[j + 1], dv.ab[ablk(i, j) - 6][lane], dv.ab[ablk(i, j + 1) - 6][lane]);
                else
                    O[i] = mma32z(O[i], Uf[j], dv.ab[ablk(i, j) - 6][lane]);
            }
#pragma unroll
        for (int i = 0; i < NTI; ++i) {
            const int tk = s + 16 * i + m;
            if (tk < lim) store4<E>(out_h + (size_t)tk * D + 16 * c + 4 * g, out4<E>(O[i]));
        }
        // R += K^T diag(eta) U
#pragma unroll
        for (int r = 0; r < ND; ++r) R[r] = mma32(R[r], k_tok(t, 0, r, m, g), k_tok(t, 1, r, m, g), EU[0], EU[1]);
#pragma unroll
        for (int r = 0; r < ND; ++r) {
            R[r] = mma32(R[r], k_tok(t, 2, r, m, g), k_tok(t, 3, r, m, g), EU[2], EU[3]);
            Rs[r].set(R[r]);
        }
    };
    pc_walk<ST, L>(raw, ld, producer, c, t0, nsb, cons, prod);

    if (!producer && seg == p.S - 1) {
        float *wf = p.w_final + (size_t)h * D * D;
#pragma unroll
        for (int r = 0; r < ND; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) wf[(size_t)(16 * r + 4 * g + j) * D + 16 * c + m] = R[r][j];
    }
}

// ---------------------------------------------------------------------------
// apply (non-causal): O = Q W_final over query segments.
// ---------------------------------------------------------------------------
template <typename E, int D, int PD>
__global__ __launch_bounds__((D / 16) * 64) void lin_apply(LinParams p, const float *wsrc,
                                                           size_t wsrc_head_stride)
{
    typedef typename Frag<E>::type F;
    constexpr int ND = D / 16;
    constexpr int NT = ND * 64;
    constexpr int ST = STAGE_Q | STAGE_PERM;
    __shared__ SbTile<E, D, ST> tiles[2];
    const int lane = threadIdx.x & 63, g = lane >> 4, m = lane & 15;
    const int c = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // column block
    (void)lane;
    const int seg = blockIdx.x % p.Sq, h = blockIdx.x / p.Sq;
    const int T = p.Tq;
    const int t0 = seg * p.seg_q;
    const int tend = min(T, t0 + p.seg_q);
    const float *ws = wsrc + (size_t)h * wsrc_head_stride;
    SplitFrag<E> Wr[ND];
#pragma unroll
    for (int r = 0; r < ND; ++r) {
        f32x4 w;
#pragma unroll
        for (int j = 0; j < 4; ++j) w[j] = ws[(size_t)(16 * r + 4 * g + j) * D + 16 * c + m];
        Wr[r].set(w);
    }
    SbLoader<E, D, ST, PD, NT> ld;
    ld.init(threadIdx.x, p.q, nullptr, nullptr, nullptr, h, T, tend);
    E *out_h = (E *)p.out + (size_t)h * T * D;
    const SbSched sc(SB);
    run_sb<E, D, ST, PD, NT, 2>(tiles, ld, sc, t0, tend, [&](SbTile<E, D, ST> &t, int n) {
        const int s = t0 + sc.start(n);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            F Qa[ND];
#pragma unroll
            for (int r = 0; r < ND; r += 2) q_row2(t, i, r, m, g, Qa[r], Qa[r + 1]);
            const f32x4 O = mma_state_a<E, ND>(zero4(), Wr, Qa);
            const int tk = s + 16 * i + m;
            if (tk < tend) store4<E>(out_h + (size_t)tk * D + 16 * c + 4 * g, out4<E>(O));
        }
    });
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

LinearPlan linear_plan(const LinearShape &s)
{
    LinearPlan pl{};
    const int T = s.Tkv;
    // Segment length: whole super-block periods (whole chunks), about one
    // workgroup per CU (longer segments lengthen the serial walk, shorter ones
    // the segment-start chain; 256 measured best on the d = 64 and d = 128
    // workloads), at least four super-blocks: with few heads, more and
    // shorter segments would fill the chip but the chain, which grows with
    // the number of segments, costs more than they save.  A caller-chosen
    // length (seg_tokens > 0) replaces that choice and is rounded up to whole
    // periods.
    const long long period = (s.chunk <= SB) ? (long long)(SB / s.chunk) * s.chunk : s.chunk;
    constexpr long long target_wg = 256;
    long long seg = (T > 0) ? ((long long)s.NH * T + target_wg - 1) / target_wg : period;
    if (seg < 4 * SB) seg = 4 * SB;
    if (s.seg_tokens > 0) seg = s.seg_tokens;
    seg = (seg + period - 1) / period * period;
    if (T > 0 && seg > T) seg = (T + period - 1) / period * period;
    pl.seg_tokens = (int)seg;
    pl.S = (T > 0) ? (int)((T + seg - 1) / seg) : 0;
    pl.Ssum = (s.order == 0) ? (pl.S > 0 ? pl.S - 1 : 0) : pl.S;
    long long segq = (s.Tq > 0) ? ((long long)s.NH * s.Tq + target_wg - 1) / target_wg : SB;
    if (segq < SB) segq = SB;
    segq = (segq + SB - 1) / SB * SB;
    pl.seg_q = (int)segq;
    pl.Sq = (s.Tq > 0) ? (int)((s.Tq + segq - 1) / segq) : 0;
    const size_t esz = s.bf16 ? 2 : 4;
    const size_t dd = (size_t)s.d * s.d;
    size_t off = 0;
    pl.offP = off;
    if (s.loss == 1) off = align_up(off + (size_t)s.NH * pl.Ssum * dd * esz, 256);
    pl.offB = off;
    off = align_up(off + (size_t)s.NH * pl.Ssum * dd * 4, 256);
    pl.offW = off;  // copy of w_init (causal, more than one segment)
    if (s.order == 0 && pl.S > 1) off = align_up(off + (size_t)s.NH * dd * 4, 256);
    pl.bytes = off;
    return pl;
}

template <typename E, int D, bool MSE, bool LT, bool SNAP>
static hipError_t launch_typed(const LinearShape &s, const LinearPlan &pl, LinParams p,
                               hipStream_t st)
{
    constexpr int ND = D / 16;
    constexpr int PD = 2;  // super-blocks in flight
    const dim3 block(ND * 64);
    if (s.Tkv > 0) {
        if (pl.Ssum > 0) lin_summary<E, D, MSE, LT, SNAP, PD><<<dim3(s.NH * pl.Ssum), block, 0, st>>>(p);
        if (s.order == 0) {
            lin_replay<E, D, MSE, LT, SNAP, PD><<<dim3(s.NH * pl.S), block, 0, st>>>(p);
        } else {
            lin_final<E, D, MSE><<<dim3(s.NH), block, 0, st>>>(p);
            if (pl.Sq > 0)
                lin_apply<E, D, PD><<<dim3(s.NH * pl.Sq), block, 0, st>>>(p, p.w_final, (size_t)D * D);
        }
    } else {
        // No key/value tokens: the state is unchanged.
        if (p.w_final != p.w_init) {
            hipError_t e = hipMemcpyAsync(p.w_final, p.w_init, (size_t)s.NH * D * D * 4,
                                          hipMemcpyDeviceToDevice, st);
            if (e != hipSuccess) return e;
        }
        if (s.order == 1 && pl.Sq > 0)
            lin_apply<E, D, PD><<<dim3(s.NH * pl.Sq), block, 0, st>>>(p, p.w_init, (size_t)D * D);
    }
    return hipGetLastError();
}

template <bool MSE, int CH>
static hipError_t launch_pc(const LinearShape &s, const LinearPlan &pl, LinParams p, hipStream_t st)
{
    const dim3 block(512);
    if (pl.Ssum > 0) lin_summary_pc<MSE, CH><<<dim3(s.NH * pl.Ssum), block, 0, st>>>(p);
    if (s.order == 0) {
        lin_replay_pc<MSE, CH><<<dim3(s.NH * pl.S), block, 0, st>>>(p);
    } else {
        lin_final<__bf16, 64, MSE><<<dim3(s.NH), dim3(256), 0, st>>>(p);
        if (pl.Sq > 0) lin_apply<__bf16, 64, 2><<<dim3(s.NH * pl.Sq), dim3(256), 0, st>>>(p, p.w_final, 64 * 64);
    }
    return hipGetLastError();
}

hipError_t linear_launch(const LinearShape &s, const LinearPlan &pl, const void *q, const void *k,
                         const void *v, const float *eta, const float *w_init, void *out,
                         float *w_final, void *ws, hipStream_t stream)
{
    LinParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.eta = eta;
    p.w_init = w_init;
    p.out = out;
    p.w_final = w_final;
    p.wsP = (char *)ws + pl.offP;
    p.wsB = (float *)((char *)ws + pl.offB);
    // The replay reads w_init at its start while the last segment writes
    // w_final at its end: a copy is needed only when the two are one buffer.
    p.wsW0 = (s.order == 0 && pl.S > 1 && (const void *)w_final == (const void *)w_init)
                 ? (float *)((char *)ws + pl.offW)
                 : nullptr;
    p.NH = s.NH;
    p.Tq = s.Tq;
    p.Tkv = s.Tkv;
    p.chunk = s.chunk;
    p.seg_tokens = pl.seg_tokens;
    p.S = pl.S;
    p.Ssum = pl.Ssum;
    p.seg_q = pl.seg_q;
    p.Sq = pl.Sq;
    const bool mse = s.loss == 1;
    // b < 64: transform by T; b > 64: chunk-start snapshots; b = 64: neither.
    const bool lt = s.chunk < SB, snap = s.chunk > SB;
    if (s.bf16 && s.d == 64 && !snap && s.Tkv > 0) {
        // producer/consumer kernels; the inner-product loss only needs the
        // super-block length (64, or 48 for b = 48)
        if (!mse) return s.chunk == 48 ? launch_pc<false, 48>(s, pl, p, stream) : launch_pc<false, 64>(s, pl, p, stream);
        switch (s.chunk) {
        case 16: return launch_pc<true, 16>(s, pl, p, stream);
        case 32: return launch_pc<true, 32>(s, pl, p, stream);
        case 48: return launch_pc<true, 48>(s, pl, p, stream);
        default: return launch_pc<true, 64>(s, pl, p, stream);
        }
    }
#define TTT_DISPATCH(E, D)                                                                  \
    if (mse) {                                                                              \
        if (lt) return launch_typed<E, D, true, true, false>(s, pl, p, stream);             \
        if (snap) return launch_typed<E, D, true, false, true>(s, pl, p, stream);           \
        return launch_typed<E, D, true, false, false>(s, pl, p, stream);                    \
    }                                                                                       \
    return launch_typed<E, D, false, false, false>(s, pl, p, stream);
    if (s.bf16) {
        if (s.d == 64) { TTT_DISPATCH(__bf16, 64) }
        if (s.d == 128) { TTT_DISPATCH(__bf16, 128) }
    } else {
        if (s.d == 64) { TTT_DISPATCH(float, 64) }
        if (s.d == 128) { TTT_DISPATCH(float, 128) }
    }
#undef TTT_DISPATCH
    return hipErrorInvalidValue;
}

}  // namespace tttk
