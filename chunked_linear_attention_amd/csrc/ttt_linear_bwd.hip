// Backward pass of the causal TTT-Linear forward (fp32, gfx950).
//
// The forward ("Test-Time Training (TTT)": "TTT definition", examples 1 and 2,
// "TTT-Linear", "Mini-batch gradient descent") in its per-chunk form, with W_c
// the chunk-start state, H = diag(eta) and M the inclusive causal mask:
//     U = V - K W_c  (MSE)  or  V  (inner product)
//     A = (Q K^T) * M,   S = A H,   O = Q W_c + S U,   W_{c+1} = W_c + K^T H U.
// Given dO and G = dL/dW_{c+1}, the chunk's adjoints are
//     dU   = S^T dO + H (K G)
//     dS   = (dO U^T) * M,          dA = dS H
//     deta = rowsum_t(dS * A)^T + rowsum((K G) * U)
//     dQ   = dO W_c^T + dA K
//     dK   = dA^T Q + H U G^T  [- dU W_c^T  (MSE)]
//     dV   = dU
//     dL/dW_c = G + Q^T dO  [- K^T dU  (MSE)]
// Only two recursions are serial over the chunks, and neither mixes the
// columns of its d x d matrix: the forward one for the chunk-start states,
//     W_{c+1} = W_c + K^T H (V - K W_c),
// and the backward one for G,
//     G_c = G_{c+1} + R_c [- K^T H K G_{c+1}],   R_c = Q^T dO [- K^T S~],  S~ = S^T dO.
// So the work runs as the state recursion and the G recursion (segmented:
// maps, chain, walks; fp32 MFMA, one wave per (head, segment, 16 columns)),
// and between and after them two passes with one workgroup per (head, chunk)
// for everything else (the G-free terms and R_c first, then the terms that
// need G_{c+1}; fp32 FMA in LDS), exchanging per-chunk matrices through the
// workspace.
#include "ttt_device.h"
#include "ttt_internal.h"

#include <hip/hip_runtime.h>

namespace tttk {
namespace {

struct LinBwdParams {
    const void *q, *k, *v, *dout;
    const float *eta, *w0, *dwf;
    void *dq, *dk, *dv;
    float *deta, *dw0;
    float *states;  // [NH][nchunks][D][D]  chunk-start states W_c
    float *gnext;   // [NH][nchunks][D][D]  G_{c+1} = dL/dW_{c+1}
    float *rc;      // [NH][nchunks][D][D]  R_c = Q^T dO [- K^T S~]
    float *ub;      // [NH][nchunks * B][D] U (MSE residuals)
    float *st;      // [NH][nchunks * B][D] S~ = S^T dO
    float *dkl;     // [NH][nchunks * B][D] dA^T Q [- S~ W_c^T]
    int T, nchunks, loss;  // T: key/value tokens (= queries in the causal order)
    int order, Tq;         // order 1: update over all key/value chunks, then apply to Tq queries
    float *wfinal;         // [NH][D][D] (order 1) final state
    float *ginit;          // [NH][D][D] (order 1) dL/dW_final incl. the apply's Q^T dO
    // The per-token buffers have head stride rstride = nchunks * chunk rows.
    long rstride;
    // Segments of the serial passes: nseg runs of seg_chunks chunks (the last
    // may be shorter) per head.  ssum: [NH][nseg][D][2D], each segment's affine
    // map as [linear part | offset]; sstart: [NH][nseg][D][D], each segment's
    // start state (states) or end adjoint (G).
    int nseg, seg_chunks;
    float *ssum, *sstart;
    // Every pass steps over 16-token tiles: tpc per chunk, nwt per head.
    int tpc, nwt;
};

template <typename E> __device__ __forceinline__ float ldf(const void *p, long i)
{
    return (float)static_cast<const E *>(p)[i];
}
template <typename E> __device__ __forceinline__ void stf(void *p, long i, float x)
{
    static_cast<E *>(p)[i] = (E)x;
}

constexpr int CB = 16;  // state columns per workgroup in the serial passes
constexpr int DEP_TPW = 8;  // tiles per workgroup of the dependent pass (chunks of several tiles)

// four consecutive floats of an LDS row (16-byte aligned)
__device__ __forceinline__ f32x4 lds4(const float *x) { return *reinterpret_cast<const f32x4 *>(x); }

// Both serial recursions are affine in their d x d matrix, chunk by chunk:
//   states  W_{c+1} = (I - K^T H K) W_c + K^T H V,
//   G       G_c     = (I - K^T H K) G_{c+1} + R_c,
// and neither mixes the matrix's columns.  So a segment of chunks is one
// affine map X -> L X + F; its two parts come out of the same walk started
// from the identity without the inputs (L) or from zero with them (F).  Three
// steps per recursion: the maps of all segments in parallel (mode 1, one wave
// per (head, segment, 16 columns of [L | F])), the chain of the maps per
// (head, 16 columns) (lbw_chain_m), and the walk of every segment from its
// own start (mode 0, per (head, segment, 16 columns)), which stores what the
// parallel passes read.  The chain, per (head, 16 columns):
// dir 0 (states): X_0 = w_init, X_{s+1} = L_s X_s + F_s, storing X_s for s >= 1;
// dir 1 (G): X_{S-1} = g0 (d_w_final, or the apply's G in the update-then-apply
// order, or zero), X_{s-1} = L_s X_s + F_s, storing X_s for s <= S - 2.

// ---------------------------------------------------------------------------
// The serial passes on the matrix cores (fp32 16x16x4 MFMA).  One wave per
// (head, segment, 16 columns) steps over 16-token tiles (a chunk of b tokens
// is b / 16 tiles: every residual of a chunk reads the chunk-start state and
// every G-term reads G_{c+1}, kept as a snapshot when a chunk has several
// tiles).  The wave holds its D x 16 slice of the matrix as D / 16
// accumulator tiles, lane (g, n) keeping rows 16 s + 4 g + r (r < 4) of
// column n.  Taking the contraction index of MFMA step j on lane group g as
// 4 g + j, that accumulator is also the B operand of the next product, and so
// is the accumulator of Y below; a tile step is
//     Y = K X                                (A: K rows, 4 features a lane)
//     X += K^T H (V - Y)   or   G -= K^T H Y  (A: K columns, B: Y itself)
// with the K tile staged in the wave's own LDS (no barriers).
// ---------------------------------------------------------------------------
constexpr int WT = 16;  // tokens per walk tile
// Walk tiles in flight per wave: a step is a few hundred cycles of MFMA work,
// short against the latency of its loads.
template <int D> constexpr int WPF = D == 64 ? 4 : 3;

template <int D> struct WalkTile {
    float k[WT][D + 4];  // rows padded by 4: row and column fragment reads spread over the banks
};

// One K tile in registers (16-byte pieces), loaded a step ahead.
template <int D, typename E> struct WalkK {
    static constexpr int PE = 16 / (int)sizeof(E);  // elements per piece
    static constexpr int PPR = D / PE;              // pieces per token row
    static constexpr int NP = WT * PPR / 64;        // pieces per lane
    static_assert(NP * 64 == WT * PPR, "walk tile shape");
    u32x4 v[NP];
    // Rows past T read the last row (an in-bounds address, no branch around
    // the load) and are zeroed when the tile is written to LDS.
    __device__ __forceinline__ void load(const void *k, long tok0, int t0, int T, int lane)
    {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int idx = lane + 64 * i, t = min(t0 + idx / PPR, T - 1);
            v[i] = *reinterpret_cast<const u32x4 *>(static_cast<const E *>(k) + (tok0 + t) * D + PE * (idx % PPR));
        }
    }
    __device__ __forceinline__ void put(WalkTile<D> &w, int lane, int n) const  // n: valid rows
    {
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int idx = lane + 64 * i, row = idx / PPR, c = PE * (idx % PPR);
            const u32x4 x = row < n ? v[i] : u32x4{0u, 0u, 0u, 0u};
            if constexpr (sizeof(E) == 2) {
                const bf16x8 b = __builtin_bit_cast(bf16x8, x);
                *reinterpret_cast<f32x4 *>(&w.k[row][c]) = f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
                *reinterpret_cast<f32x4 *>(&w.k[row][c + 4]) = f32x4{(float)b[4], (float)b[5], (float)b[6], (float)b[7]};
            } else {
                *reinterpret_cast<f32x4 *>(&w.k[row][c]) = __builtin_bit_cast(f32x4, x);
            }
        }
    }
};

// A operand K[m][16 s + 4 q + j] (contraction over features) ...
template <int D>
__device__ __forceinline__ f32x4 walk_rows(const WalkTile<D> &w, int s, int m, int q)
{
    return *reinterpret_cast<const f32x4 *>(&w.k[m][16 * s + 4 * q]);
}
// ... and K[4 q + j][16 s + m] (contraction over tokens: rows of K^T).
template <int D>
__device__ __forceinline__ f32x4 walk_cols(const WalkTile<D> &w, int s, int m, int q)
{
    return f32x4{w.k[4 * q][16 * s + m], w.k[4 * q + 1][16 * s + m], w.k[4 * q + 2][16 * s + m],
                 w.k[4 * q + 3][16 * s + m]};
}

// Rows 4 g + r of the tile starting at token t0, column col of a token-major
// [T][D] tensor, and the tokens' eta, as loaded (raw); walk_f32 turns them
// into floats, zero past T (rows past T read row T - 1: no branch around a
// load, so its wait can sit at the first use, a step later).
template <typename E> struct WalkCol {
    E x[4];
};
template <typename E>
__device__ __forceinline__ WalkCol<E> walk_col4(const void *x, long tok0, int t0, int T, int D, int col, int g)
{
    WalkCol<E> r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.x[i] = static_cast<const E *>(x)[(tok0 + min(t0 + 4 * g + i, T - 1)) * D + col];
    return r;
}
__device__ __forceinline__ WalkCol<float> walk_eta4(const float *eta, long tok0, int t0, int T, int g)
{
    WalkCol<float> r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.x[i] = eta[tok0 + min(t0 + 4 * g + i, T - 1)];
    return r;
}
template <typename E>
__device__ __forceinline__ f32x4 walk_f32(const WalkCol<E> &c, int t0, int T, int g)
{
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = t0 + 4 * g + i < T ? (float)c.x[i] : 0.f;
    return r;
}

// A D x 16 column slice of a row-major matrix with row stride ld <-> accumulator tiles.
template <int NS>
__device__ __forceinline__ void slice_load(f32x4 *X, const float *src, long ld, int g, int m)
{
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) X[s][r] = src[(long)(16 * s + 4 * g + r) * ld + m];
}
template <int NS>
__device__ __forceinline__ void slice_store(float *dst, const f32x4 *X, long ld, int g, int m)
{
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(long)(16 * s + 4 * g + r) * ld + m] = X[s][r];
}
template <int NS>
__device__ __forceinline__ void slice_identity(f32x4 *X, int j0, int g, int m, bool one)
{
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) X[s][r] = (one && 16 * s + 4 * g + r == j0 + m) ? 1.f : 0.f;
}

// Walk of the state recursion over one segment (mode 0: from its start state,
// storing every chunk-start state, and the final state in the
// update-then-apply order; mode 1: the segment's map, wave columns [0, D) the
// linear part from the identity without V, [D, 2D) the offset from zero).
template <int D, typename E>
__global__ __launch_bounds__(256) void lbw_states_m(LinBwdParams p, int mode)
{
    constexpr int NS = D / 16;
    __shared__ WalkTile<D> tiles[4];
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
    const int ncol = (mode == 1 ? 2 : 1) * NS;
    const int nsl = mode == 1 ? p.nseg - 1 : p.nseg;  // the last segment's map is never needed
    int w = blockIdx.x * 4 + wv;
    const int cbk = w % ncol;
    w /= ncol;
    const int seg = w % nsl, h = w / nsl;
    const bool lin = mode == 1 && cbk < NS;
    const bool mse = p.loss == 1;
    const int j0 = (cbk % NS) * 16, tpc = p.tpc;
    const long tok0 = (long)h * p.T;
    const int ca = seg * p.seg_chunks, cb = min(p.nchunks, ca + p.seg_chunks);
    const int ta = ca * tpc, tb = min(cb * tpc, p.nwt);
    WalkTile<D> &kt = tiles[wv];
    f32x4 X[NS], S[NS];
    if (mode == 1)
        slice_identity<NS>(X, j0, g, m, lin);
    else
        slice_load<NS>(X, (seg == 0 ? p.w0 + (long)h * D * D : p.sstart + ((long)h * p.nseg + seg) * D * D) + j0,
                       D, g, m);
    // WPF tiles in flight, ring slots fixed at compile time by unrolling
    constexpr int PF = WPF<D>;
    WalkK<D, E> nk[PF];
    WalkCol<E> vn[PF];
    WalkCol<float> en[PF];
    auto fetch = [&](int j, int t) {
        nk[j].load(p.k, tok0, t * WT, p.T, lane);
        vn[j] = walk_col4<E>(p.v, tok0, t * WT, p.T, D, j0 + m, g);
        en[j] = walk_eta4(p.eta, tok0, t * WT, p.T, g);
    };
    // Every slot is refilled unconditionally (tiles past the segment or past T
    // read in-bounds rows and go unused), so no ring register is ever merged
    // with an unloaded value and no load needs an early wait.
#pragma unroll
    for (int j = 0; j < PF; ++j) fetch(j, ta + j);
    for (int t0 = ta; t0 < tb; t0 += PF) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            // slots are staged and refilled past the segment's end too (no exit
            // from the group: the ring registers stay in place)
            const int t = t0 + j;
            nk[j].put(kt, lane, p.T - t * WT);
            const f32x4 vc = lin ? zero4() : walk_f32(vn[j], t * WT, p.T, g);
            const f32x4 ec = walk_f32(en[j], t * WT, p.T, g);
            fetch(j, t + PF);
            if (t < tb) {
                if (t % tpc == 0) {  // a chunk starts: store its state (and snapshot it)
                    if (mode == 0)
                        slice_store<NS>(p.states + ((long)h * p.nchunks + t / tpc) * D * D + j0, X, D, g, m);
                    if (tpc > 1 && mse)
#pragma unroll
                        for (int s = 0; s < NS; ++s) S[s] = X[s];
                }
                f32x4 U = vc;
                if (mse) {  // U = V - K W_c
                    f32x4 Y = zero4();
#pragma unroll
                    for (int s = 0; s < NS; ++s) Y = mma16(Y, walk_rows<D>(kt, s, m, g), tpc > 1 ? S[s] : X[s]);
                    U = vc - Y;
                }
                const f32x4 HU = U * ec;
#pragma unroll
                for (int s = 0; s < NS; ++s) X[s] = mma16(X[s], walk_cols<D>(kt, s, m, g), HU);
            }
        }
    }
    if (mode == 1)
        slice_store<NS>(p.ssum + ((long)h * p.nseg + seg) * D * 2 * D + (lin ? 0 : D) + j0, X, 2 * D, g, m);
    else if (p.order == 1 && seg == p.nseg - 1)
        slice_store<NS>(p.wfinal + (long)h * D * D + j0, X, D, g, m);
}

// Walk of the G recursion over one segment, last tile first (mode 0: from the
// segment's end adjoint, storing every G_{c+1}, and d_w_init at the start of
// the first segment; mode 1: the map of segments 1 .. S-1, wave columns
// [0, D) the linear part from the identity without R_c, [D, 2D) the offset
// from zero).  G_c = G_{c+1} + R_c [- K^T H K G_{c+1}].
template <int D, typename E, bool MSE>
__global__ __launch_bounds__(256) void lbw_grad_m(LinBwdParams p, int mode)
{
    constexpr int NS = D / 16;
    __shared__ WalkTile<D> tiles[4];
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave-uniform
    const int ncol = (mode == 1 ? 2 : 1) * NS;
    const int nsl = mode == 1 ? p.nseg - 1 : p.nseg;
    int w = blockIdx.x * 4 + wv;
    const int cbk = w % ncol;
    w /= ncol;
    const int seg = w % nsl + (mode == 1 ? 1 : 0), h = w / nsl;
    const bool lin = mode == 1 && cbk < NS;
    const bool addr = !lin && p.order == 0;  // R_c enters (none in the update-then-apply order)
    const int j0 = (cbk % NS) * 16, tpc = p.tpc;
    const long tok0 = (long)h * p.T;
    const int ca = seg * p.seg_chunks, ce = min(p.nchunks, ca + p.seg_chunks);
    const int ta = ca * tpc, last = min(ce * tpc, p.nwt) - 1;
    // the first tile of a chunk in this (reverse) order: its last one
    auto chunk_end = [&](int t) { return t == p.nwt - 1 || t % tpc == tpc - 1; };
    WalkTile<D> &kt = tiles[wv];
    f32x4 G[NS], Gs[NS];
    if (mode == 1) {
        slice_identity<NS>(G, j0, g, m, lin);
    } else {
        const float *g0 = p.order == 1 ? p.ginit : p.dwf;  // null: zero
        const float *src = seg == p.nseg - 1 ? (g0 ? g0 + (long)h * D * D : nullptr)
                                             : p.sstart + ((long)h * p.nseg + seg) * D * D;
        if (src)
            slice_load<NS>(G, src + j0, D, g, m);
        else
            slice_identity<NS>(G, j0, g, m, false);
    }
    constexpr int PF = WPF<D>;
    WalkK<D, E> nk[PF];
    WalkCol<float> en[PF];
    auto fetch = [&](int j, int t) {  // unconditional, as in the state walk
        if constexpr (MSE) {
            nk[j].load(p.k, tok0, max(t, 0) * WT, p.T, lane);
            en[j] = walk_eta4(p.eta, tok0, max(t, 0) * WT, p.T, g);
        }
    };
#pragma unroll
    for (int j = 0; j < PF; ++j) fetch(j, last - j);
    for (int t0 = last; t0 >= ta; t0 -= PF) {
#pragma unroll
        for (int j = 0; j < PF; ++j) {
            const int t = t0 - j;  // below ta: staged, refilled, not computed
            f32x4 ec = zero4();
            if constexpr (MSE) {
                nk[j].put(kt, lane, p.T - max(t, 0) * WT);
                ec = walk_f32(en[j], max(t, 0) * WT, p.T, g);
            }
            fetch(j, t - PF);
            if (t < ta) continue;
            const bool ce_t = chunk_end(t);
            if (ce_t) {  // G = G_{c+1} of this chunk: store it (and snapshot it)
                if (mode == 0) slice_store<NS>(p.gnext + ((long)h * p.nchunks + t / tpc) * D * D + j0, G, D, g, m);
                if (tpc > 1 && MSE)
#pragma unroll
                    for (int s = 0; s < NS; ++s) Gs[s] = G[s];
            }
            if constexpr (MSE) {
                f32x4 Y = zero4();
#pragma unroll
                for (int s = 0; s < NS; ++s) Y = mma16(Y, walk_rows<D>(kt, s, m, g), tpc > 1 ? Gs[s] : G[s]);
                const f32x4 HY = -(Y * ec);
#pragma unroll
                for (int s = 0; s < NS; ++s) G[s] = mma16(G[s], walk_cols<D>(kt, s, m, g), HY);
            }
            if (ce_t && addr) {
                f32x4 R[NS];
                slice_load<NS>(R, p.rc + ((long)h * p.nchunks + t / tpc) * D * D + j0, D, g, m);
#pragma unroll
                for (int s = 0; s < NS; ++s) G[s] += R[s];
            }
        }
    }
    if (mode == 1)
        slice_store<NS>(p.ssum + ((long)h * p.nseg + seg) * D * 2 * D + (lin ? 0 : D) + j0, G, 2 * D, g, m);
    else if (seg == 0)
        slice_store<NS>(p.dw0 + (long)h * D * D + j0, G, D, g, m);
}

// The chain of the segment maps on the matrix cores, one wave per (head, 16
// columns): X <- L_s X + F_s in the direction and with the stores above.
template <int D>
__global__ __launch_bounds__(256) void lbw_chain_m(LinBwdParams p, int dir)
{
    constexpr int NS = D / 16;
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    const int w = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int h = w / NS, j0 = (w % NS) * 16;
    const int S = p.nseg;
    const float *x0 = dir == 0 ? p.w0 : (p.order == 1 ? p.ginit : p.dwf);
    f32x4 X[NS];
    if (x0)
        slice_load<NS>(X, x0 + (long)h * D * D + j0, D, g, m);
    else
        slice_identity<NS>(X, j0, g, m, false);
    const int nst = S - 1;  // maps applied
    if constexpr (D == 64) {
        // the next map's fragments (80 registers) load while this one applies;
        // steps in pairs so the two register sets are fixed, loads clamped to
        // the last map (no branch around a load)
        f32x4 L[2][NS][NS], F[2][NS];
        auto fetch = [&](int k, int t) {
            t = min(t, nst - 1);
            const float *M = p.ssum + ((long)h * S + (dir == 0 ? t : S - 1 - t)) * D * 2 * D;
            slice_load<NS>(F[k], M + D + j0, 2 * D, g, m);
#pragma unroll
            for (int a = 0; a < NS; ++a)
#pragma unroll
                for (int b = 0; b < NS; ++b)
                    L[k][a][b] = *reinterpret_cast<const f32x4 *>(M + (long)(16 * a + m) * 2 * D + 16 * b + 4 * g);
        };
        if (nst > 0) fetch(0, 0);
        for (int t0 = 0; t0 < nst; t0 += 2) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int t = t0 + k;
                fetch(k ^ 1, t + 1);
                if (t < nst) {
                    const int o = dir == 0 ? t + 1 : S - 2 - t;  // the segment whose start this gives
                    f32x4 Xn[NS];
#pragma unroll
                    for (int a = 0; a < NS; ++a) {
                        Xn[a] = F[k][a];
#pragma unroll
                        for (int b = 0; b < NS; ++b) Xn[a] = mma16(Xn[a], L[k][a][b], X[b]);
                    }
#pragma unroll
                    for (int a = 0; a < NS; ++a) X[a] = Xn[a];
                    slice_store<NS>(p.sstart + ((long)h * S + o) * D * D + j0, X, D, g, m);
                }
            }
        }
    } else {
        for (int t = 0; t < nst; ++t) {
            const int s = dir == 0 ? t : S - 1 - t;  // the map applied
            const int o = dir == 0 ? s + 1 : s - 1;  // the segment whose start it gives
            const float *M = p.ssum + ((long)h * S + s) * D * 2 * D;
            f32x4 Xn[NS];
            slice_load<NS>(Xn, M + D + j0, 2 * D, g, m);  // F_s
#pragma unroll
            for (int a = 0; a < NS; ++a)
#pragma unroll
                for (int b = 0; b < NS; ++b)
                    Xn[a] = mma16(Xn[a], *reinterpret_cast<const f32x4 *>(M + (long)(16 * a + m) * 2 * D + 16 * b + 4 * g),
                                  X[b]);
#pragma unroll
            for (int a = 0; a < NS; ++a) X[a] = Xn[a];
            slice_store<NS>(p.sstart + ((long)h * S + o) * D * D + j0, X, D, g, m);
        }
    }
}

// Stage one or two D x D fp32 matrices (row-major) into LDS rows of pitch P,
// 256 threads: eight 16-byte loads per matrix in flight per thread before
// their stores (a load-store loop would wait out the memory latency once per
// piece).
template <int D, int P, bool TWO, int NT = 256>
__device__ __forceinline__ void stage_mats(float (*d0)[P], const float *s0, float (*d1)[P], const float *s1, int tid)
{
    constexpr int N = D * D / 4 / NT, BT = N < 8 ? N : 8;
    static_assert(N % BT == 0, "staging shape");
#pragma unroll
    for (int b0 = 0; b0 < N; b0 += BT) {
        f32x4 v0[BT], v1[BT];
#pragma unroll
        for (int i = 0; i < BT; ++i) {
            const int e = tid + NT * (b0 + i), r = e / (D / 4), c = 4 * (e % (D / 4));
            v0[i] = *reinterpret_cast<const f32x4 *>(s0 + (long)r * D + c);
            if constexpr (TWO) v1[i] = *reinterpret_cast<const f32x4 *>(s1 + (long)r * D + c);
        }
#pragma unroll
        for (int i = 0; i < BT; ++i) {
            const int e = tid + NT * (b0 + i), r = e / (D / 4), c = 4 * (e % (D / 4));
            *reinterpret_cast<f32x4 *>(&d0[r][c]) = v0[i];
            if constexpr (TWO) *reinterpret_cast<f32x4 *>(&d1[r][c]) = v1[i];
        }
    }
}

// Waves per workgroup of the local and dependent passes: eight at d = 128,
// where their LDS allows one workgroup per CU (two waves per SIMD then), four
// at d = 64.
template <int D> constexpr int PW = D == 128 ? 8 : 4;

// Four consecutive elements of a token-major tensor as floats (i a multiple of 4).
template <typename E> __device__ __forceinline__ f32x4 ld4f(const void *p, long i)
{
    if constexpr (sizeof(E) == 2)
        return to_f32x4(*reinterpret_cast<const bf16x4 *>(static_cast<const __bf16 *>(p) + i));
    else
        return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(p) + i);
}

// Parallel pass 2 on the matrix cores for 16-token chunks (fp32 16x16x4
// MFMA): one workgroup per (head, chunk), four waves, wave w owning column
// tiles w, w + 4, ... of the D / 16.  W_c and the chunk's token rows are
// staged in LDS (rows padded by 4 floats); the chunk's 16 x 16 products A =
// (Q K^T) * M and dA = (dO U^T) * M are formed by every wave (one tile each),
// and their accumulators serve directly as the A operand of A^T X and dA^T X.
template <int D, typename E, bool MSE>
__global__ __launch_bounds__(64 * PW<D>) void lbw_local_m(LinBwdParams p)
{
    constexpr int NS = D / 16, NW = PW<D>, NT = 64 * NW, NCT = NS / NW, P = D + 4;
    __shared__ __align__(16) float Wm[D][P];
    __shared__ __align__(16) float Qs[WT][P], Ks[WT][P], Os[WT][P], Us[WT][P], Ss[WT][P];
    __shared__ __align__(16) float dAs[WT][WT + 4];
    __shared__ float et[WT];
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = blockIdx.x / p.nchunks, c = blockIdx.x % p.nchunks;
    const long tok0 = (long)h * p.T;
    const int t0 = c * WT, n = min(WT, p.T - t0);
    const long cb = (long)h * p.nchunks + c;
    const long row0 = (long)h * p.rstride + t0;  // the chunk's rows in the per-token buffers
    {
        stage_mats<D, P, false, NT>(Wm, p.states + cb * D * D, Wm, nullptr, tid);
        for (int e = tid; e < WT * D / 4; e += NT) {
            const int i = e / (D / 4), col = 4 * (e % (D / 4));
            const long gi = (tok0 + t0 + min(i, n - 1)) * D + col;
            const bool ok = i < n;
            const f32x4 q = ld4f<E>(p.q, gi), k = ld4f<E>(p.k, gi), v = ld4f<E>(p.v, gi), o = ld4f<E>(p.dout, gi);
            *reinterpret_cast<f32x4 *>(&Qs[i][col]) = ok ? q : zero4();
            *reinterpret_cast<f32x4 *>(&Ks[i][col]) = ok ? k : zero4();
            *reinterpret_cast<f32x4 *>(&Us[i][col]) = ok ? v : zero4();
            *reinterpret_cast<f32x4 *>(&Os[i][col]) = ok ? o : zero4();
        }
        if (tid < WT) et[tid] = tid < n ? p.eta[tok0 + t0 + tid] : 0.f;
    }
    __syncthreads();
    if constexpr (MSE) {  // U = V - K W_c (rows stored for the dependent pass)
        f32x4 Uc[NCT];
#pragma unroll
        for (int u = 0; u < NCT; ++u) {
            const int col = 16 * (wv + NW * u) + m;
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < NS; ++s)
                acc = mma16(acc, *reinterpret_cast<const f32x4 *>(&Ks[m][16 * s + 4 * g]),
                            f32x4{Wm[16 * s + 4 * g][col], Wm[16 * s + 4 * g + 1][col], Wm[16 * s + 4 * g + 2][col],
                                  Wm[16 * s + 4 * g + 3][col]});
#pragma unroll
            for (int r = 0; r < 4; ++r) Uc[u][r] = Us[4 * g + r][col] - acc[r];
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < NCT; ++u) {
            const int col = 16 * (wv + NW * u) + m;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Us[4 * g + r][col] = Uc[u][r];
                p.ub[(row0 + 4 * g + r) * D + col] = Uc[u][r];
            }
        }
        __syncthreads();
    }
    // A = (Q K^T) * M and dA = (dO U^T) * M: lane (g, n) holds [t = 4 g + r][i = n]
    f32x4 A = zero4(), dA = zero4();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        A = mma16(A, *reinterpret_cast<const f32x4 *>(&Qs[m][16 * s + 4 * g]),
                  *reinterpret_cast<const f32x4 *>(&Ks[m][16 * s + 4 * g]));
        dA = mma16(dA, *reinterpret_cast<const f32x4 *>(&Os[m][16 * s + 4 * g]),
                   *reinterpret_cast<const f32x4 *>(&Us[m][16 * s + 4 * g]));
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const bool keep = 4 * g + r >= m;  // key i = m not after query t
        A[r] = keep ? A[r] : 0.f;
        dA[r] = keep ? dA[r] : 0.f;
    }
    const float eti = et[m];
    if (wv == 0) {  // d_eta, the G-free part: sum_t dS[t][i] A[t][i]
        float x = dA[0] * A[0] + dA[1] * A[1] + dA[2] * A[2] + dA[3] * A[3];
        x += __shfl_xor(x, 16, 64);
        x += __shfl_xor(x, 32, 64);
        if (g == 0 && m < n) p.deta[tok0 + t0 + m] = x;
    }
    dA = dA * eti;  // dA H (column i scaled by eta_i)
    if (wv == 0)
#pragma unroll
        for (int r = 0; r < 4; ++r) dAs[4 * g + r][m] = dA[r];
    // S~ = H A^T dO (rows i), kept for dK and R_c and stored for the dependent pass
#pragma unroll
    for (int u = 0; u < NCT; ++u) {
        const int col = 16 * (wv + NW * u) + m;
        f32x4 sv = mma16(zero4(), A, f32x4{Os[4 * g][col], Os[4 * g + 1][col], Os[4 * g + 2][col], Os[4 * g + 3][col]});
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = et[4 * g + r] * sv[r];
            Ss[4 * g + r][col] = x;
            p.st[(row0 + 4 * g + r) * D + col] = x;
        }
    }
    __syncthreads();  // S~ rows and dA H complete
#pragma unroll
    for (int u = 0; u < NCT; ++u) {
        const int col = 16 * (wv + NW * u) + m;
        // dQ = dO W_c^T + dA K
        f32x4 dq = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s)
            dq = mma16(dq, *reinterpret_cast<const f32x4 *>(&Os[m][16 * s + 4 * g]),
                       *reinterpret_cast<const f32x4 *>(&Wm[col][16 * s + 4 * g]));
        dq = mma16(dq, *reinterpret_cast<const f32x4 *>(&dAs[m][4 * g]),
                   f32x4{Ks[4 * g][col], Ks[4 * g + 1][col], Ks[4 * g + 2][col], Ks[4 * g + 3][col]});
        // dK part = dA^T Q [- S~ W_c^T]
        f32x4 dk = mma16(zero4(), dA, f32x4{Qs[4 * g][col], Qs[4 * g + 1][col], Qs[4 * g + 2][col], Qs[4 * g + 3][col]});
        if constexpr (MSE) {
            f32x4 sw = zero4();
#pragma unroll
            for (int s = 0; s < NS; ++s)
                sw = mma16(sw, *reinterpret_cast<const f32x4 *>(&Ss[m][16 * s + 4 * g]),
                           *reinterpret_cast<const f32x4 *>(&Wm[col][16 * s + 4 * g]));
            dk -= sw;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * g + r;
            if (i < n) stf<E>(p.dq, (tok0 + t0 + i) * D + col, dq[r]);
            p.dkl[(row0 + i) * D + col] = dk[r];
        }
        // R_c = Q^T dO [- K^T S~], rows a = 16 ra + 4 g + r of this column tile
        float *R = p.rc + cb * D * D;
        const f32x4 ob = f32x4{Os[4 * g][col], Os[4 * g + 1][col], Os[4 * g + 2][col], Os[4 * g + 3][col]};
        const f32x4 sb = f32x4{Ss[4 * g][col], Ss[4 * g + 1][col], Ss[4 * g + 2][col], Ss[4 * g + 3][col]};
#pragma unroll
        for (int ra = 0; ra < NS; ++ra) {
            const int a = 16 * ra + m;
            f32x4 rv = mma16(zero4(), f32x4{Qs[4 * g][a], Qs[4 * g + 1][a], Qs[4 * g + 2][a], Qs[4 * g + 3][a]}, ob);
            if constexpr (MSE)
                rv -= mma16(zero4(), f32x4{Ks[4 * g][a], Ks[4 * g + 1][a], Ks[4 * g + 2][a], Ks[4 * g + 3][a]}, sb);
#pragma unroll
            for (int r = 0; r < 4; ++r) R[(long)(16 * ra + 4 * g + r) * D + col] = rv[r];
        }
    }
}

// Parallel pass 4 on the matrix cores (fp32 16x16x4 MFMA): one workgroup per
// (head, chunk, group of up to DEP_TPW 16-token tiles of the chunk), four
// waves, wave w owning column tiles w, w + 4, ... of the D / 16.  G_{c+1} and
// W_c are staged once per workgroup, rows padded by 4 floats; per tile
//     KG = K G                          (B: columns of G, 4 scalar reads)
//     dV = S~ + H KG,  d_eta += rowsum(KG * U)
//     dK = part + H (U G^T [- KG W_c^T]) (B: rows of G and W_c, 16-byte reads)
// with U and KG exchanged as token rows through LDS (their accumulator order
// is not the A-operand order).  In the update-then-apply order there are no
// G-free parts and U is V [- K W_c] (computed here).
template <int D, typename E, bool MSE>
__global__ __launch_bounds__(64 * PW<D>) void lbw_dep_m(LinBwdParams p)
{
    constexpr int NS = D / 16, NW = PW<D>, NT = 64 * NW, NCT = NS / NW, P = D + 4;
    __shared__ __align__(16) float Gm[D][P];
    __shared__ __align__(16) float Wm[MSE ? D : 1][P];
    __shared__ __align__(16) float Us[WT][P];
    __shared__ __align__(16) float KGs[WT][P];
    __shared__ float dpart[NW][WT];
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tpc = p.tpc, gpc = (tpc + DEP_TPW - 1) / DEP_TPW;
    const int h = blockIdx.x / (p.nchunks * gpc), rem = blockIdx.x % (p.nchunks * gpc);
    const int ch = rem / gpc, grp = rem % gpc;
    const int chunk = tpc * WT;
    const int tstart = ch * chunk + grp * DEP_TPW * WT;
    const int tend = min(min(tstart + DEP_TPW * WT, (ch + 1) * chunk), p.T);
    const long tok0 = (long)h * p.T;
    const long cb = (long)h * p.nchunks + ch;
    const bool nc = p.order == 1;
    {
        stage_mats<D, P, MSE, NT>(Gm, p.gnext + cb * D * D, Wm, p.states + cb * D * D, tid);
    }
    for (int t0 = tstart; t0 < tend; t0 += WT) {
        const int n = min(WT, tend - t0);
        const long row0 = (long)h * p.rstride + t0;  // the tile's rows in the per-token buffers
        // U rows: the forward's residuals (MSE, stored by the local pass) or V
        for (int e = tid; e < WT * D / 4; e += NT) {
            const int i = e / (D / 4), c = 4 * (e % (D / 4));
            const int ic = min(i, n - 1);
            const f32x4 x = (MSE && !nc) ? *reinterpret_cast<const f32x4 *>(p.ub + (row0 + ic) * D + c)
                                         : ld4f<E>(p.v, (tok0 + t0 + ic) * D + c);
            *reinterpret_cast<f32x4 *>(&Us[i][c]) = i < n ? x : zero4();
        }
        f32x4 Ka[NS];  // A operand: K[t0 + m][16 s + 4 g + j]
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const f32x4 x = ld4f<E>(p.k, (tok0 + t0 + min(m, n - 1)) * D + 16 * s + 4 * g);
            Ka[s] = m < n ? x : zero4();
        }
        f32x4 e4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = p.eta[tok0 + t0 + min(4 * g + r, n - 1)];
            e4[r] = 4 * g + r < n ? x : 0.f;
        }
        __syncthreads();  // G, W_c (first tile) and U staged
        if (MSE && nc) {  // U = V - K W_c
            f32x4 Uc[NCT];
#pragma unroll
            for (int u = 0; u < NCT; ++u) {
                const int ct = wv + NW * u;
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    acc = mma16(acc, Ka[s],
                                f32x4{Wm[16 * s + 4 * g][16 * ct + m], Wm[16 * s + 4 * g + 1][16 * ct + m],
                                      Wm[16 * s + 4 * g + 2][16 * ct + m], Wm[16 * s + 4 * g + 3][16 * ct + m]});
#pragma unroll
                for (int r = 0; r < 4; ++r) Uc[u][r] = Us[4 * g + r][16 * ct + m] - acc[r];
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < NCT; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) Us[4 * g + r][16 * (wv + NW * u) + m] = Uc[u][r];
            __syncthreads();
        }
        // KG, dV, this wave's part of d_eta; KG rows to LDS
        float dp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NCT; ++u) {
            const int ct = wv + NW * u, col = 16 * ct + m;
            f32x4 kg = zero4();
#pragma unroll
            for (int s = 0; s < NS; ++s)
                kg = mma16(kg, Ka[s],
                           f32x4{Gm[16 * s + 4 * g][col], Gm[16 * s + 4 * g + 1][col], Gm[16 * s + 4 * g + 2][col],
                                 Gm[16 * s + 4 * g + 3][col]});
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * g + r;
                dp[r] += kg[r] * Us[i][col];
                KGs[i][col] = kg[r];
                if (i < n)
                    stf<E>(p.dv, (tok0 + t0 + i) * D + col, (nc ? 0.f : p.st[(row0 + i) * D + col]) + e4[r] * kg[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) dp[r] += __shfl_xor(dp[r], o, 64);
            if (m == 0) dpart[wv][4 * g + r] = dp[r];
        }
        __syncthreads();  // KG rows and the d_eta parts
        if (tid < n) {
            const long te = tok0 + t0 + tid;
            float x = dpart[0][tid];
#pragma unroll
            for (int w = 1; w < NW; ++w) x += dpart[w][tid];
            p.deta[te] = (nc ? 0.f : p.deta[te]) + x;
        }
        // dK = part + H (U G^T [- KG W_c^T])
#pragma unroll
        for (int u = 0; u < NCT; ++u) {
            const int ct = wv + NW * u, col = 16 * ct + m;
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < NS; ++s)
                acc = mma16(acc, *reinterpret_cast<const f32x4 *>(&Us[m][16 * s + 4 * g]),
                            *reinterpret_cast<const f32x4 *>(&Gm[col][16 * s + 4 * g]));
            if constexpr (MSE) {
                f32x4 acc2 = zero4();
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    acc2 = mma16(acc2, *reinterpret_cast<const f32x4 *>(&KGs[m][16 * s + 4 * g]),
                                 *reinterpret_cast<const f32x4 *>(&Wm[col][16 * s + 4 * g]));
                acc -= acc2;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * g + r;
                if (i < n)
                    stf<E>(p.dk, (tok0 + t0 + i) * D + col, (nc ? 0.f : p.dkl[(row0 + i) * D + col]) + e4[r] * acc[r]);
            }
        }
        __syncthreads();  // the next tile overwrites U, KG and the d_eta parts
    }
}

// ---------------------------------------------------------------------------
// Chunks of more than 32 tokens (causal order).  The chunk's B x B products
// (A = (Q K^T) * M and dS = (dO U^T) * M) are taken 16 x 16 blocks at a time:
// the wave of tile I walks the tiles of its chunk after I (for the columns i
// of A and dS that I owns: S~, d_eta's first part, the dA^T Q part of dK) and
// before I (for the rows t it owns: dA K in dQ).  The residuals U of every
// tile come first (they are read by the other tiles' waves), R_c last (a sum
// over the whole chunk).
// ---------------------------------------------------------------------------

// U = V - K W_c (MSE) of 16-token tiles on the matrix cores: one workgroup per
// (head, chunk, group of up to DEP_TPW tiles), W_c staged once, wave w owning
// column tiles w, w + 4, ...
template <int D, typename E>
__global__ __launch_bounds__(256) void lbw_u_m(LinBwdParams p)
{
    constexpr int NS = D / 16, NCT = D / 64, P = D + 4;
    __shared__ __align__(16) float Wm[D][P];
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tpc = p.tpc, gpc = (tpc + DEP_TPW - 1) / DEP_TPW;
    const int h = blockIdx.x / (p.nchunks * gpc), rem = blockIdx.x % (p.nchunks * gpc);
    const int ch = rem / gpc, grp = rem % gpc;
    const int tstart = ch * tpc * WT + grp * DEP_TPW * WT;
    const int tend = min(min(tstart + DEP_TPW * WT, (ch + 1) * tpc * WT), p.T);
    const long tok0 = (long)h * p.T;
    {
        stage_mats<D, P, false>(Wm, p.states + ((long)h * p.nchunks + ch) * D * D, Wm, nullptr, tid);
    }
    __syncthreads();
    for (int t0 = tstart; t0 < tend; t0 += WT) {
        const int n = min(WT, tend - t0);
        const long row0 = (long)h * p.rstride + t0;
        f32x4 Ka[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const f32x4 x = ld4f<E>(p.k, (tok0 + t0 + min(m, n - 1)) * D + 16 * s + 4 * g);
            Ka[s] = m < n ? x : zero4();
        }
#pragma unroll
        for (int u = 0; u < NCT; ++u) {
            const int col = 16 * (wv + 4 * u) + m;
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < NS; ++s)
                acc = mma16(acc, Ka[s],
                            f32x4{Wm[16 * s + 4 * g][col], Wm[16 * s + 4 * g + 1][col], Wm[16 * s + 4 * g + 2][col],
                                  Wm[16 * s + 4 * g + 3][col]});
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 4 * g + r;
                const float v = ldf<E>(p.v, (tok0 + t0 + min(i, n - 1)) * D + col);
                p.ub[(row0 + i) * D + col] = i < n ? v - acc[r] : 0.f;
            }
        }
    }
}

// R_c = Q^T dO [- K^T S~] over a whole chunk on the matrix cores: one
// workgroup per (head, chunk), wave w owning column tiles w, w + 4, ... and
// every row tile; the chunk's 16-token tiles are staged in LDS one at a time
// (the next one loaded into registers meanwhile).
template <int D, typename E, bool MSE>
__global__ __launch_bounds__(256) void lbw_rc_m(LinBwdParams p)
{
    constexpr int NS = D / 16, NCT = D / 64, P = D + 4;
    constexpr int NL = WT * D / 4 / 256;  // 4-element pieces per thread and tensor
    __shared__ __align__(16) float Qs[WT][P], Os[WT][P], Ks[MSE ? WT : 1][P], Ss[MSE ? WT : 1][P];
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = blockIdx.x / p.nchunks, c = blockIdx.x % p.nchunks;
    const long tok0 = (long)h * p.T;
    const int t0 = c * p.tpc * WT, t1 = min(p.T, t0 + p.tpc * WT);
    f32x4 acc[NS][NCT];
#pragma unroll
    for (int ra = 0; ra < NS; ++ra)
#pragma unroll
        for (int u = 0; u < NCT; ++u) acc[ra][u] = zero4();
    f32x4 rq[NL], ro[NL], rk[MSE ? NL : 1], rs[MSE ? NL : 1];
    auto load = [&](int s0) {
        const int n = min(WT, t1 - s0);
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int e = tid + 256 * k, i = e / (D / 4), col = 4 * (e % (D / 4));
            const int ic = min(i, n - 1);
            const bool ok = i < n;
            const long gi = (tok0 + s0 + ic) * D + col;
            const f32x4 q = ld4f<E>(p.q, gi), o = ld4f<E>(p.dout, gi);
            rq[k] = ok ? q : zero4();
            ro[k] = ok ? o : zero4();
            if constexpr (MSE) {
                const f32x4 kk = ld4f<E>(p.k, gi);
                const f32x4 ss = *reinterpret_cast<const f32x4 *>(p.st + ((long)h * p.rstride + s0 + ic) * D + col);
                rk[k] = ok ? kk : zero4();
                rs[k] = ok ? ss : zero4();
            }
        }
    };
    load(t0);
    for (int s0 = t0; s0 < t1; s0 += WT) {
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int e = tid + 256 * k, i = e / (D / 4), col = 4 * (e % (D / 4));
            *reinterpret_cast<f32x4 *>(&Qs[i][col]) = rq[k];
            *reinterpret_cast<f32x4 *>(&Os[i][col]) = ro[k];
            if constexpr (MSE) {
                *reinterpret_cast<f32x4 *>(&Ks[i][col]) = rk[k];
                *reinterpret_cast<f32x4 *>(&Ss[i][col]) = rs[k];
            }
        }
        __syncthreads();
        if (s0 + WT < t1) load(s0 + WT);
#pragma unroll
        for (int u = 0; u < NCT; ++u) {
            const int col = 16 * (wv + 4 * u) + m;
            const f32x4 ob = f32x4{Os[4 * g][col], Os[4 * g + 1][col], Os[4 * g + 2][col], Os[4 * g + 3][col]};
            f32x4 sb = zero4();
            if constexpr (MSE) sb = -f32x4{Ss[4 * g][col], Ss[4 * g + 1][col], Ss[4 * g + 2][col], Ss[4 * g + 3][col]};
#pragma unroll
            for (int ra = 0; ra < NS; ++ra) {
                const int a = 16 * ra + m;
                acc[ra][u] = mma16(acc[ra][u], f32x4{Qs[4 * g][a], Qs[4 * g + 1][a], Qs[4 * g + 2][a], Qs[4 * g + 3][a]}, ob);
                if constexpr (MSE)
                    acc[ra][u] =
                        mma16(acc[ra][u], f32x4{Ks[4 * g][a], Ks[4 * g + 1][a], Ks[4 * g + 2][a], Ks[4 * g + 3][a]}, sb);
            }
        }
        __syncthreads();
    }
    float *R = p.rc + ((long)h * p.nchunks + c) * D * D;
#pragma unroll
    for (int u = 0; u < NCT; ++u)
#pragma unroll
        for (int ra = 0; ra < NS; ++ra)
#pragma unroll
            for (int r = 0; r < 4; ++r) R[(long)(16 * ra + 4 * g + r) * D + 16 * (wv + 4 * u) + m] = acc[ra][u][r];
}

// Everything of the tiles of a chunk that needs no G, on the matrix cores:
// one workgroup per (head, chunk, group of 4 tiles), one wave per tile I
// (K_I, U_I and dO_I held as fragments, its S~, dK part and dQ as
// accumulators over all columns).  The chunk's other tiles J are staged in
// LDS once for the four waves: first J >= I (Q_J and dO_J: A[t][i] = q_t . k_i
// and dS[t][i] = dO_t . u_i for t in J, i in I, giving S~ += A^T dO_J,
// dK += dS^T Q_J and d_eta), then J <= I (U_J and K_J: dA^T[s][t] = eta_s
// u_s . dO_t for s in J, t in I, giving dQ += dA K_J).  Last, dQ += dO_I W_c^T
// and dK = H dK [- S~ W_c^T] with W_c read from L2.
template <int D, typename E, bool MSE>
__global__ __launch_bounds__(256) void lbw_local_tiled_m(LinBwdParams p)
{
    constexpr int NS = D / 16, P = D + 4;
    constexpr int NL = WT * D / 4 / 256;  // 4-element pieces per thread and tensor of a J tile
    __shared__ __align__(16) float XJ[WT][P], YJ[WT][P];
    __shared__ __align__(16) float SW[4][WT][P];  // each wave's S~ rows
    __shared__ float etJ[WT];
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tpc = p.tpc, gpc = (tpc + 3) / 4;
    const int h = blockIdx.x / (p.nchunks * gpc), rem = blockIdx.x % (p.nchunks * gpc);
    const int ch = rem / gpc, grp = rem % gpc;
    const int J0 = ch * tpc, J1 = min(J0 + tpc, p.nwt);  // the chunk's tiles [J0, J1)
    const int Imin = J0 + 4 * grp, Imax = min(Imin + 3, J1 - 1);
    if (Imin >= J1) return;  // a group past the end of a short last chunk (uniform: before any barrier)
    const int I = Imin + wv;
    const bool valid = I <= Imax;
    const long tok0 = (long)h * p.T, hrow = (long)h * p.rstride;
    const int c0 = min(I, Imax) * WT, n = min(WT, p.T - c0);
    // this wave's tile: K, U (or V) and dO rows as fragments, eta of its rows
    f32x4 KIf[NS], UIf[NS], OIf[NS], etI;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const long gi = (tok0 + c0 + min(m, n - 1)) * D + 16 * s + 4 * g;
        const f32x4 kk = ld4f<E>(p.k, gi), oo = ld4f<E>(p.dout, gi);
        const f32x4 uu = MSE ? *reinterpret_cast<const f32x4 *>(p.ub + (hrow + c0 + min(m, n - 1)) * D + 16 * s + 4 * g)
                             : ld4f<E>(p.v, gi);
        KIf[s] = m < n ? kk : zero4();
        UIf[s] = m < n ? uu : zero4();
        OIf[s] = m < n ? oo : zero4();
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float x = p.eta[tok0 + c0 + min(4 * g + r, n - 1)];
        etI[r] = 4 * g + r < n ? x : 0.f;
    }
    f32x4 sv[NS], dk[NS], dq[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) sv[s] = dk[s] = dq[s] = zero4();
    float de = 0.f;
    // J tiles go global -> registers one tile ahead
    f32x4 rx[NL], ry[NL];
    float re = 0.f;
    auto load = [&](int J, bool after) {
        const int cj = J * WT, nj = min(WT, p.T - cj);
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int e = tid + 256 * k, i = e / (D / 4), col = 4 * (e % (D / 4));
            const int ic = min(i, nj - 1);
            const long gi = (tok0 + cj + ic) * D + col;
            f32x4 x, y;
            if (after) {
                x = ld4f<E>(p.q, gi);
                y = ld4f<E>(p.dout, gi);
            } else {
                x = MSE ? *reinterpret_cast<const f32x4 *>(p.ub + (hrow + cj + ic) * D + col) : ld4f<E>(p.v, gi);
                y = ld4f<E>(p.k, gi);
            }
            rx[k] = i < nj ? x : zero4();
            ry[k] = i < nj ? y : zero4();
        }
        if (!after && tid < WT) re = tid < nj ? p.eta[tok0 + cj + tid] : 0.f;
    };
    auto put = [&]() {
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int e = tid + 256 * k, i = e / (D / 4), col = 4 * (e % (D / 4));
            *reinterpret_cast<f32x4 *>(&XJ[i][col]) = rx[k];
            *reinterpret_cast<f32x4 *>(&YJ[i][col]) = ry[k];
        }
        if (tid < WT) etJ[tid] = re;
    };
    // J >= I
    load(Imin, true);
    for (int J = Imin; J < J1; ++J) {
        put();
        __syncthreads();
        if (J + 1 < J1)
            load(J + 1, true);
        else
            load(J0, false);
        if (valid && J >= I) {
            f32x4 A = zero4(), dS = zero4();
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                A = mma16(A, *reinterpret_cast<const f32x4 *>(&XJ[m][16 * s + 4 * g]), KIf[s]);
                dS = mma16(dS, *reinterpret_cast<const f32x4 *>(&YJ[m][16 * s + 4 * g]), UIf[s]);
            }
            if (J == I) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    A[r] = 4 * g + r >= m ? A[r] : 0.f;
                    dS[r] = 4 * g + r >= m ? dS[r] : 0.f;
                }
            }
            de += dS[0] * A[0] + dS[1] * A[1] + dS[2] * A[2] + dS[3] * A[3];
#pragma unroll
            for (int ct = 0; ct < NS; ++ct) {
                const int col = 16 * ct + m;
                sv[ct] = mma16(sv[ct], A, f32x4{YJ[4 * g][col], YJ[4 * g + 1][col], YJ[4 * g + 2][col], YJ[4 * g + 3][col]});
                dk[ct] = mma16(dk[ct], dS, f32x4{XJ[4 * g][col], XJ[4 * g + 1][col], XJ[4 * g + 2][col], XJ[4 * g + 3][col]});
            }
        }
        __syncthreads();
    }
    // J <= I
    for (int J = J0; J <= Imax; ++J) {
        put();
        __syncthreads();
        if (J + 1 <= Imax) load(J + 1, false);
        if (valid && J <= I) {
            f32x4 dAT = zero4();  // lane (g, n): dA^T[s = 4 g + r][t = n]
#pragma unroll
            for (int s = 0; s < NS; ++s) dAT = mma16(dAT, *reinterpret_cast<const f32x4 *>(&XJ[m][16 * s + 4 * g]), OIf[s]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = dAT[r] * etJ[4 * g + r];
                dAT[r] = (J < I || 4 * g + r <= m) ? x : 0.f;
            }
#pragma unroll
            for (int ct = 0; ct < NS; ++ct) {
                const int col = 16 * ct + m;
                dq[ct] = mma16(dq[ct], dAT, f32x4{YJ[4 * g][col], YJ[4 * g + 1][col], YJ[4 * g + 2][col], YJ[4 * g + 3][col]});
            }
        }
        __syncthreads();
    }
    if (!valid) return;
    // S~ = H A^T dO: stored, and kept as rows for S~ W_c^T
#pragma unroll
    for (int ct = 0; ct < NS; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = etI[r] * sv[ct][r];
            SW[wv][4 * g + r][16 * ct + m] = x;
            p.st[(hrow + c0 + 4 * g + r) * D + 16 * ct + m] = x;
        }
    de += __shfl_xor(de, 16, 64);
    de += __shfl_xor(de, 32, 64);
    if (g == 0 && m < n) p.deta[tok0 + c0 + m] = de;
    const float *Wc = p.states + ((long)h * p.nchunks + ch) * D * D;
#pragma unroll
    for (int ct = 0; ct < NS; ++ct) {
        const int col = 16 * ct + m;
        f32x4 fq = dq[ct], sk = zero4();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const f32x4 wf = *reinterpret_cast<const f32x4 *>(Wc + (long)col * D + 16 * s + 4 * g);
            fq = mma16(fq, OIf[s], wf);
            if constexpr (MSE) sk = mma16(sk, *reinterpret_cast<const f32x4 *>(&SW[wv][m][16 * s + 4 * g]), wf);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 4 * g + r;
            if (i < n) stf<E>(p.dq, (tok0 + c0 + i) * D + col, fq[r]);
            p.dkl[(hrow + c0 + i) * D + col] = etI[r] * dk[ct][r] - sk[r];
        }
    }
}

// Update-then-apply order on the matrix cores.  The apply's adjoint G_final =
// dW_final + Q^T dO: one workgroup per (head, 16 columns), its four waves
// taking a quarter of the queries each (16-token tiles staged in the wave's
// own LDS, the walk's fragments: Q^T as the A operand, dO in accumulator
// order as B), the four partial sums added in a fixed order at the end.
template <int D, typename E>
__global__ __launch_bounds__(256) void lbw_nc_g_m(LinBwdParams p)
{
    constexpr int NS = D / 16;
    __shared__ WalkTile<D> tiles[4];
    __shared__ __align__(16) f32x4 part[4][NS][64];
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int h = blockIdx.x / NS, j0 = (blockIdx.x % NS) * 16;
    const long q0 = (long)h * p.Tq;
    const int ntq = (p.Tq + WT - 1) / WT, per = (ntq + 3) / 4;
    const int ta = wv * per, tb = min(ntq, ta + per);
    f32x4 X[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) X[s] = zero4();
    WalkK<D, E> nk;
    WalkCol<E> on;
    if (ta < tb) {
        nk.load(p.q, q0, ta * WT, p.Tq, lane);
        on = walk_col4<E>(p.dout, q0, ta * WT, p.Tq, D, j0 + m, g);
    }
    for (int t = ta; t < tb; ++t) {
        nk.put(tiles[wv], lane, p.Tq - t * WT);
        const f32x4 oc = walk_f32(on, t * WT, p.Tq, g);
        const int tn = min(t + 1, tb - 1);  // clamped: no branch around the loads
        nk.load(p.q, q0, tn * WT, p.Tq, lane);
        on = walk_col4<E>(p.dout, q0, tn * WT, p.Tq, D, j0 + m, g);
#pragma unroll
        for (int s = 0; s < NS; ++s) X[s] = mma16(X[s], walk_cols<D>(tiles[wv], s, m, g), oc);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) part[wv][s][lane] = X[s];
    __syncthreads();
    if (wv == 0) {
        f32x4 Gf[NS];
        if (p.dwf)
            slice_load<NS>(Gf, p.dwf + (long)h * D * D + j0, D, g, m);
        else
            slice_identity<NS>(Gf, j0, g, m, false);
#pragma unroll
        for (int s = 0; s < NS; ++s) Gf[s] += ((part[0][s][lane] + part[1][s][lane]) + part[2][s][lane]) + part[3][s][lane];
        slice_store<NS>(p.ginit + (long)h * D * D + j0, Gf, D, g, m);
    }
}

// ... and dQ = dO W_final^T: one workgroup per (head, 64 queries), W_final
// staged in LDS, wave w owning column tiles w, w + 4, ...
template <int D, typename E>
__global__ __launch_bounds__(256) void lbw_nc_dq_m(LinBwdParams p)
{
    constexpr int NS = D / 16, NCT = D / 64, P = D + 4;
    __shared__ __align__(16) float Wm[D][P];
    const int tid = threadIdx.x, lane = tid & 63, m = lane & 15, g = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nqt = (p.Tq + 63) / 64;
    const int h = blockIdx.x / nqt, tq0 = (blockIdx.x % nqt) * 64;
    const long q0 = (long)h * p.Tq;
    stage_mats<D, P, false>(Wm, p.wfinal + (long)h * D * D, Wm, nullptr, tid);
    __syncthreads();
    for (int t0 = tq0; t0 < min(tq0 + 64, p.Tq); t0 += WT) {
        const int n = min(WT, p.Tq - t0);
        f32x4 Oa[NS];  // A operand: dO[t0 + m][16 s + 4 g + j]
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const f32x4 x = ld4f<E>(p.dout, (q0 + t0 + min(m, n - 1)) * D + 16 * s + 4 * g);
            Oa[s] = m < n ? x : zero4();
        }
#pragma unroll
        for (int u = 0; u < NCT; ++u) {
            const int col = 16 * (wv + 4 * u) + m;
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < NS; ++s) acc = mma16(acc, Oa[s], *reinterpret_cast<const f32x4 *>(&Wm[col][16 * s + 4 * g]));
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * g + r < n) stf<E>(p.dq, (q0 + t0 + 4 * g + r) * D + col, acc[r]);
        }
    }
}

}  // namespace

// Segments of the serial passes.  A walk step (one 16-token tile) costs about
// the same in every wave, and one wave per SIMD runs at full speed (a second
// one shares its matrix core), so the time goes as the segment's tiles times
// the rounds of 1024 waves the maps (2 NH (S - 1) d / 16 waves) and the walks
// (NH S d / 16) take, plus the chain; S = 1 is the plain walk.  The smallest
// estimate wins (ties: fewer segments), with at least 64 tokens per segment.
static void seg_plan(int NH, int nch, int chunk, int d, int &nseg, int &seg_chunks)
{
    const long slots = 1024;
    const long cols = (long)NH * (d / CB);
    const int tpc = chunk / 16;
    const int min_chunks = max(1, 64 / chunk);
    const int most = max(1, min(64, nch / min_chunks));
    long best = -1;
    nseg = 1;
    seg_chunks = nch;
    for (int s = 1; s <= most; ++s) {
        const int sc = (nch + s - 1) / s, ns = (nch + sc - 1) / sc;
        const long rounds = (2 * cols * (ns - 1) + slots - 1) / slots + (cols * ns + slots - 1) / slots;
        const long est = (long)sc * tpc * rounds + 2L * (ns - 1);
        if (best < 0 || est < best) {
            best = est;
            nseg = ns;
            seg_chunks = sc;
        }
    }
}

#ifndef TTT_LBW_TILED_UNIT
size_t linear_bwd_workspace(int NH, int Tkv, int d, int chunk)
{
    const size_t nch = (Tkv + chunk - 1) / chunk;
    int nseg = 1, segc = 1;
    seg_plan(NH, (int)nch, chunk, d, nseg, segc);
    // states, G_{c+1}, R_c (d x d per chunk) and U, S~, dK part (chunk x d per chunk), plus
    // the final state and dL/dW_final (update-then-apply order), plus the
    // segment maps (d x 2d) and starts (d x d), fp32
    return (size_t)NH *
           (nch * (3 * (size_t)d * d + 3 * (size_t)chunk * d) + 2 * (size_t)d * d + (size_t)nseg * 3 * d * d) *
           sizeof(float);
}
#endif

// The two serial recursions, each as segment maps, chain, walks.
// (one wave per (head, segment, 16 columns), four waves a workgroup: the
// column counts D / 16 and 2 D / 16 are multiples of four)
template <int D, typename E>
static void lbw_serial_states(const LinBwdParams &p, int NH, hipStream_t st)
{
    const dim3 b(256);
    constexpr int NC = D / CB / 4;  // workgroups per (head, segment) and D columns
    if (p.nseg > 1) {
        lbw_states_m<D, E><<<dim3(NH * (p.nseg - 1) * 2 * NC), b, 0, st>>>(p, 1);
        lbw_chain_m<D><<<dim3(NH * NC), b, 0, st>>>(p, 0);
    }
    lbw_states_m<D, E><<<dim3(NH * p.nseg * NC), b, 0, st>>>(p, 0);
}

template <int D, typename E>
static void lbw_serial_grad(const LinBwdParams &p, int NH, hipStream_t st)
{
    const dim3 b(256);
    constexpr int NC = D / CB / 4;
    if (p.nseg > 1) {
        if (p.loss == 1)
            lbw_grad_m<D, E, true><<<dim3(NH * (p.nseg - 1) * 2 * NC), b, 0, st>>>(p, 1);
        else
            lbw_grad_m<D, E, false><<<dim3(NH * (p.nseg - 1) * 2 * NC), b, 0, st>>>(p, 1);
        lbw_chain_m<D><<<dim3(NH * NC), b, 0, st>>>(p, 1);
    }
    if (p.loss == 1)
        lbw_grad_m<D, E, true><<<dim3(NH * p.nseg * NC), b, 0, st>>>(p, 0);
    else
        lbw_grad_m<D, E, false><<<dim3(NH * p.nseg * NC), b, 0, st>>>(p, 0);
}

// The dependent pass: one workgroup per (head, chunk, group of DEP_TPW tiles).
template <int D, typename E>
static void lbw_dep_launch(const LinBwdParams &p, int NH, hipStream_t st)
{
    const dim3 grid(NH * p.nchunks * ((p.tpc + DEP_TPW - 1) / DEP_TPW));
    if (p.loss == 1)
        lbw_dep_m<D, E, true><<<grid, dim3(64 * PW<D>), 0, st>>>(p);
    else
        lbw_dep_m<D, E, false><<<grid, dim3(64 * PW<D>), 0, st>>>(p);
}

template <int D, typename E>
static void lbw_run(const LinBwdParams &p, int NH, hipStream_t st)
{
    const dim3 b(256);
    lbw_serial_states<D, E>(p, NH, st);
    if (p.order == 0) {
        if (p.loss == 1)
            lbw_local_m<D, E, true><<<dim3(NH * p.nchunks), dim3(64 * PW<D>), 0, st>>>(p);
        else
            lbw_local_m<D, E, false><<<dim3(NH * p.nchunks), dim3(64 * PW<D>), 0, st>>>(p);
    } else {
        lbw_nc_g_m<D, E><<<dim3(NH * (D / CB)), b, 0, st>>>(p);
        if (p.Tq > 0) lbw_nc_dq_m<D, E><<<dim3(NH * ((p.Tq + 63) / 64)), b, 0, st>>>(p);
    }
    lbw_serial_grad<D, E>(p, NH, st);
    lbw_dep_launch<D, E>(p, NH, st);
}

// Chunks of 16 k tokens, k > 1: the serial and dependent
// passes step over 16-token tiles (snapshotting the chunk-start state and
// G_{c+1}), the G-free terms run tile against tile.
template <int D, typename E>
static void lbw_run_tiled(const LinBwdParams &p, int NH, hipStream_t st)
{
    const dim3 b(256);
    lbw_serial_states<D, E>(p, NH, st);
    if (p.order == 0) {
        const int ngrp = NH * p.nchunks * ((p.tpc + 3) / 4);
        if (p.loss == 1) {
            lbw_u_m<D, E><<<dim3(NH * p.nchunks * ((p.tpc + DEP_TPW - 1) / DEP_TPW)), b, 0, st>>>(p);
            lbw_local_tiled_m<D, E, true><<<dim3(ngrp), b, 0, st>>>(p);
            lbw_rc_m<D, E, true><<<dim3(NH * p.nchunks), b, 0, st>>>(p);
        } else {
            lbw_local_tiled_m<D, E, false><<<dim3(ngrp), b, 0, st>>>(p);
            lbw_rc_m<D, E, false><<<dim3(NH * p.nchunks), b, 0, st>>>(p);
        }
    } else {
        lbw_nc_g_m<D, E><<<dim3(NH * (D / CB)), b, 0, st>>>(p);
        if (p.Tq > 0) lbw_nc_dq_m<D, E><<<dim3(NH * ((p.Tq + 63) / 64)), b, 0, st>>>(p);
    }
    lbw_serial_grad<D, E>(p, NH, st);
    lbw_dep_launch<D, E>(p, NH, st);
}

static LinBwdParams lbw_params(int NH, int Tq, int Tkv, int d, int chunk, int loss, int order,
                               const void *q, const void *k, const void *v, const float *eta, const float *w0,
                               const void *dout, const float *dwf, void *dq, void *dk, void *dv, float *deta,
                               float *dw0, void *ws)
{
    const int nch = (Tkv + chunk - 1) / chunk;
    float *base = static_cast<float *>(ws);
    const size_t dd = (size_t)NH * nch * d * d, bd = (size_t)NH * nch * chunk * d;
    float *tail = base + 3 * dd + 3 * bd;
    LinBwdParams p{q, k, v, dout, eta, w0, dwf, dq, dk, dv, deta, dw0, base, base + dd,
                   base + 2 * dd, base + 3 * dd, base + 3 * dd + bd, base + 3 * dd + 2 * bd, Tkv,
                   nch, loss, order, Tq, tail, tail + (size_t)NH * d * d};
    p.rstride = (long)nch * chunk;
    seg_plan(NH, nch, chunk, d, p.nseg, p.seg_chunks);
    p.ssum = tail + 2 * (size_t)NH * d * d;
    p.sstart = p.ssum + (size_t)NH * p.nseg * 2 * d * d;
    p.tpc = chunk / 16;
    p.nwt = (Tkv + 15) / 16;
    return p;
}

// This source is compiled twice: the main unit runs 16-token chunks (a chunk
// is one tile) and the unit built with TTT_LBW_TILED_UNIT, whose MFMA
// operands are forced into VGPRs, runs chunks of several tiles (measured: the
// VGPR form is 3-18% faster on every multi-tile chunk size and 2-4% slower
// on 16-token chunks).
#ifdef TTT_LBW_TILED_UNIT
hipError_t linear_bwd_launch_tiled(int NH, int Tq, int Tkv, int d, int chunk, int loss, int order,
                                   int bf16, const void *q, const void *k, const void *v,
                                   const float *eta, const float *w0, const void *dout, const float *dwf,
                                   void *dq, void *dk, void *dv, float *deta, float *dw0, void *ws,
                                   hipStream_t st)
{
    const LinBwdParams p = lbw_params(NH, Tq, Tkv, d, chunk, loss, order, q, k, v, eta, w0, dout, dwf, dq, dk,
                                      dv, deta, dw0, ws);
    if (d == 128) {
        if (bf16) lbw_run_tiled<128, __bf16>(p, NH, st);
        else lbw_run_tiled<128, float>(p, NH, st);
    } else {
        if (bf16) lbw_run_tiled<64, __bf16>(p, NH, st);
        else lbw_run_tiled<64, float>(p, NH, st);
    }
    return hipGetLastError();
}
#else
hipError_t linear_bwd_launch(int NH, int Tq, int Tkv, int d, int chunk, int loss, int order,
                             int bf16, const void *q, const void *k, const void *v,
                             const float *eta, const float *w0, const void *dout, const float *dwf,
                             void *dq, void *dk, void *dv, float *deta, float *dw0, void *ws,
                             hipStream_t st)
{
    if (chunk != 16)  // several tiles a chunk
        return linear_bwd_launch_tiled(NH, Tq, Tkv, d, chunk, loss, order, bf16, q, k, v, eta, w0, dout, dwf,
                                       dq, dk, dv, deta, dw0, ws, st);
    const LinBwdParams p = lbw_params(NH, Tq, Tkv, d, chunk, loss, order, q, k, v, eta, w0, dout, dwf, dq, dk,
                                      dv, deta, dw0, ws);
    if (d == 128) {
        if (bf16) lbw_run<128, __bf16>(p, NH, st);
        else lbw_run<128, float>(p, NH, st);
    } else {
        if (bf16) lbw_run<64, __bf16>(p, NH, st);
        else lbw_run<64, float>(p, NH, st);
    }
    return hipGetLastError();
}
#endif

}  // namespace tttk
