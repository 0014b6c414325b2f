// TTT-Linear forward on gfx950: segment-parallel chunked gradient descent.
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
//    and O, so one wave owns a 16-column block of the state and runs its
//    chain with the state resident in MFMA accumulators (fp32), never
//    leaving registers across chunks.  A workgroup = one wave per column
//    block, sharing the token tiles it stages in LDS.
//  * Sub-blocks of 16 tokens.  A chunk of b tokens (b a multiple of 16) is
//    walked 16 tokens at a time: U uses the chunk-start snapshot of the
//    state, the inter-chunk read uses the running state (which already holds
//    the chunk's earlier sub-blocks), and the diagonal 16 x 16 block supplies
//    the rest of the causal intra-chunk term.  This is the same sum as the
//    b x b masked product, regrouped; work per token is O(d^2) for every b.
//  * Segments.  The chunk update is affine in the state,
//    W_{c+1} = (I - K_c^T H_c K_c) W_c + K_c^T H_c V_c, so a run of whole
//    chunks (a segment) is one affine map W -> W - P W + B.  Three kernels:
//      summary : every segment (but the last, causal) computes P and B from
//                its keys/values alone, all segments in parallel;
//      prefix  : per (head, column block), W_start(s+1) = W_s - P_s W_s + B_s;
//      replay  : every segment replays its chunks from W_start(s) and writes
//                its outputs; the last segment writes the final state.
//    For the inner-product loss P = 0 and the prefix is a running sum.
//  * Non-causal order: summary over all segments, prefix to W_final, then an
//    apply kernel O = Q W_final.
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
    float *wsB;     // [NH][Ssum][d][d]
    float *wsW;     // [NH][S + 1][d][d]: W_start(s); slot S = final state
    int NH, Tq, Tkv, chunk, seg_tokens, S, Ssum, seg_q, Sq;
};

// LDS image of one 16-token sub-block, token-major.  The fragments that need
// four consecutive tokens of one feature (K^T for the update, V in the
// accumulator layout) come from the same token-major tiles through gfx950's
// transposing LDS read for 16-bit data; the fp32 path keeps feature-major
// copies instead (kt, vt; rows padded to 20 elements).
template <typename E, int D> struct alignas(16) SubTile {
    static constexpr bool TR = sizeof(E) == 2;
    static constexpr int RP = D + (sizeof(E) == 2 ? 8 : 4);  // token-major row pitch
    static constexpr int FP = 20;                            // feature-major row pitch
    E qs[16][RP];
    E ks[16][RP];
    E vs[TR ? 16 : 1][RP];
    E kt[TR ? 1 : D][FP];
    E vt[TR ? 1 : D][FP];
    float eta[16];
};

// Transposing read (16-bit elements): within each group of 16 lanes, lane i
// slot j receives the element that lane 4j + i/4 would read at slot i%4.
// Lane (m, g) pointing at row 4g + m/4, column c0 + 4(m%4) of a token-major
// tile therefore receives tile[4g + j][c0 + m], j = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16 *p)
{
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
    const v4bf r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) v4bf *)((__attribute__((address_space(3))) char *)p));
    return __builtin_bit_cast(bf16x4, r);
}

// Fragment with k = token (4 consecutive tokens per lane) of column block
// `blk` of K or V: lane (m, g) gets X[4g + j][16 blk + m].
template <typename E, int D>
__device__ __forceinline__ typename Frag<E>::type tok_frag(const SubTile<E, D> &tl, bool from_v, int blk,
                                                           int m, int g)
{
    if constexpr (SubTile<E, D>::TR) {
        const E(*src)[SubTile<E, D>::RP] = from_v ? tl.vs : tl.ks;
        return lds_read_tr(&src[4 * g + (m >> 2)][16 * blk + 4 * (m & 3)]);
    } else {
        const E(*src)[SubTile<E, D>::FP] = from_v ? tl.vt : tl.kt;
        return load4<E>(&src[16 * blk + m][4 * g]);
    }
}

// Which tensors a kernel stages.
enum { STAGE_Q = 1, STAGE_K = 2, STAGE_V = 4, STAGE_E = 8 };

// Cooperative global -> register -> LDS loader with a ring of PD register
// slots.  Every thread runs the same instruction stream: for each staged
// tensor it moves CPT pieces of 4 consecutive features of one token (8 bytes
// bf16, 16 bytes fp32) and one eta value, with buffer loads: the per-thread
// byte offset is fixed, the sub-block's position is the scalar offset, and
// the buffer's extent ends at the segment's last token, so rows past it read
// as zero in hardware (no clamps, selects or 64-bit address arithmetic).
template <typename E, int D, int STAGE, int PD, int NT> struct Loader {
    typedef typename Vec4<E>::type V4;
    static constexpr bool LQ = STAGE & STAGE_Q, LK = STAGE & STAGE_K, LV = STAGE & STAGE_V,
                          LE = STAGE & STAGE_E;
    static constexpr int CPT = (4 * D) / NT;  // pieces per tensor per thread (16 rows x D/4 pieces)
    static_assert(CPT >= 1 && CPT * NT == 4 * D, "loader shape");
    int row[CPT], col[CPT];
    int voff[CPT];
    __amdgpu_buffer_rsrc_t rq, rk, rv, re;
    V4 vq[PD][CPT], vk[PD][CPT], vv[PD][CPT];
    float ve[PD];

    __device__ void init(int tid, const LinParams &p, int h, int T, int tend)
    {
        const size_t hoff = (size_t)h * T * D;
        const int bytes = tend * D * (int)sizeof(E);
        rq = __builtin_amdgcn_make_buffer_rsrc((void *)((const E *)p.q + hoff), (short)0, LQ ? bytes : 0, 0x00020000);
        rk = __builtin_amdgcn_make_buffer_rsrc((void *)((const E *)p.k + hoff), (short)0, LK ? bytes : 0, 0x00020000);
        rv = __builtin_amdgcn_make_buffer_rsrc((void *)((const E *)p.v + hoff), (short)0, LV ? bytes : 0, 0x00020000);
        re = __builtin_amdgcn_make_buffer_rsrc((void *)(LE ? p.eta + (size_t)h * T : p.eta), (short)0,
                                               LE ? tend * 4 : 0, 0x00020000);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int piece = tid + i * NT;
            row[i] = piece / (D / 4);
            col[i] = piece % (D / 4);
            voff[i] = (row[i] * D + 4 * col[i]) * (int)sizeof(E);
        }
    }

    __device__ __forceinline__ V4 bload(__amdgpu_buffer_rsrc_t r, int vo, int so)
    {
        if constexpr (sizeof(E) == 2)
            return __builtin_bit_cast(V4, __builtin_amdgcn_raw_buffer_load_b64(r, vo, so, 0));
        else
            return __builtin_bit_cast(V4, __builtin_amdgcn_raw_buffer_load_b128(r, vo, so, 0));
    }

    __device__ __forceinline__ void issue(int s, int tb0)
    {
        const int so = tb0 * D * (int)sizeof(E);
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            if (LQ) vq[s][i] = bload(rq, voff[i], so);
            if (LK) vk[s][i] = bload(rk, voff[i], so);
            if (LV) vv[s][i] = bload(rv, voff[i], so);
        }
        if (LE) ve[s] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(re, (int)(threadIdx.x & 15) * 4, tb0 * 4, 0));
    }

    // Write slot s to LDS.
    __device__ __forceinline__ void commit(int s, SubTile<E, D> &tl)
    {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int r = row[i], c = 4 * col[i];
            if (LQ) store4<E>(&tl.qs[r][c], vq[s][i]);
            if (LK) {
                store4<E>(&tl.ks[r][c], vk[s][i]);
                if constexpr (!SubTile<E, D>::TR) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) tl.kt[c + j][r] = vk[s][i][j];
                }
            }
            if (LV) {
                if constexpr (SubTile<E, D>::TR) {
                    store4<E>(&tl.vs[r][c], vv[s][i]);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) tl.vt[c + j][r] = vv[s][i][j];
                }
            }
        }
        if (LE) tl.eta[threadIdx.x & 15] = ve[s];
    }
};

// Drive the staged loop over the sub-blocks [t0, tend) of one head; `body` is
// called once per sub-block with the LDS tile and the sub-block's first token.
// The sub-block count is padded up to a multiple of PD so that the ring runs
// without branches; padded sub-blocks are all-zero (eta = 0) and change
// nothing, and bodies mask their stores with t < tend.
template <typename E, int D, int STAGE, int PD, int NT, typename Body>
__device__ __forceinline__ void run_subblocks(SubTile<E, D> *tiles, Loader<E, D, STAGE, PD, NT> &ld,
                                              int t0, int tend, Body &&body)
{
    static_assert(PD % 2 == 0, "PD must be even");
    const int nsb = (tend - t0 + 15) / 16;
    const int ngroups = (nsb + PD - 1) / PD;
#pragma unroll
    for (int s = 0; s < PD; ++s) ld.issue(s, t0 + 16 * s);
    ld.commit(0, tiles[0]);
    lds_barrier();
    for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
        for (int j = 0; j < PD; ++j) {
            const int sb = gi * PD + j;
            ld.issue(j, t0 + 16 * (sb + PD));
            ld.commit((j + 1) % PD, tiles[(j + 1) & 1]);
            body(tiles[j & 1], t0 + 16 * sb);
            lds_barrier();
        }
    }
}

template <typename E> __device__ __forceinline__ typename Frag<E>::type lds_frag(const E *p)
{
    return load4<E>(p);
}

// A state tile as MFMA operand.  bf16: hi = bf16(x), lo = bf16(x - hi), so
// products with exact bf16 inputs keep ~16 mantissa bits of the state (the
// state sits near the identity, where a single bf16 would lose the update).
// fp32: hi = x, lo unused.
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
// summary: P_s (MSE) and B_s of a segment.  The state X = [P | B] starts at 0
// and follows X <- X + K^T H (R - K X_c) over the segment's chunks, with
// R = [K | V] (MSE; A = I - P is the product of the chunk transitions) or
// R = V (inner product, where X_c does not enter).  Column blocks 0..ND-1 of
// X are P, ND..2ND-1 are B (MSE); each wave owns CPW column blocks.
// ---------------------------------------------------------------------------
template <typename E, int D, bool MSE, int CPW, bool SNAP, int PD>
__global__ __launch_bounds__((MSE ? 2 : 1) * (D / 16) / CPW * 64) void lin_summary(LinParams p)
{
    typedef typename Frag<E>::type F;
    constexpr int ND = D / 16;
    constexpr int NW = (MSE ? 2 : 1) * ND / CPW;
    constexpr int NT = NW * 64;
    __shared__ SubTile<E, D> tiles[2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, m = lane & 15;
    const int seg = blockIdx.x % p.Ssum, h = blockIdx.x / p.Ssum;
    const int T = p.Tkv;
    const int t0 = seg * p.seg_tokens;
    const int tend = min(T, t0 + p.seg_tokens);

    Loader<E, D, STAGE_K | STAGE_V | STAGE_E, PD, NT> ld;
    ld.init(threadIdx.x, p, h, T, tend);
    const float *eta_h = p.eta + (size_t)h * T;

    // X starts at 0 and stays moderate, so one bf16 rounding per element is
    // enough for the residual product.
    f32x4 X[CPW][ND];
    F Xr[CPW][ND], Xs[SNAP ? CPW : 1][ND];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int r = 0; r < ND; ++r) {
            X[c][r] = zero4();
            Xr[c][r] = to_frag<E>(zero4());
            if (SNAP) Xs[c][r] = Xr[c][r];
        }

    run_subblocks<E, D, STAGE_K | STAGE_V | STAGE_E, PD, NT>(tiles, ld, t0, tend,
        [&](SubTile<E, D> &tl, int tg) {
            if (SNAP && MSE && (tg % p.chunk) == 0) {
#pragma unroll
                for (int c = 0; c < CPW; ++c)
#pragma unroll
                    for (int r = 0; r < ND; ++r) Xs[c][r] = Xr[c][r];
            }
            F Ka[ND];
            if (MSE) {
#pragma unroll
                for (int r = 0; r < ND; ++r) Ka[r] = lds_frag<E>(&tl.ks[m][16 * r + 4 * g]);
            }
            const f32x4 et = *reinterpret_cast<const f32x4 *>(&tl.eta[4 * g]);
            F EU[CPW];
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                const int x = wave * CPW + c;
                const bool pcol = MSE && x < ND;
                const int cb = pcol ? x : x - (MSE ? ND : 0);
                f32x4 U = frag_to_f32(tok_frag<E, D>(tl, !pcol, cb, m, g));
                if (MSE) U = U - mma_b<F, ND>(zero4(), Ka, SNAP ? Xs[c] : Xr[c]);
                EU[c] = to_frag<E>(U * et);
            }
            F KtA[ND];
#pragma unroll
            for (int r = 0; r < ND; ++r) KtA[r] = tok_frag<E, D>(tl, false, r, m, g);
#pragma unroll
            for (int c = 0; c < CPW; ++c)
#pragma unroll
                for (int r = 0; r < ND; ++r) {
                    X[c][r] = mma16(X[c][r], KtA[r], EU[c]);
                    if (MSE) Xr[c][r] = to_frag<E>(X[c][r]);
                }
        });

    const size_t base = ((size_t)h * p.Ssum + seg) * D * D;
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int x = wave * CPW + c;
        const bool pcol = MSE && x < ND;
        const int cb = pcol ? x : x - (MSE ? ND : 0);
        if (pcol) {
            E *dst = (E *)p.wsP + base;
#pragma unroll
            for (int r = 0; r < ND; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    dst[(size_t)(16 * r + 4 * g + j) * D + 16 * cb + m] = (E)X[c][r][j];
        } else {
            float *dst = p.wsB + base;
#pragma unroll
            for (int r = 0; r < ND; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j) dst[(size_t)(16 * r + 4 * g + j) * D + 16 * cb + m] = X[c][r][j];
        }
    }
}

// ---------------------------------------------------------------------------
// prefix: per (head, column block), one wave per 16-row tile of the state.
// W_start(0) = w_init; W_start(s+1) = W_start(s) - P_s W_start(s) + B_s.
// Writes every W_start(s) (slot s of wsW); with WRITE_FINAL also the state
// after the last summarised segment into slot S and into w_final.
// ---------------------------------------------------------------------------
template <typename E, int D, bool MSE, bool WRITE_FINAL>
__global__ __launch_bounds__((D / 16) * 64) void lin_prefix(LinParams p)
{
    typedef typename Frag<E>::type F;
    constexpr int ND = D / 16;
    constexpr int PP = (D == 64) ? 8 : 4;  // steps of P/B prefetched ahead (memory latency)
    __shared__ SplitFrag<E> xch[2][ND][64];
    const int lane = threadIdx.x & 63, r = threadIdx.x >> 6, g = lane >> 4, m = lane & 15;
    const int cb = blockIdx.x % ND, h = blockIdx.x / ND;
    const float *w0 = p.w_init + (size_t)h * D * D;
    float *wsW = p.wsW + (size_t)h * (p.S + 1) * D * D;

    f32x4 W;
#pragma unroll
    for (int j = 0; j < 4; ++j) W[j] = w0[(size_t)(16 * r + 4 * g + j) * D + 16 * cb + m];
#pragma unroll
    for (int j = 0; j < 4; ++j) wsW[(size_t)(16 * r + 4 * g + j) * D + 16 * cb + m] = W[j];

    // Steps are padded up to a multiple of PP so the prefetch ring runs
    // without branches: padded steps read the last valid step's data, add
    // nothing (masked to zero at use) and rewrite the last slot unchanged.
    const int nst = p.Ssum;
    const int ngroups = (nst + PP - 1) / PP;
    F PA[PP][ND];
    f32x4 BB[PP];
    auto issue = [&](int slot, int s) {
        const size_t base = ((size_t)h * p.Ssum + min(s, nst - 1)) * D * D;
        if (MSE) {
            const E *P = (const E *)p.wsP + base;
#pragma unroll
            for (int q = 0; q < ND; ++q) PA[slot][q] = load4<E>(P + (size_t)(16 * r + m) * D + 16 * q + 4 * g);
        }
        const float *Bm = p.wsB + base;
#pragma unroll
        for (int j = 0; j < 4; ++j) BB[slot][j] = Bm[(size_t)(16 * r + 4 * g + j) * D + 16 * cb + m];
    };
#pragma unroll
    for (int s = 0; s < PP; ++s) issue(s, s);
    for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
        for (int jj = 0; jj < PP; ++jj) {
            const int s = gi * PP + jj;
            const bool live = s < nst;
            f32x4 upd = BB[jj];
            if (MSE) {
                SplitFrag<E> mine;
                mine.set(W);
                xch[jj & 1][r][lane] = mine;
                lds_barrier();
                SplitFrag<E> Wb[ND];
#pragma unroll
                for (int q = 0; q < ND; ++q) Wb[q] = xch[jj & 1][q][lane];
                upd = upd - mma_state_b<E, ND>(zero4(), PA[jj], Wb);
            }
            W = W + (live ? upd : zero4());
            issue(jj, s + PP);
            float *dst = wsW + (size_t)min(s + 1, nst) * D * D;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[(size_t)(16 * r + 4 * g + j) * D + 16 * cb + m] = W[j];
        }
    }
    if (WRITE_FINAL) {
        float *wf = p.w_final + (size_t)h * D * D;
#pragma unroll
        for (int j = 0; j < 4; ++j) wf[(size_t)(16 * r + 4 * g + j) * D + 16 * cb + m] = W[j];
    }
}

// ---------------------------------------------------------------------------
// replay (causal): outputs of one segment from its start state.  Each wave
// owns CPW column blocks; the query/key fragments and the masked Q K^T block
// are shared by them.  SNAP: chunks longer than one sub-block need a separate
// chunk-start snapshot of the state for the residual.
// ---------------------------------------------------------------------------
template <typename E, int D, bool MSE, int CPW, bool SNAP, int PD>
__global__ __launch_bounds__((D / 16) / CPW * 64) void lin_replay(LinParams p)
{
    typedef typename Frag<E>::type F;
    constexpr int ND = D / 16;
    constexpr int NW = ND / CPW;
    constexpr int NT = NW * 64;
    __shared__ SubTile<E, D> tiles[2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, m = lane & 15;
    const int seg = blockIdx.x % p.S, h = blockIdx.x / p.S;
    const int T = p.Tkv;
    const int t0 = seg * p.seg_tokens;
    const int tend = min(T, t0 + p.seg_tokens);

    const float *ws = (p.S > 1) ? p.wsW + ((size_t)h * (p.S + 1) + seg) * D * D
                                : p.w_init + (size_t)h * D * D;
    // State = W0 + dW: the start state enters products as a split (hi/lo)
    // pair computed once; the change dW since the segment start stays small,
    // so one bf16 rounding of it per sub-block is enough.
    SplitFrag<E> W0[CPW][ND];
    f32x4 dW[CPW][ND];
    F dWr[CPW][ND], dWs[SNAP ? CPW : 1][ND];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int cb = wave * CPW + c;
#pragma unroll
        for (int r = 0; r < ND; ++r) {
            f32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = ws[(size_t)(16 * r + 4 * g + j) * D + 16 * cb + m];
            W0[c][r].set(w);
            dW[c][r] = zero4();
            dWr[c][r] = to_frag<E>(zero4());
            if (SNAP) dWs[c][r] = dWr[c][r];
        }
    }

    Loader<E, D, STAGE_Q | STAGE_K | STAGE_V | STAGE_E, PD, NT> ld;
    ld.init(threadIdx.x, p, h, T, tend);
    E *out_h = (E *)p.out + (size_t)h * T * D;

    run_subblocks<E, D, STAGE_Q | STAGE_K | STAGE_V | STAGE_E, PD, NT>(tiles, ld, t0, tend,
        [&](SubTile<E, D> &tl, int tg) {
            if (SNAP && MSE && (tg % p.chunk) == 0) {
#pragma unroll
                for (int c = 0; c < CPW; ++c)
#pragma unroll
                    for (int r = 0; r < ND; ++r) dWs[c][r] = dWr[c][r];
            }
            F Qa[ND], Ka[ND];
#pragma unroll
            for (int r = 0; r < ND; ++r) {
                Qa[r] = lds_frag<E>(&tl.qs[m][16 * r + 4 * g]);
                Ka[r] = lds_frag<E>(&tl.ks[m][16 * r + 4 * g]);
            }
            const f32x4 et = *reinterpret_cast<const f32x4 *>(&tl.eta[4 * g]);
            // S^T[i][t] = k_i . q_t, kept for i <= t, times eta_i.
            f32x4 St = mma_b<F, ND>(zero4(), Ka, Qa);
#pragma unroll
            for (int j = 0; j < 4; ++j) St[j] = (4 * g + j <= m) ? St[j] * et[j] : 0.f;
            const F Sf = to_frag<E>(St);
            const int t = tg + m;
            F EU[CPW];
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                const int cb = wave * CPW + c;
                f32x4 U = frag_to_f32(tok_frag<E, D>(tl, true, cb, m, g));
                if (MSE) {
                    f32x4 P = zero4();
#pragma unroll
                    for (int r = 0; r < ND; r += 2) P = mma32(P, Ka[r], Ka[r + 1], W0[c][r].hi, W0[c][r + 1].hi);
                    P = mma_b<F, ND>(P, Ka, SNAP ? dWs[c] : dWr[c]);
                    U = U - P;
                }
                // O^T = W^T Q^T + U^T S^T with W = W0 + dW (running).  The two
                // terms use separate accumulators: no accumulation chain mixes
                // MFMA shapes (16x16x32 feeding 16x16x16).
                const f32x4 Oi = mma16(zero4(), to_frag<E>(U), Sf);
                f32x4 O = mma_state_a<E, ND>(zero4(), W0[c], Qa);
#pragma unroll
                for (int r = 0; r < ND; r += 2) O = mma32(O, dWr[c][r], dWr[c][r + 1], Qa[r], Qa[r + 1]);
                O = O + Oi;
                if (t < tend) store4<E>(out_h + (size_t)t * D + 16 * cb + 4 * g, out4<E>(O));
                EU[c] = to_frag<E>(U * et);
            }
            // dW += K^T (eta * U)
            F KtA[ND];
#pragma unroll
            for (int r = 0; r < ND; ++r) KtA[r] = tok_frag<E, D>(tl, false, r, m, g);
#pragma unroll
            for (int c = 0; c < CPW; ++c)
#pragma unroll
                for (int r = 0; r < ND; ++r) {
                    dW[c][r] = mma16(dW[c][r], KtA[r], EU[c]);
                    dWr[c][r] = to_frag<E>(dW[c][r]);
                }
        });

    if (seg == p.S - 1) {
        // final state = start state + change; all reads before any write (w_final
        // may alias w_init when there is a single segment)
        float *wf = p.w_final + (size_t)h * D * D;
        f32x4 w0f[CPW][ND];
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int r = 0; r < ND; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    w0f[c][r][j] = ws[(size_t)(16 * r + 4 * g + j) * D + 16 * (wave * CPW + c) + m];
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int r = 0; r < ND; ++r)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    wf[(size_t)(16 * r + 4 * g + j) * D + 16 * (wave * CPW + c) + m] = w0f[c][r][j] + dW[c][r][j];
    }
}

// ---------------------------------------------------------------------------
// apply (non-causal): O = Q W_final over query segments.
// ---------------------------------------------------------------------------
template <typename E, int D, int CPW, int PD>
__global__ __launch_bounds__((D / 16) / CPW * 64) void lin_apply(LinParams p, const float *wsrc,
                                                                 size_t wsrc_head_stride)
{
    typedef typename Frag<E>::type F;
    constexpr int ND = D / 16;
    constexpr int NT = ND / CPW * 64;
    __shared__ SubTile<E, D> tiles[2];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, m = lane & 15;
    const int seg = blockIdx.x % p.Sq, h = blockIdx.x / p.Sq;
    const int T = p.Tq;
    const int t0 = seg * p.seg_q;
    const int tend = min(T, t0 + p.seg_q);
    const float *ws = wsrc + (size_t)h * wsrc_head_stride;
    SplitFrag<E> Wr[CPW][ND];
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
        for (int r = 0; r < ND; ++r) {
            f32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = ws[(size_t)(16 * r + 4 * g + j) * D + 16 * (wave * CPW + c) + m];
            Wr[c][r].set(w);
        }
    Loader<E, D, STAGE_Q, PD, NT> ld;
    ld.init(threadIdx.x, p, h, T, tend);
    E *out_h = (E *)p.out + (size_t)h * T * D;
    run_subblocks<E, D, STAGE_Q, PD, NT>(tiles, ld, t0, tend,
        [&](SubTile<E, D> &tl, int tg) {
            F Qa[ND];
#pragma unroll
            for (int r = 0; r < ND; ++r) Qa[r] = lds_frag<E>(&tl.qs[m][16 * r + 4 * g]);
            const int t = tg + m;
#pragma unroll
            for (int c = 0; c < CPW; ++c) {
                const f32x4 O = mma_state_a<E, ND>(zero4(), Wr[c], Qa);
                if (t < tend) store4<E>(out_h + (size_t)t * D + 16 * (wave * CPW + c) + 4 * g, out4<E>(O));
            }
        });
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static int env_int(const char *name, int dflt)
{
    const char *s = getenv(name);
    if (!s || !*s) return dflt;
    return atoi(s);
}

LinearPlan linear_plan(const LinearShape &s)
{
    LinearPlan pl{};
    const int T = s.Tkv;
    // Segment length: whole chunks, enough segments to give every CU a few
    // workgroups, at least 64 tokens.
    const long long target_wg = env_int("TTT_LINEAR_TARGET_WG", 512);
    long long seg = (T > 0) ? ((long long)s.NH * T + target_wg - 1) / target_wg : s.chunk;
    if (seg < 64) seg = 64;
    const int forced = env_int("TTT_LINEAR_SEG_TOKENS", 0);
    if (forced > 0) seg = forced;
    seg = (seg + s.chunk - 1) / s.chunk * s.chunk;
    if (T > 0 && seg > T) seg = (T + s.chunk - 1) / s.chunk * s.chunk;
    pl.seg_tokens = (int)seg;
    pl.S = (T > 0) ? (int)((T + seg - 1) / seg) : 0;
    pl.Ssum = (s.order == 0) ? (pl.S > 0 ? pl.S - 1 : 0) : pl.S;
    long long segq = (s.Tq > 0) ? ((long long)s.NH * s.Tq + target_wg - 1) / target_wg : 16;
    if (segq < 64) segq = 64;
    segq = (segq + 15) / 16 * 16;
    pl.seg_q = (int)segq;
    pl.Sq = (s.Tq > 0) ? (int)((s.Tq + segq - 1) / segq) : 0;
    const size_t esz = s.bf16 ? 2 : 4;
    const size_t dd = (size_t)s.d * s.d;
    size_t off = 0;
    pl.offP = off;
    if (s.loss == 1) off = align_up(off + (size_t)s.NH * pl.Ssum * dd * esz, 256);
    pl.offB = off;
    off = align_up(off + (size_t)s.NH * pl.Ssum * dd * 4, 256);
    pl.offW = off;
    off = align_up(off + (size_t)s.NH * (pl.S + 1) * dd * 4, 256);
    pl.bytes = off;
    return pl;
}

template <typename E, int D, bool MSE, bool SNAP>
static hipError_t launch_typed(const LinearShape &s, const LinearPlan &pl, LinParams p,
                               hipStream_t st)
{
    constexpr int ND = D / 16;
    constexpr int PD = (D == 64) ? 8 : 4;  // sub-blocks in flight; even (LDS buffer = slot parity)
    constexpr int CPW_R = (D == 128) ? 2 : 1;             // replay / apply
    constexpr int CPW_S = (MSE || D == 128) ? 2 : 1;      // summary
    constexpr int NW_S = (MSE ? 2 : 1) * ND / CPW_S;
    if (s.Tkv > 0) {
        if (pl.Ssum > 0) {
            lin_summary<E, D, MSE, CPW_S, SNAP, PD><<<dim3(s.NH * pl.Ssum), dim3(NW_S * 64), 0, st>>>(p);
            if (s.order == 0)
                lin_prefix<E, D, MSE, false><<<dim3(s.NH * ND), dim3(ND * 64), 0, st>>>(p);
            else
                lin_prefix<E, D, MSE, true><<<dim3(s.NH * ND), dim3(ND * 64), 0, st>>>(p);
        }
        if (s.order == 0) {
            lin_replay<E, D, MSE, CPW_R, SNAP, PD><<<dim3(s.NH * pl.S), dim3(ND / CPW_R * 64), 0, st>>>(p);
        } else if (pl.Sq > 0) {
            lin_apply<E, D, CPW_R, PD><<<dim3(s.NH * pl.Sq), dim3(ND / CPW_R * 64), 0, st>>>(
                p, p.wsW + (size_t)pl.S * D * D, (size_t)(pl.S + 1) * D * D);
        }
    } else {
        // No key/value tokens: the state is unchanged.
        if (p.w_final != p.w_init) {
            hipError_t e = hipMemcpyAsync(p.w_final, p.w_init, (size_t)s.NH * D * D * 4,
                                          hipMemcpyDeviceToDevice, st);
            if (e != hipSuccess) return e;
        }
        if (s.order == 1 && pl.Sq > 0)
            lin_apply<E, D, CPW_R, PD><<<dim3(s.NH * pl.Sq), dim3(ND / CPW_R * 64), 0, st>>>(
                p, p.w_init, (size_t)D * D);
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
    p.wsW = (float *)((char *)ws + pl.offW);
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
    const bool snap = s.chunk > 16;
#define TTT_DISPATCH(E, D)                                                            \
    if (mse) return snap ? launch_typed<E, D, true, true>(s, pl, p, stream)           \
                         : launch_typed<E, D, true, false>(s, pl, p, stream);         \
    return launch_typed<E, D, false, false>(s, pl, p, stream);
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
