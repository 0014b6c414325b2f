// LaCT SwiGLU fast-weight forward on gfx950 (bf16 MFMA, fp32 masters).
//
// What is computed ("LaCT: Test-Time Training Done Right", sections 3.2,
// 3.3 and 4): per (batch, head) a fast weight f(x) = W2 (silu(W1 x) * (W3 x))
// with W1, W3 [hid x d] and W2 [d x hid].  Per chunk of key tokens, with the
// chunk-start weights:
//   dY  = -eta * V                       (inner-product loss)
//       =  eta * (f(K) - V)              (MSE loss)
//   G   = silu(K W1^T) * (K W3^T)        dG = dY W2
//   dH3 = dG * silu(K W1^T)              dH1 = dG * (K W3^T) * silu'(K W1^T)
//   W1 -= dH1^T K,  W3 -= dH3^T K,  W2 -= dY^T G, then (optionally) every row
//   is rescaled to its L2 norm before the step.
// Causal: the queries of chunk c read the weights the chunk started with.
// Non-causal: every query reads the final weights.
//
// Kernels (one launch each):
//   lact_prep_weights  fp32 masters from the inits (where they do not alias)
//                 and the bf16 hi/lo weight copies of the first chunk.
//   lact_fwdgrad  per (head, 128-token tile, 128-wide hidden slice): the three
//                 products K W1^T, K W3^T, dY W2 share the d-long contraction
//                 (K and V read token-major as stored); the epilogue does the
//                 SwiGLU backward and writes G^T, dH1^T, dH3^T (hidden-major,
//                 token-contiguous: the next GEMM's k).
//   lact_wgrad    the three weight gradients as GEMMs over the chunk's tokens,
//                 split over tokens, fp32 partials; K and V (or dY) are read
//                 token-major as k-major operands through the transposing LDS
//                 read.
//   lact_update   sums the partials, takes the step (gradient descent,
//                 momentum, or Muon's Newton-Schulz direction), row norms, fp32
//                 masters, bf16 copies of the new weights.
//   lact_ns_gram, lact_ns_apply  Muon's Newton-Schulz iteration.
//   lact_apply1   G_q = silu(Q W1^T) * (Q W3^T) for every query, each with its
//                 chunk's weights (computed transposed so G_q lands
//                 token-major).
//   lact_apply2   O = G_q W2^T (computed transposed so O lands token-major);
//                 with the MSE loss the same two kernels give f(K) and dY.
// Every product is a bf16 16x16x32 MFMA with fp32 accumulation; tiles move
// global -> registers -> LDS with a ring of register stages and LDS-only
// barriers.
#include "lact_common.h"
#include "ttt_internal.h"

namespace tttk {

// ---------------------------------------------------------------------------
// prep: fp32 masters from the inits (skipped where they alias) and the bf16
// copies of slot 0.  Grid-stride over NH * 3 * hid * d elements.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lact_prep_weights(LactParams p)
{
    const long n13 = (long)p.hid * p.d;
    const long total = (long)p.NH * 3 * n13;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int h = (int)(i / (3 * n13));
        const long r = i % (3 * n13);
        const int which = (int)(r / n13);
        const long e = r % n13;
        if (which < 2) {
            const float *src = which == 0 ? p.w1i : p.w3i;
            float *dst = which == 0 ? p.w1 : p.w3;
            const float x = src[(long)h * n13 + e];
            if (dst != src) dst[(long)h * n13 + e] = x;
            const int row = (int)(e / p.d), col = (int)(e % p.d);
            const long o = (long)packed_row(row, which) * p.d + col;
            bf16 hi, lo;
            split1(x, hi, lo);
            p.w13b[slot_off13(p, 0, h, 0) + o] = hi;
            p.w13b[slot_off13(p, 0, h, 1) + o] = lo;
        } else {
            const float x = p.w2i[(long)h * n13 + e];
            if (p.w2 != p.w2i) p.w2[(long)h * n13 + e] = x;
            bf16 hi, lo;
            split1(x, hi, lo);
            p.w2b[slot_off2(p, 0, h, 0) + e] = hi;
            p.w2b[slot_off2(p, 0, h, 1) + e] = lo;
        }
    }
}

// ---------------------------------------------------------------------------
// fwdgrad: per (head, 128-token tile, 128-wide hidden slice) of chunk c.  Four
// waves as 2 x 2 tiles of 64 tokens x 64 hidden units, each holding all three
// products (K W1^T, K W3^T, dY W2) of its tile: 48 MFMAs per 32-wide k step
// for 20 fragment reads.
// ---------------------------------------------------------------------------
// k step, LDS row pitch (96-byte rows: measured ~3% faster on both LaCT
// workloads than 80-byte ones; the bank-conflict counter reads ~41% of
// LDS-active cycles with either pitch, so the conflicts come from other
// accesses), register stages (even, divides d / FBK)
constexpr int FBK = 32, FPITCH = FBK + 16, FPD = 2;
constexpr int F2PITCH = 128 + 16;  // W2 slice rows: transposing reads of 8 rows hit distinct banks

struct FwdGradLds {
    bf16 ak[2][128][FPITCH];   // K tile
    bf16 ay[2][128][FPITCH];   // dY tile
    bf16 b1[2][128][FPITCH];   // W1 rows of the slice
    bf16 b3[2][128][FPITCH];   // W3 rows of the slice
    bf16 b2[2][FBK][F2PITCH];  // W2 rows (k) of the slice, as stored
};
// Waves per workgroup: 8 (4 x 2 waves of 32 tokens x 64 hidden units; 96
// accumulator registers per wave, so two waves fit on each SIMD and one wave's
// MFMAs cover the other's loads) or 4 (2 x 2 waves of 64 tokens x 64 hidden
// units, one wave per SIMD; about 2% slower on the LaCT layer shapes).
#ifndef FWD_NW
#define FWD_NW 8
#endif
// After the k loop: each wave's three output tiles (its hidden units x its
// tokens), hidden-major, rows padded by 4 (the 16 rows a fragment write
// touches and the rows of a 16-lane read fall on distinct banks)
template <int NW> struct FwdGradOut {
    static constexpr int TOK = 128 / (NW / 2);  // tokens per wave
    static constexpr int PITCH = TOK + 4;
};
template <int NW> union FwdGradLdsAllT {
    FwdGradLds k;
    bf16 out[NW][3][64][FwdGradOut<NW>::PITCH];
};

template <int NW>
__global__ __launch_bounds__(64 * NW) void lact_fwdgrad(LactParams p, int c, int slot)
{
    constexpr int NT = 64 * NW;
    constexpr int MI = 4 / (NW / 4);      // 16-token m-tiles per wave (4 or 2)
    constexpr int TOKW = 16 * MI;         // tokens per wave
    constexpr int NI = 2 / (NW / 4);      // loader passes over the 128 tile rows (2 or 1)
    __shared__ FwdGradLdsAllT<NW> LA;
    FwdGradLds &L = LA.k;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, mm = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;
    const int nslice = p.hid / 128;
    const int ntile = p.cpad / 128;
    int bid = xcd_block(blockIdx.x, gridDim.x);
    const int sl = bid % nslice;
    bid /= nslice;
    const int tt = bid % ntile;
    const int h = bid / ntile;
    const int cstart = c * p.chunk;
    const int clen = min(p.chunk, p.Tkv - cstart);
    const int r0 = tt * 128;
    const int h0 = sl * 128;
    const int d = p.d;
    const bf16 *kh = p.k + ((long)h * p.Tkv + cstart) * d;
    const bf16 *vh = p.v + ((long)h * p.Tkv + cstart) * d;
    const float *eh = p.eta + (long)h * p.Tkv + cstart;
    const bf16 *dyh = p.dy + (long)h * p.cpad * d;
    const bf16 *w13 = p.w13b + slot_off13(p, slot, h);
    const bf16 *w2 = p.w2b + slot_off2(p, slot, h);
    const bool dot = (p.loss == 0);

    // 128 rows x 32 columns per operand and stage: rows tid/4 (+ 64 with four
    // waves), 8 columns each.  W2: k rows tid/16 (+ 16), 8 hidden columns.
    const int lrow = tid >> 2, lcol = (tid & 3) * 8;
    const int orow = tid >> 4, hcol = (tid & 15) * 8;
    float erow[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int t = r0 + lrow + 64 * i;
        erow[i] = (t < clen) ? (dot ? -eh[t] : 1.f) : 0.f;
    }
    // d is a multiple of 128, so the k steps fill whole groups of FPD and
    // every step computes: the loads, LDS writes and MFMAs of a step form one
    // basic block and interleave
    const int nst = d / FBK;
    const int ngroups = nst / FPD;
    B8 rk[FPD][NI], ry[FPD][NI], r1[FPD][NI], r3[FPD][NI], r2[FPD][NI];
    auto issue = [&](int s, int st) {
        const int kk = min(st, nst - 1) * FBK;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int t = min(r0 + lrow + 64 * i, clen - 1);
            rk[s][i] = ld16(kh + (long)t * d + kk + lcol);
            ry[s][i] = ld16((dot ? vh : dyh) + (long)t * d + kk + lcol);
            r1[s][i] = ld16(w13 + (long)packed_row(h0 + lrow + 64 * i, 0) * d + kk + lcol);
            r3[s][i] = ld16(w13 + (long)packed_row(h0 + lrow + 64 * i, 1) * d + kk + lcol);
            r2[s][i] = ld16(w2 + (long)(kk + orow + 16 * i) * p.hid + h0 + hcol);
        }
    };
    auto commit = [&](int s, int buf) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int row = lrow + 64 * i;
            const bool ok = r0 + row < clen;
            st16(&L.ak[buf][row][lcol], ok ? rk[s][i] : zero16());
            const bf16x8 vb = as_bf8(ry[s][i]);
            bf16x8 o;
#pragma unroll
            for (int j = 0; j < 8; ++j) o[j] = dot ? (bf16)((float)vb[j] * erow[i]) : (ok ? vb[j] : (bf16)0.f);
            st16(&L.ay[buf][row][lcol], B8{__builtin_bit_cast(u32x4v, o)});
            st16(&L.b1[buf][row][lcol], r1[s][i]);
            st16(&L.b3[buf][row][lcol], r3[s][i]);
            st16(&L.b2[buf][kperm(orow + 16 * i)][hcol], r2[s][i]);
        }
    };
    // wave (wm, wn): tokens TOKW wm .. TOKW wm + TOKW - 1 (MI m-tiles), hidden
    // 64 wn .. 64 wn + 63 of the slice (4 n-tiles)
    f32x4 a1[MI][4], a3[MI][4], a2[MI][4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) a1[i][q] = a3[i][q] = a2[i][q] = zero4();

#pragma unroll
    for (int s = 0; s < FPD; ++s) issue(s, s);
    commit(0, 0);
    lds_barrier();
    for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
        for (int j = 0; j < FPD; ++j) {
            const int st = gi * FPD + j;
            const int buf = j & 1;  // FPD is even: the LDS buffer is the k-step parity
            // All fragments of the step first, all in natural k order (8
            // consecutive k per lane).  W2's fragments come from the
            // transposing read; its stage holds k row 8g + j at row kperm (4g +
            // j, or 16 + 4g + j - 4), so the two reads return k = 8g .. 8g + 7
            // and dY's fragments are one 16-byte read like K's.
            bf16x8 fk[MI], fy[MI], f1[4], f3[4], f2[4];
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int row = wm * TOKW + 16 * i + mm;
                fk[i] = as_bf8(ld16(&L.ak[buf][row][8 * g]));
                fy[i] = as_bf8(ld16(&L.ay[buf][row][8 * g]));
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = wn * 64 + 16 * q;
                f1[q] = as_bf8(ld16(&L.b1[buf][col + mm][8 * g]));
                f3[q] = as_bf8(ld16(&L.b3[buf][col + mm][8 * g]));
                const bf16x4 w0 = lds_read_tr(&L.b2[buf][4 * g + (mm >> 2)][col + 4 * (mm & 3)]);
                const bf16x4 w1 = lds_read_tr(&L.b2[buf][16 + 4 * g + (mm >> 2)][col + 4 * (mm & 3)]);
                f2[q] = __builtin_shufflevector(w0, w1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            // the loads and LDS writes of later steps go into the MFMAs' shadow
            issue(j, st + FPD);
            commit((j + 1) % FPD, (j + 1) & 1);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    a1[i][q] = mfma32(a1[i][q], fk[i], f1[q]);
                    a3[i][q] = mfma32(a3[i][q], fk[i], f3[q]);
                    a2[i][q] = mfma32(a2[i][q], fy[i], f2[q]);
                }
            // schedule: the fragment reads, then the MFMAs with a global load
            // or an LDS write after every second one
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * MI + 16, 0);
#pragma unroll
            for (int x = 0; x < 5 * NI; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
#pragma unroll
            for (int x = 0; x < 5 * NI; ++x) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 12 * MI - 20 * NI, 0);
            lds_barrier();
        }
    }
    // lane: tokens TOKW wm + 16 i + 4 g + (0..3), hidden 64 wn + 16 q + mm of
    // the tile.  Rows past the chunk have K = dY = 0, so every output there is
    // 0.  The three outputs go through the wave's own LDS tiles (the k loop
    // ended with a barrier, so the operand buffers are free) and leave as whole
    // rows of the wave's tokens.
    // Inner product: G^T is written with each token's -eta folded in, so the
    // weight gradient of W2 (sum over tokens of dY^T G, dY = -eta V) reads V.
    constexpr int OP = FwdGradOut<NW>::PITCH;
    bf16(*st)[64][OP] = LA.out[wave];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        f32x4 ge;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t = r0 + wm * TOKW + 16 * i + 4 * g + j;
            ge[j] = dot ? ((t < clen) ? -eh[t] : 0.f) : 1.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 gv, v1, v3;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float z1 = a1[i][q][j], z3 = a3[i][q][j], dg = a2[i][q][j];
                const float sg = sigmoidf_(z1);
                const float act = z1 * sg;
                gv[j] = act * z3 * ge[j];
                v3[j] = dg * act;
                v1[j] = dg * z3 * (sg * (1.f + z1 * (1.f - sg)));
            }
            store4<bf16>(&st[0][16 * q + mm][16 * i + 4 * g], to_bf16x4(gv));
            store4<bf16>(&st[1][16 * q + mm][16 * i + 4 * g], to_bf16x4(v1));
            store4<bf16>(&st[2][16 * q + mm][16 * i + 4 * g], to_bf16x4(v3));
        }
    }
    bf16 *const outs[3] = {p.gt + (long)h * p.hid * p.cpad, p.dh1t + (long)h * p.hid * p.cpad,
                           p.dh3t + (long)h * p.hid * p.cpad};
    constexpr int LPR = TOKW / 8;             // lanes per output row (16 bytes each)
    const int orowl = lane / LPR, ocol = (lane % LPR) * 8;
#pragma unroll
    for (int o = 0; o < 3; ++o)
#pragma unroll
        for (int r = 0; r < 64 / (64 / LPR); ++r) {
            const int row = (64 / LPR) * r + orowl;
            const bf16x4 x0 = load4<bf16>(&st[o][row][ocol]);
            const bf16x4 x1 = load4<bf16>(&st[o][row][ocol + 4]);
            const bf16x8 x = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
            st16(outs[o] + (long)(h0 + wn * 64 + row) * p.cpad + r0 + wm * TOKW + ocol,
                 B8{__builtin_bit_cast(u32x4v, x)});
        }
}

// ---------------------------------------------------------------------------
// wgrad: the three weight gradients of chunk c, split over its tokens.
//   which 0: dW1[h][i] = sum_t dH1^T[h][t] K^T[i][t]   as GEMM (M = i, N = h)
//   which 1: dW3 likewise with dH3^T
//   which 2: dW2[o][h] = sum_t dY^T[o][t] G^T[h][t]     as GEMM (M = h, N = o)
// A lane's four consecutive M indices are the contiguous dimension of the
// stored gradient.  Token ranges are whole 64-token steps: past the chunk end
// dH^T, G^T are zero (and dY^T too), so no guard is needed on k.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lact_wgrad(LactParams p, int c)
{
    __shared__ GemmLds L;
    const int d = p.d, hid = p.hid;
    const int t13 = (d / 128) * (hid / 128);
    int bid = xcd_block(blockIdx.x, gridDim.x);
    const int tile = bid % (3 * t13);
    bid /= 3 * t13;
    const int sk = bid % p.splitk;
    const int h = bid / p.splitk;
    const int which = tile / t13, ti = tile % t13;
    const int cstart = c * p.chunk;
    const int clen64 = (min(p.chunk, p.Tkv - cstart) + 63) / 64 * 64;
    const int kper = ((clen64 + p.splitk - 1) / p.splitk + 63) / 64 * 64;
    const int k0 = min(clen64, sk * kper);
    const int k1 = min(clen64, k0 + kper);
    float *part = p.part + (((long)sk * p.NH + h) * 3 + which) * (long)hid * d;
    const int Mdim = (which < 2) ? d : hid, Ndim = (which < 2) ? hid : d;
    const int tm = ti / (Ndim / 128), tn = ti % (Ndim / 128);
    if (k1 <= k0) {
        for (int e = threadIdx.x; e < 128 * 128; e += 256)
            part[(long)(tn * 128 + (e >> 7)) * Mdim + tm * 128 + (e & 127)] = 0.f;
        return;
    }
    // K and V (inner product) or dY (MSE) are read token-major straight from
    // their tensors, as k-major operands; rows past the chunk read as zero.
    const int clen = min(p.chunk, p.Tkv - cstart);
    const int kvalid = clen - k0;
    auto epi = [&](f32x4 (&acc)[4][4], int mb, int nb, int g, int mm) {
                     // the 128 x 128 partial staged in the GEMM's LDS (rows
                     // padded to 132 floats) and written as whole 512-byte rows
                     float(*sp)[132] = reinterpret_cast<float(*)[132]>(&L);
                     const int ml = mb - tm * 128, nl = nb - tn * 128;
#pragma unroll
                     for (int i = 0; i < 4; ++i)
#pragma unroll
                         for (int q = 0; q < 4; ++q)
                             *reinterpret_cast<f32x4 *>(&sp[nl + 16 * q + mm][ml + 16 * i + 4 * g]) = acc[i][q];
                     lds_barrier();
#pragma unroll
                     for (int r = 0; r < 16; ++r) {
                         const int piece = threadIdx.x + 256 * r;  // 128 rows x 32 pieces of 16 bytes
                         const int row = piece >> 5, ch = 4 * (piece & 31);
                         *reinterpret_cast<f32x4 *>(part + (long)(tn * 128 + row) * Mdim + tm * 128 + ch) =
                             *reinterpret_cast<const f32x4 *>(&sp[row][ch]);
                     }
                 };
    if (which < 2) {
        const bf16 *as[1] = {p.k + ((long)h * p.Tkv + cstart + k0) * d};
        const bf16 *bs[1] = {(which == 0 ? p.dh1t : p.dh3t) + (long)h * hid * p.cpad + k0};
        gemm_nt_tile<true, false>(L, as, d, bs, p.cpad, Mdim, Ndim, k1 - k0, 1, tm * 128, tn * 128, kvalid, epi);
    } else {
        // dW2 = sum_t dY_t^T G_t.  Inner product: dY = -eta V, and G^T already
        // carries the -eta, so B is V itself.
        const bf16 *as[1] = {p.gt + (long)h * hid * p.cpad + k0};
        const bf16 *bs[1] = {p.loss == 0 ? p.v + ((long)h * p.Tkv + cstart + k0) * d
                                         : p.dy + ((long)h * p.cpad + k0) * d};
        gemm_nt_tile<false, true>(L, as, p.cpad, bs, d, Mdim, Ndim, k1 - k0, 1, tm * 128, tn * 128, kvalid, epi);
    }
}

// ---------------------------------------------------------------------------
// update: one wave per row of W1, W3 (length d) or W2 (length hid).
// phase 0: W <- W - D, then the row back to its old L2 norm; writes the fp32
//   master and the bf16 copy of slot `dst_slot`.  D = the summed gradient G
//   (gradient descent), M = beta M + G (momentum, M written back), or lr X_k
//   (Muon: the Newton-Schulz iterate left in partial split 0).
// phase 1 (Muon, before the iteration): D = G or M = beta M + G, written in
//   place over partial split 0 (fp32) and as bf16 into the first iterate copy.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// At least five waves per SIMD: left to itself the compiler keeps a whole row's
// loads in flight per wave (148 registers, three waves per SIMD), so the 5120
// row waves of the causal LM workload ran in two rounds; with 68 registers
// they run in one (momentum 1.18 -> 1.12 ms, Muon 3.11 -> 2.96 ms per call).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5, 8))) void lact_update(LactParams p,
                                                                                             int dst_slot,
                                                                                             int phase)
{
    const int lane = threadIdx.x & 63;
    const int rows_per_head = 2 * p.hid + p.d;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= p.NH * rows_per_head) return;
    const int h = gw / rows_per_head, r = gw % rows_per_head;
    int which, row, len;
    if (r < p.hid) { which = 0; row = r; len = p.d; }
    else if (r < 2 * p.hid) { which = 1; row = r - p.hid; len = p.d; }
    else { which = 2; row = r - 2 * p.hid; len = p.hid; }
    const long n13 = (long)p.hid * p.d;
    float *w = (which == 0 ? p.w1 : which == 1 ? p.w3 : p.w2) + (long)h * n13 + (long)row * len;
    const long eoff = ((long)h * 3 + which) * n13 + (long)row * len;  // element 0 of the row
    float *mrow = nullptr;
    if (p.rule == 1 || (p.rule == 2 && p.beta != 0.f))
        mrow = (which == 0 ? p.m1 : which == 1 ? p.m3 : p.m2) + (long)h * n13 + (long)row * len;
    if (phase == 1) {
        for (int col = lane; col < len; col += 64) {
            float gsum = 0.f;
            for (int s = 0; s < p.splitk; ++s) gsum += p.part[(long)s * p.NH * 3 * n13 + eoff + col];
            if (mrow) {
                gsum += p.beta * mrow[col];
                mrow[col] = gsum;
            }
            p.part[eoff + col] = gsum;
            p.nsb[eoff + col] = (bf16)gsum;
        }
        return;
    }
    // Each lane owns four consecutive columns per 256-column step (rows are
    // multiples of 128 long, at most 1024), and every load of the row is issued
    // before the first use: the kernel is one round of latency, not of issue.
    constexpr int MAXE = 4;
    f32x4 ov[MAXE], dv[MAXE];
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        ov[e] = dv[e] = zero4();
        const int col = 4 * lane + 256 * e;
        if (col < len) ov[e] = load4<float>(w + col);
    }
    if (p.rule == 2) {
#pragma unroll
        for (int e = 0; e < MAXE; ++e) {
            const int col = 4 * lane + 256 * e;
            if (col < len) dv[e] = p.lr * load4<float>(p.part + eoff + col);
        }
    } else {
        for (int sp = 0; sp < p.splitk; ++sp) {
            const float *ps = p.part + (long)sp * p.NH * 3 * n13 + eoff;
#pragma unroll
            for (int e = 0; e < MAXE; ++e) {
                const int col = 4 * lane + 256 * e;
                if (col < len) dv[e] += load4<float>(ps + col);
            }
        }
        if (mrow) {
#pragma unroll
            for (int e = 0; e < MAXE; ++e) {
                const int col = 4 * lane + 256 * e;
                if (col < len) {
                    dv[e] += p.beta * load4<float>(mrow + col);
                    store4<float>(mrow + col, dv[e]);
                }
            }
        }
    }
    float so = 0.f, sn = 0.f;
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        const int col = 4 * lane + 256 * e;
        if (col < len) {
            const f32x4 x = ov[e] - dv[e];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                so += ov[e][j] * ov[e][j];
                sn += x[j] * x[j];
            }
            if (p.save_w) {
                const long so_off = (long)p.save_c * p.NH * 3 * n13 + eoff + col;
                store4<float>(p.save_w + so_off, ov[e]);
                store4<float>(p.save_d + so_off, dv[e]);
            }
            ov[e] = x;
        }
    }
    float scale = 1.f;
    if (p.rownorm) {
        so = wave_sum(so);
        sn = wave_sum(sn);
        scale = (sn > 0.f) ? sqrtf(so) / sqrtf(sn) : 1.f;
    }
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        const int col = 4 * lane + 256 * e;
        if (col < len) {
            // rounded once: the bf16 pair below must encode exactly the stored
            // master (a product fused into the split would give a different lo
            // part than a later call rebuilding the pair from the master)
            f32x4 x;
            bf16x4 hi, lo;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma clang fp contract(off)
                x[j] = ov[e][j] * scale;
                bf16 h1, l1;
                split1(x[j], h1, l1);
                hi[j] = h1;
                lo[j] = l1;
            }
            store4<float>(w + col, x);
            if (which < 2) {
                const long o = (long)packed_row(row, which) * p.d + col;
                store4<bf16>(p.w13b + slot_off13(p, dst_slot, h, 0) + o, hi);
                store4<bf16>(p.w13b + slot_off13(p, dst_slot, h, 1) + o, lo);
            } else {
                const long o = (long)row * p.hid + col;
                store4<bf16>(p.w2b + slot_off2(p, dst_slot, h, 0) + o, hi);
                store4<bf16>(p.w2b + slot_off2(p, dst_slot, h, 1) + o, lo);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Muon: k steps of the cubic Newton-Schulz iteration for the orthogonal polar
// factor of each matrix's step direction D ("LaCT" section 3.3 names Muon's
// Newton-Schulz map without coefficients; the textbook cubic form is used):
//     X_0 = D / ||D||_F,   X_{j+1} = 1.5 X_j - 0.5 X_j (X_j^T X_j).
// With T the tall view of a matrix (W1, W3 gradients [hid][d] as they are,
// W2's [d][hid] transposed) the Gram matrix T^T T is d x d for all three, and
// the product is written as T (T^T T) for W1 and W3 and (T^T T) T^T for W2,
// so every launch covers the three matrices of all heads.  Step 0 runs on the
// unscaled D: its Gram diagonal (fp32) gives ||D||_F^2, and the apply scales
// by it.  Operands are bf16 copies of the iterate; the iterate itself and all
// accumulations are fp32.
// ---------------------------------------------------------------------------
// Both kernels run 64 x 128 output tiles: the matrices are small (a few
// hundred rows), so the launches are latency-bound and the smaller tile
// doubles the workgroups and halves each wave's products per k step.
constexpr int NSMB = 2, NSBM = 32 * NSMB;
using NsLds = GemmLdsT<NSBM>;
// fp32 staging of a product tile in the GEMM's LDS (rows padded by 4: a
// fragment write's 4 row groups fall 16 banks apart)
constexpr int NSPITCH = 128 + 4;
static_assert(sizeof(float[NSBM][NSPITCH]) <= sizeof(NsLds), "staged tile fits the GEMM's LDS");

__global__ __launch_bounds__(256) void lact_ns_gram(LactParams p, int step)
{
    __shared__ NsLds L;
    const int d = p.d, hid = p.hid;
    const int tpn = d / 128, tpt = (d / NSBM) * tpn;
    int bid = xcd_block(blockIdx.x, gridDim.x);
    const int tile = bid % tpt;
    bid /= tpt;
    const int which = bid % 3, h = bid / 3;
    const int tm = tile / tpn, tn = tile % tpn;
    const long n13 = (long)hid * d;
    const bf16 *x = p.nsb + (long)(step & 1) * p.NH * 3 * n13 + ((long)h * 3 + which) * n13;
    bf16 *gr = p.gram + ((long)h * 3 + which) * d * d;
    float *dg = p.diag + ((long)h * 3 + which) * d;
    // direct stores: staging this small bf16 tile through LDS measured ~1% slower
    auto epi = [&](f32x4 (&acc)[NSMB][4], int mb, int nb, int g, int mm) {
#pragma unroll
        for (int i = 0; i < NSMB; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int m = mb + 16 * i + 4 * g + j, n = nb + 16 * q + mm;
                    gr[(long)m * d + n] = (bf16)acc[i][q][j];
                    if (step == 0 && m == n) dg[m] = acc[i][q][j];
                }
    };
    const bf16 *as[1] = {x};
    if (which < 2)  // T = X [hid][d]: T^T T, both operands k-major
        gemm_nt_tile<true, true, NSMB>(L, as, d, as, d, d, d, hid, 1, tm * NSBM, tn * 128, hid, epi);
    else            // T = X^T, X [d][hid]: X X^T
        gemm_nt_tile<false, false, NSMB>(L, as, hid, as, hid, d, d, hid, 1, tm * NSBM, tn * 128, 1 << 30, epi);
}

__global__ __launch_bounds__(256) void lact_ns_apply(LactParams p, int step)
{
    __shared__ NsLds L;
    __shared__ float red[4];
    const int d = p.d, hid = p.hid;
    const int tpm = (hid / NSBM) * (d / 128);  // tiles per matrix (either orientation)
    int bid = xcd_block(blockIdx.x, gridDim.x);
    const int tile = bid % tpm;
    bid /= tpm;
    const int which = bid % 3, h = bid / 3;
    const long n13 = (long)hid * d;
    const long moff = ((long)h * 3 + which) * n13;
    const bf16 *x = p.nsb + (long)(step & 1) * p.NH * 3 * n13 + moff;
    bf16 *xn = p.nsb + (long)((step + 1) & 1) * p.NH * 3 * n13 + moff;
    float *xf = p.part + moff;
    const bf16 *gr = p.gram + ((long)h * 3 + which) * d * d;
    // step 0: the iterate is D itself; X_1 = (1.5 D - 0.5 D (D^T D) / s^2) / s, s = ||D||_F
    float a = 1.5f, b = -0.5f;
    if (step == 0) {
        float ss = 0.f;
        for (int e = threadIdx.x; e < d; e += 256) ss += p.diag[((long)h * 3 + which) * d + e];
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
        __syncthreads();
        ss = red[0] + red[1] + red[2] + red[3];
        const float inv = ss > 0.f ? 1.f / sqrtf(ss) : 0.f;
        a = 1.5f * inv;
        b = ss > 0.f ? -0.5f * inv / ss : 0.f;
    }
    const int N = (which < 2) ? d : hid;
    const int tm = (which < 2) ? tile / (d / 128) : tile / (hid / 128);
    const int tn = (which < 2) ? tile % (d / 128) : tile % (hid / 128);
    const int m0 = tm * NSBM, n0 = tn * 128;
    auto epi = [&](f32x4 (&acc)[NSMB][4], int mb, int nb, int g, int mm) {
        // the product tile goes through LDS (free after the k loop's last
        // barrier); the iterate is then read and written as whole rows
        float(*S)[NSPITCH] = reinterpret_cast<float(*)[NSPITCH]>(&L);
#pragma unroll
        for (int i = 0; i < NSMB; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    S[mb - m0 + 16 * i + 4 * g + j][nb - n0 + 16 * q + mm] = acc[i][q][j];
        __syncthreads();
        const int t = threadIdx.x;
#pragma unroll 4
        for (int it = 0; it < NSBM / 8; ++it) {
            const int r = (t >> 5) + 8 * it, c = (t & 31) * 4;
            const long e = (long)(m0 + r) * N + n0 + c;
            const f32x4 xo = load4<float>(xf + e);
            const f32x4 pr = load4<float>(&S[r][c]);
            f32x4 v;
            bf16x4 vb;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j] = a * xo[j] + b * pr[j];
                vb[j] = (bf16)v[j];
            }
            store4<float>(xf + e, v);
            store4<bf16>(xn + e, vb);
        }
    };
    if (which < 2) {  // X [hid][d]: X G, G symmetric (row-major = its own transpose)
        const bf16 *as[1] = {x};
        const bf16 *bs[1] = {gr};
        gemm_nt_tile<false, false, NSMB>(L, as, d, bs, d, hid, d, d, 1, m0, n0, 1 << 30, epi);
    } else {          // X [d][hid]: G X, X read k-major
        const bf16 *as[1] = {gr};
        const bf16 *bs[1] = {x};
        gemm_nt_tile<false, true, NSMB>(L, as, d, bs, hid, d, hid, d, 1, m0, n0, d, epi);
    }
}

// ---------------------------------------------------------------------------
// apply1: G[t][hh] = silu(x_t . W1[hh]) * (x_t . W3[hh]) for the rows of X
// (queries, or the chunk's keys for the MSE loss), computed as the GEMM
// packed(W1, W3) X^T so each lane holds 4 consecutive hidden units of one token.
// Token tiles never straddle chunks (chunk % 128 == 0 or one chunk).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lact_apply1(LactParams p, const bf16 *X, long x_head_stride,
                                                   int T, int slot_fixed, int slot0)
{
    __shared__ GemmLds L;
    const int mt = (2 * p.hid) / 128, nt = (T + 127) / 128;
    int bid = xcd_block(blockIdx.x, gridDim.x);
    const int tm = bid % mt;
    bid /= mt;
    const int tn = bid % nt;
    const int h = bid / nt;
    const int slot = (slot_fixed >= 0) ? slot_fixed : slot0 + (tn * 128) / p.chunk;
    // X (W_hi + W_lo)^T: two K segments over the same X rows
    const bf16 *as[2] = {p.w13b + slot_off13(p, slot, h, 0), p.w13b + slot_off13(p, slot, h, 1)};
    const bf16 *B = X + (long)h * x_head_stride;
    const bf16 *bs[2] = {B, B};
    bf16 *G = p.gq + (long)h * 2 * p.qpad * p.hid;
    bf16 *Glo = G + (long)p.qpad * p.hid;
    gemm_nt_tile(L, as, p.d, bs, p.d, 2 * p.hid, T, p.d, 2, tm * 128, tn * 128, 1 << 30,
                 [&](f32x4 (&acc)[4][4], int mb, int nb, int g, int mm) {
                     // G of the tile's 128 tokens x 64 hidden units, hi and lo,
                     // staged token-major in the GEMM's LDS (free after its last
                     // barrier; rows padded to 34 dwords) and written as whole
                     // 128-byte rows
                     bf16(*sh)[68] = reinterpret_cast<bf16(*)[68]>(&L);
                     bf16(*sl)[68] = sh + 128;
                     const int ml = mb - tm * 128, nl = nb - tn * 128;
#pragma unroll
                     for (int i = 0; i < 4; i += 2)
#pragma unroll
                         for (int q = 0; q < 4; ++q) {
                             const int tl = nl + 16 * q + mm;
                             const int hl = (ml + 16 * i) / 2 + 4 * g;
                             f32x4 gv;
#pragma unroll
                             for (int j = 0; j < 4; ++j) {
                                 const float z1 = acc[i][q][j], z3 = acc[i + 1][q][j];
                                 gv[j] = z1 * sigmoidf_(z1) * z3;
                             }
                             const bf16x4 hi = to_bf16x4(gv);
                             store4<bf16>(&sh[tl][hl], hi);
                             store4<bf16>(&sl[tl][hl], to_bf16x4(gv - to_f32x4(hi)));
                         }
                     lds_barrier();
#pragma unroll
                     for (int r = 0; r < 4; ++r) {
                         const int piece = threadIdx.x + 256 * r;  // 128 rows x 8 pieces of 16 bytes
                         const int row = piece >> 3, ch = 8 * (piece & 7);
                         const int t = tn * 128 + row;
                         if (t < T) {
                             const long off = (long)t * p.hid + tm * 64 + ch;
                             st16(G + off, B8{__builtin_bit_cast(u32x4v, __builtin_shufflevector(
                                                  load4<bf16>(&sh[row][ch]), load4<bf16>(&sh[row][ch + 4]),
                                                  0, 1, 2, 3, 4, 5, 6, 7))});
                             st16(Glo + off, B8{__builtin_bit_cast(u32x4v, __builtin_shufflevector(
                                                    load4<bf16>(&sl[row][ch]), load4<bf16>(&sl[row][ch + 4]),
                                                    0, 1, 2, 3, 4, 5, 6, 7))});
                         }
                     }
                 });
}

// apply2: Y[t][o] = G[t] . W2[o], as the GEMM W2 G^T (4 consecutive outputs of
// one token per lane).  mode 0: out = Y (bf16).  mode 1 (MSE): dY = eta (Y - V)
// token-major into p.dy (chunk-local tokens).
__global__ __launch_bounds__(256) void lact_apply2(LactParams p, int T, int slot_fixed, int mode,
                                                   int c, int slot0)
{
    __shared__ GemmLds L;
    const int mt = p.d / 128, nt = (T + 127) / 128;
    int bid = xcd_block(blockIdx.x, gridDim.x);
    const int tm = bid % mt;
    bid /= mt;
    const int tn = bid % nt;
    const int h = bid / nt;
    const int slot = (slot_fixed >= 0) ? slot_fixed : slot0 + (tn * 128) / p.chunk;
    // (W2_hi G_hi + W2_lo G_hi + W2_hi G_lo): three K segments
    const bf16 *whi = p.w2b + slot_off2(p, slot, h, 0), *wlo = p.w2b + slot_off2(p, slot, h, 1);
    const bf16 *ghi = p.gq + (long)h * 2 * p.qpad * p.hid, *glo = ghi + (long)p.qpad * p.hid;
    const bf16 *as[3] = {whi, wlo, whi}, *bs[3] = {ghi, ghi, glo};
    const int cstart = c * p.chunk;
    gemm_nt_tile(L, as, p.hid, bs, p.hid, p.d, T, p.hid, 3, tm * 128, tn * 128, 1 << 30,
                 [&](f32x4 (&acc)[4][4], int mb, int nb, int g, int mm) {
                     if (mode == 0) {
                         // O of the tile's 128 tokens x 128 outputs staged
                         // token-major in the GEMM's LDS (rows padded to 66
                         // dwords) and written as whole 256-byte rows
                         bf16(*so)[132] = reinterpret_cast<bf16(*)[132]>(&L);
                         const int ml = mb - tm * 128, nl = nb - tn * 128;
#pragma unroll
                         for (int i = 0; i < 4; ++i)
#pragma unroll
                             for (int q = 0; q < 4; ++q)
                                 store4<bf16>(&so[nl + 16 * q + mm][ml + 16 * i + 4 * g], to_bf16x4(acc[i][q]));
                         lds_barrier();
#pragma unroll
                         for (int r = 0; r < 8; ++r) {
                             const int piece = threadIdx.x + 256 * r;  // 128 rows x 16 pieces of 16 bytes
                             const int row = piece >> 4, ch = 8 * (piece & 15);
                             const int t = tn * 128 + row;
                             if (t < T)
                                 st16(p.out + ((long)h * p.Tq + cstart + t) * p.d + tm * 128 + ch,
                                      B8{__builtin_bit_cast(u32x4v, __builtin_shufflevector(
                                                            load4<bf16>(&so[row][ch]), load4<bf16>(&so[row][ch + 4]),
                                                            0, 1, 2, 3, 4, 5, 6, 7))});
                         }
                         return;
                     }
#pragma unroll
                     for (int i = 0; i < 4; ++i)
#pragma unroll
                         for (int q = 0; q < 4; ++q) {
                             const int t = nb + 16 * q + mm;
                             const int o = mb + 16 * i + 4 * g;
                             if (t >= T) continue;  // the readers treat rows past the chunk as zero
                             const long tk = (long)h * p.Tkv + cstart + t;
                             const float e = p.eta[tk];
                             const f32x4 vv = to_f32x4(load4<bf16>(p.v + tk * p.d + o));
                             store4<bf16>(p.dy + ((long)h * p.cpad + t) * p.d + o, to_bf16x4((acc[i][q] - vv) * e));
                         }
                 });
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

static int lact_splitk(const LactShape &s, int clen)
{
    const int t13 = (s.d / 128) * (s.hid / 128);
    const int tiles = s.NH * 3 * t13;
    // Up to two workgroups per CU.  Each split adds a 3 x hid x d fp32 partial
    // per head, written here and read back by the update: beyond two splits
    // only while that stays within a tenth of the chunk's own token traffic
    // (K and V read, G^T, dH1^T and dH3^T written and read).
    int sk = 512 / tiles;
    const long tok_bytes = (long)clen * (4L * s.d + 6L * s.hid);
    const long split_bytes = 24L * s.hid * s.d;
    const long cap = tok_bytes / (10 * split_bytes);
    if (sk > (cap > 2 ? cap : 2)) sk = (int)(cap > 2 ? cap : 2);
    const int maxsk = (clen + 511) / 512;          // at least 512 tokens per split
    if (sk > maxsk) sk = maxsk;
    return sk < 1 ? 1 : sk;
}

LactPlan lact_plan(const LactShape &s)
{
    LactPlan pl{};
    const int chunk = (s.Tkv > 0 && s.chunk >= s.Tkv) ? s.Tkv : s.chunk;
    pl.nchunks = (s.Tkv > 0) ? (s.Tkv + chunk - 1) / chunk : 0;
    const int clen = (s.Tkv > 0) ? (chunk < s.Tkv ? chunk : s.Tkv) : 0;
    const size_t cpad = (size_t)((clen + 127) / 128 * 128);
    const size_t qpad = (size_t)(((s.Tq > (int)cpad ? s.Tq : (int)cpad) + 127) / 128 * 128);
    pl.maxc = (int)cpad;
    const int nslots = (s.order == 0) ? pl.nchunks + 1 : 1;
    const int splitk = lact_splitk(s, clen);
    const size_t NH = s.NH, d = s.d, hid = s.hid;
    size_t off = 0;
    auto take = [&](int idx, size_t bytes) {
        pl.off[idx] = off;
        off = al256(off + bytes);
    };
    const bool muon = s.rule == 2;
    take(0, muon ? 2 * NH * 3 * hid * d * 2 : 0);   // Newton-Schulz iterate, bf16 ping-pong
    take(1, muon ? NH * 3 * d * d * 2 : 0);         // Gram matrices, bf16
    take(13, muon ? NH * 3 * d * 4 : 0);            // first Gram diagonal, fp32
    take(2, s.loss == 1 ? NH * cpad * d * 2 : 0);  // dy
    take(3, (size_t)nslots * NH * 2 * 2 * hid * d * 2);  // w13b (hi, lo)
    take(4, (size_t)nslots * NH * 2 * d * hid * 2);      // w2b (hi, lo)
    take(5, NH * hid * cpad * 2);               // gt
    take(6, NH * hid * cpad * 2);               // dh1t
    take(7, NH * hid * cpad * 2);               // dh3t
    take(8, NH * 2 * qpad * hid * 2);           // gq (hi, lo)
    take(9, (size_t)splitk * NH * 3 * hid * d * 4);  // gradient partials
    pl.off[10] = (size_t)splitk;
    pl.off[11] = (size_t)nslots;
    pl.off[12] = cpad;
    pl.off[14] = qpad;
    pl.off[15] = (size_t)chunk;
    pl.bytes = off;
    return pl;
}

hipError_t lact_launch(const LactShape &s, const LactPlan &pl, const void *q, const void *k,
                       const void *v, const float *eta, const float *w1, const float *w2,
                       const float *w3, void *out, float *w1f, float *w2f, float *w3f, void *ws,
                       hipStream_t st, hipStream_t aux, float *m1, float *m2, float *m3)
{
    LactParams p;
    char *base = (char *)ws;
    p.q = (const bf16 *)q;
    p.k = (const bf16 *)k;
    p.v = (const bf16 *)v;
    p.eta = eta;
    p.w1i = w1;
    p.w2i = w2;
    p.w3i = w3;
    p.out = (bf16 *)out;
    p.w1 = w1f;
    p.w2 = w2f;
    p.w3 = w3f;
    p.NH = s.NH;
    p.Tq = s.Tq;
    p.Tkv = s.Tkv;
    p.d = s.d;
    p.hid = s.hid;
    p.chunk = (int)pl.off[15];
    p.nchunks = pl.nchunks;
    p.cpad = (int)pl.off[12];
    p.qpad = (int)pl.off[14];
    p.loss = s.loss;
    p.order = s.order;
    p.rownorm = s.rownorm;
    p.splitk = (int)pl.off[10];
    p.nslots = (int)pl.off[11];
    p.dy = (bf16 *)(base + pl.off[2]);
    p.w13b = (bf16 *)(base + pl.off[3]);
    p.w2b = (bf16 *)(base + pl.off[4]);
    p.gt = (bf16 *)(base + pl.off[5]);
    p.dh1t = (bf16 *)(base + pl.off[6]);
    p.dh3t = (bf16 *)(base + pl.off[7]);
    p.gq = (bf16 *)(base + pl.off[8]);
    p.part = (float *)(base + pl.off[9]);
    p.rule = s.rule;
    p.beta = s.beta;
    p.lr = s.lr;
    p.m1 = m1;
    p.m2 = m2;
    p.m3 = m3;
    p.nsb = (bf16 *)(base + pl.off[0]);
    p.gram = (bf16 *)(base + pl.off[1]);
    p.diag = (float *)(base + pl.off[13]);
    p.save_w = s.save_w;
    p.save_d = s.save_d;

    const long n3 = (long)s.NH * 3 * s.hid * s.d;
    const int wblocks = (int)((n3 + 255) / 256 < 4096 ? (n3 + 255) / 256 : 4096);
    lact_prep_weights<<<dim3(wblocks), dim3(256), 0, st>>>(p);
    const int t13 = (s.d / 128) * (s.hid / 128);
    const int urows = s.NH * (2 * s.hid + s.d);
    // Causal, inner-product loss: the queries of chunk c read the weights the
    // chunk starts with, so their two apply GEMMs can run on the caller's
    // second stream `aux` as soon as those weights exist, beside the
    // (latency-bound) update chain of the later chunks; `st` waits for them at
    // the end.  Two events, made for this call and released at its end, order
    // the streams.  Without `aux`, or while `st` is being captured into a
    // graph, every launch stays on `st` and the applies run after the chain.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cap) != hipSuccess) cap = hipStreamCaptureStatusActive;
    bool use_aux = aux && aux != st && s.order == 0 && s.loss == 0 && s.Tq > 0 &&
                   cap == hipStreamCaptureStatusNone;
    hipEvent_t ready = nullptr, done = nullptr;
    if (use_aux) {
        hipError_t e = hipEventCreateWithFlags(&ready, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&done, hipEventDisableTiming);
        if (e != hipSuccess) {
            if (ready) (void)hipEventDestroy(ready);
            return e;
        }
    }
    hipError_t serr = hipSuccess;  // first failure of an event call: the result is then invalid
    auto chk = [&](hipError_t e) {
        if (e != hipSuccess && serr == hipSuccess) serr = e;
    };
    // The queries of chunks [c0, c0 + n) in one pair of launches (each tile
    // reads its own chunk's weights), as soon as the last of those weights
    // exist.  One chunk per group: grouping two (twice the workgroups per
    // launch) measured slower on the causal LM workload (1.14 -> 1.27 ms), the
    // larger launches taking compute units from the update chain, which is the
    // critical path.
    constexpr int APPLY_GROUP = 1;
    const int nq = use_aux ? (s.Tq + p.chunk - 1) / p.chunk : 0;
    int next_q = 0;  // first chunk whose queries are not yet enqueued
    auto apply_ready = [&](int slots_ready) {
        while (next_q < nq) {
            const int n = (next_q + APPLY_GROUP <= nq) ? APPLY_GROUP : nq - next_q;
            if (next_q + n - 1 > slots_ready) break;
            chk(hipEventRecord(ready, st));
            chk(hipStreamWaitEvent(aux, ready, 0));
            const int q0 = next_q * p.chunk;
            const int qlen = ((next_q + n) * p.chunk <= s.Tq ? n * p.chunk : s.Tq - q0);
            lact_apply1<<<dim3(s.NH * ((2 * s.hid) / 128) * ((qlen + 127) / 128)), dim3(256), 0, aux>>>(
                p, p.q + (long)q0 * s.d, (long)s.Tq * s.d, qlen, -1, next_q);
            lact_apply2<<<dim3(s.NH * (s.d / 128) * ((qlen + 127) / 128)), dim3(256), 0, aux>>>(
                p, qlen, -1, 0, next_q, next_q);
            next_q += n;
        }
    };
    apply_ready(0);
    for (int c = 0; c < pl.nchunks; ++c) {
        const int slot = (s.order == 0) ? c : 0;
        const int dst = (s.order == 0) ? c + 1 : 0;
        const int clen = (c + 1) * p.chunk <= s.Tkv ? p.chunk : s.Tkv - c * p.chunk;
        if (s.loss == 1) {
            // dY = eta (f(K_c) - V_c): G of the chunk's keys, then W2.
            lact_apply1<<<dim3(s.NH * ((2 * s.hid) / 128) * ((clen + 127) / 128)), dim3(256), 0, st>>>(
                p, p.k + (long)c * p.chunk * s.d, (long)s.Tkv * s.d, clen, slot, 0);
            lact_apply2<<<dim3(s.NH * (s.d / 128) * ((clen + 127) / 128)), dim3(256), 0, st>>>(
                p, clen, slot, 1, c, 0);
        }
        lact_fwdgrad<FWD_NW><<<dim3(s.NH * (p.cpad / 128) * (s.hid / 128)), dim3(64 * FWD_NW), 0, st>>>(p, c, slot);
        lact_wgrad<<<dim3(s.NH * p.splitk * 3 * t13), dim3(256), 0, st>>>(p, c);
        if (s.rule == 2) {
            lact_update<<<dim3((urows + 3) / 4), dim3(256), 0, st>>>(p, dst, 1);
            for (int j = 0; j < s.ns_steps; ++j) {
                lact_ns_gram<<<dim3(s.NH * 3 * (s.d / NSBM) * (s.d / 128)), dim3(256), 0, st>>>(p, j);
                lact_ns_apply<<<dim3(s.NH * 3 * (s.hid / NSBM) * (s.d / 128)), dim3(256), 0, st>>>(p, j);
            }
        }
        p.save_c = c;
        lact_update<<<dim3((urows + 3) / 4), dim3(256), 0, st>>>(p, dst, 0);
        apply_ready(c + 1);
    }
    if (use_aux) {
        chk(hipEventRecord(done, aux));
        chk(hipStreamWaitEvent(st, done, 0));
        // released once the device has passed them (the waits stay enqueued)
        chk(hipEventDestroy(ready));
        chk(hipEventDestroy(done));
    } else if (s.Tq > 0) {
        const int fixed = (s.order == 0) ? -1 : 0;
        lact_apply1<<<dim3(s.NH * ((2 * s.hid) / 128) * ((s.Tq + 127) / 128)), dim3(256), 0, st>>>(
            p, p.q, (long)s.Tq * s.d, s.Tq, fixed, 0);
        lact_apply2<<<dim3(s.NH * (s.d / 128) * ((s.Tq + 127) / 128)), dim3(256), 0, st>>>(
            p, s.Tq, fixed, 0, 0, 0);
    }
    if (serr != hipSuccess) return serr;
    return hipGetLastError();
}

}  // namespace tttk
