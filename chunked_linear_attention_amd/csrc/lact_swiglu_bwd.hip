// LaCT SwiGLU backward on gfx950: the gradients of a scalar loss through
// lact_swiglu_fwd (inner-product loss, gradient descent, with or without the
// row rescale, either order) with respect to Q, K, V, eta and the initial
// weights, given the upstream gradients of the outputs and of the final
// weights.
//
// What is differentiated ("LaCT: Test-Time Training Done Right", sections 3.2,
// 3.3, 4; the pages train the layer end to end but give no backward): per
// chunk c, with chunk-start weights W_c, the summed gradient D_c of
// sum_t eta_t L_t, L_t = -f(k_t) . v_t, the step U = W_c - D_c and the row
// rescale W_{c+1}[r] = U[r] |W_c[r]| / |U[r]|; the causal queries of chunk c
// read W_c, the non-causal queries read the final weights.  Reverse mode of
// those steps (rows are tokens; H1 = K W1^T, H3 = K W3^T, A = silu(H1),
// A' = silu'(H1), A'' = silu''(H1), G = A * H3, dY = -eta V, dG = dY W2,
// dH1 = dG * H3 * A', dH3 = dG * A):
//   step:  n = |W_c[r]|, m = |U[r]|, Lam = adjoint of W_{c+1}[r]:
//          bar_U = (n/m) Lam - (U . Lam) n U / m^3,
//          bar_W_c = bar_U + (U . Lam) / (m n) W_c[r],   Gam = -bar_U
//   D's reverse (Gam = adjoint of D):  P1 = K Gam1^T, P3 = K Gam3^T, P2 = dY Gam2,
//          bar_dG = P1 H3 A' + P3 A,  bar_H3 = P1 dG A' + P2 A,
//          bar_H1 = P1 dG H3 A'' + (P3 dG + P2 H3) A',
//          bar_W1 += bar_H1^T K, bar_W3 += bar_H3^T K, bar_W2 += dY^T bar_dG,
//          bar_K = dH1 Gam1 + dH3 Gam3 + bar_H1 W1 + bar_H3 W3,
//          bar_dY = G Gam2^T + bar_dG W2^T,  bar_V = -eta bar_dY,
//          bar_eta = -rowsum(bar_dY * V)
//   apply's reverse (rows X, upstream dO):  bar_G = dO W2,  bar_W2 += dO^T G,
//          bar_H3 = bar_G A, bar_H1 = bar_G H3 A',  bar_W1 += bar_H1^T X,
//          bar_W3 += bar_H3^T X,  bar_X = bar_H1 W1 + bar_H3 W3
//
// Schedule: a replay of the forward (no applies) saves every chunk's start
// weights and step direction; then, chunk by chunk in reverse, one row kernel
// takes the step's reverse (and writes bf16 copies of W_c and Gam as matrix
// operands), every product above runs as a head-batched bf16 MFMA GEMM on the
// shared tile (fp32 accumulation; the weight adjoints accumulate in fp32), and
// two elementwise kernels form the SwiGLU terms.  Precision: every operand
// that is not an exact bf16 input (weights, Gam, dY, the SwiGLU terms) enters
// as a bf16 pair hi = bf16(x), lo = bf16(x - hi), and each product sums
// hi*hi + lo*hi + hi*lo: the gradients are heavy-tailed (their largest
// elements reach 10-18 times their RMS), and one bf16 rounding per operand
// moves those elements by several percent of the RMS.
#include "lact_common.h"
#include "ttt_internal.h"

namespace tttk {

// ---------------------------------------------------------------------------
// Head-batched GEMM on the shared tile: for every head h,
//   C_h[m][n] (op)= sum_s sum_k A_s,h[m][k] B_s,h[n][k]
// with the operand layouts of gemm_nt_tile (AT / BT: k-major).  out: 0 store
// fp32, 1 add into fp32, 2 store bf16.  Rows m >= M and columns n >= N are not
// written.  With P set the output goes to fp32 partials instead.  Split-K
// (ksplit > 1, P set): workgroup ks takes either the k rows
// [ks kper, (ks + 1) kper) of every segment (split_rows, both operands
// k-major) or the segments [ks nseg/ksplit, (ks + 1) nseg/ksplit), and stores
// its fp32 partial at P + ks p_ss + h p_hs + m ldc + n; a reduction kernel
// sums the partials in split order (the result does not depend on timing).
// ---------------------------------------------------------------------------
constexpr int BWD_MAXSEG = 12;
struct BwdGemm {
    const bf16 *A[BWD_MAXSEG];
    const bf16 *B[BWD_MAXSEG];
    long a_hs, b_hs, lda, ldb;   // head strides and leading dimensions (elements)
    int M, N, kseg, nseg, kvalid;
    float *C;
    bf16 *Cb;
    long c_hs, ldc;
    int out;
    int ksplit, split_rows, kper;
    float *P;
    long p_ss, p_hs;
};

// Operand of segment s of a job: the job's pointer for segment s0 + s (read
// from the kernel arguments with a scalar load when the tile needs it, so the
// twelve segment pointers never occupy registers) at head h and k offset.
struct BwdSegPtr {
    const bf16 *const *p;
    int s0;
    long off;
    __device__ __forceinline__ const bf16 *operator[](int s) const { return p[s0 + s] + off; }
};

template <bool AT, bool BT>
__global__ __launch_bounds__(256) void lbk_gemm(BwdGemm j)
{
    __shared__ GemmLds L;
    const int tm_n = (j.M + 127) / 128, tn_n = (j.N + 127) / 128;
    int bid = xcd_block(blockIdx.x, gridDim.x);
    const int ks = bid % j.ksplit;
    bid /= j.ksplit;
    const int tn = bid % tn_n;
    bid /= tn_n;
    const int tm = bid % tm_n;
    const int h = bid / tm_n;
    int s0 = 0, ns = j.nseg, kseg = j.kseg, kvalid = j.kvalid;
    long koff_a = 0, koff_b = 0;
    if (j.ksplit > 1) {
        if (j.split_rows) {
            const int k0 = ks * j.kper;
            kseg = j.kper;
            kvalid = min(j.kper, j.kvalid - k0);
            koff_a = (long)k0 * j.lda;
            koff_b = (long)k0 * j.ldb;
        } else {
            ns = j.nseg / j.ksplit;
            s0 = ks * ns;
        }
    }
    const BwdSegPtr as{j.A, s0, (long)h * j.a_hs + koff_a}, bs{j.B, s0, (long)h * j.b_hs + koff_b};
    float *P = j.P ? j.P + (long)ks * j.p_ss + (long)h * j.p_hs : nullptr;
    float *C = j.C ? j.C + (long)h * j.c_hs : nullptr;
    bf16 *Cb = j.Cb ? j.Cb + (long)h * j.c_hs : nullptr;
    if (P && kvalid <= 0) {
        // an empty k range contributes zero (the partial is still written)
        for (int e = threadIdx.x; e < 128 * 128; e += 256) {
            const int m = tm * 128 + (e >> 7), n = tn * 128 + (e & 127);
            if (m < j.M && n < j.N) P[(long)m * j.ldc + n] = 0.f;
        }
        return;
    }
    gemm_nt_tile<AT, BT>(L, as, j.lda, bs, j.ldb, j.M, j.N, kseg, ns, tm * 128, tn * 128, kvalid,
                         [&](f32x4 (&acc)[4][4], int mb, int nb, int g, int mm) {
#pragma unroll
                             for (int i = 0; i < 4; ++i)
#pragma unroll
                                 for (int q = 0; q < 4; ++q) {
                                     const int n = nb + 16 * q + mm;
                                     if (n >= j.N) continue;
#pragma unroll
                                     for (int r = 0; r < 4; ++r) {
                                         const int m = mb + 16 * i + 4 * g + r;
                                         if (m >= j.M) continue;
                                         const long o = (long)m * j.ldc + n;
                                         if (P)
                                             P[o] = acc[i][q][r];
                                         else if (j.out == 0)
                                             C[o] = acc[i][q][r];
                                         else if (j.out == 1)
                                             C[o] += acc[i][q][r];
                                         else
                                             Cb[o] = (bf16)acc[i][q][r];
                                     }
                                 }
                         });
}

// Sum of ksplit fp32 partial planes in split order, four consecutive elements
// per thread with up to eight planes' loads in flight at once (the adds keep
// the order k = 0, 1, ..., so the result is the same as one plane at a time).
__device__ __forceinline__ f32x4 red_planes(const float *P, int ksplit, long stride, long e)
{
    f32x4 x = zero4();
    for (int k0 = 0; k0 < ksplit; k0 += 8) {
        f32x4 v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = (k0 + k < ksplit) ? load4<float>(P + (long)(k0 + k) * stride + e) : zero4();
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (k0 + k < ksplit) x += v[k];
    }
    return x;
}

// lam[i] += sum_ks P[ks stride + i], in split order (n and stride multiples
// of 4, 16-byte aligned planes)
__global__ __launch_bounds__(256) void lbk_red_add(const float *P, int ksplit, long stride, float *lam, long n)
{
    for (long i = 4 * ((long)blockIdx.x * 256 + threadIdx.x); i < n; i += 4 * (long)gridDim.x * 256)
        store4<float>(lam + i, load4<float>(lam + i) + red_planes(P, ksplit, stride, i));
}

// out[h][t][i] = sum_ks P[ks stride + (h rpad + t) d + i] for t < rows; out as
// bf16 (ob, head stride o_hs) or fp32 (of, same layout as the partials); d and
// stride multiples of 4
__global__ __launch_bounds__(256) void lbk_red_rows(const float *P, int ksplit, long stride, int NH, int rows,
                                                    int rpad, int d, bf16 *ob, long o_hs, float *of)
{
    const long n = (long)NH * rows * d;
    for (long i = 4 * ((long)blockIdx.x * 256 + threadIdx.x); i < n; i += 4 * (long)gridDim.x * 256) {
        const int h = (int)(i / ((long)rows * d));
        const long r = i % ((long)rows * d);
        const long src = (long)h * rpad * d + r;
        const f32x4 x = red_planes(P, ksplit, stride, src);
        if (ob)
            store4<bf16>(ob + (long)h * o_hs + r, to_bf16x4(x));
        else
            store4<float>(of + src, x);
    }
}

// ---------------------------------------------------------------------------
// Step reverse, one wave per row of W1, W3 (length d) or W2 (length hid), in
// the update kernel's order: per head rows [0, hid) of W1, [hid, 2 hid) of
// W3, then d rows of W2.  lam (fp32 [NH][3][hid d], in place): the adjoint of
// the stepped weights on entry, that of W_c through the step's direct path on
// exit.  gam, wcb (bf16 [2][NH][3][hid d], hi then lo): -bar_U and W_c as
// matrix operand pairs.
// ---------------------------------------------------------------------------
struct BwdStep {
    const float *w, *dir;   // chunk-start weights and the step direction (saved by the replay)
    float *lam;
    bf16 *gam, *wcb;
    int NH, d, hid, rownorm;
};

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (x - hi is exact in fp32)
__device__ __forceinline__ void put_pair(bf16 *base, long lo_off, long i, float x)
{
    const bf16 hi = (bf16)x;
    base[i] = hi;
    base[lo_off + i] = (bf16)(x - (float)hi);
}

__device__ __forceinline__ float wsum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__global__ __launch_bounds__(256) void lbk_step(BwdStep p)
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
    const long off = ((long)h * 3 + which) * n13 + (long)row * len;
    constexpr int MAXE = 16;  // len <= 1024
    float wv[MAXE], uv[MAXE], lv[MAXE];
    float nn = 0.f, mm = 0.f, ul = 0.f;
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        const int col = lane + 64 * e;
        wv[e] = uv[e] = lv[e] = 0.f;
        if (col < len) {
            wv[e] = p.w[off + col];
            uv[e] = wv[e] - p.dir[off + col];
            lv[e] = p.lam[off + col];
            nn += wv[e] * wv[e];
            mm += uv[e] * uv[e];
            ul += uv[e] * lv[e];
        }
    }
    float s = 1.f, cu = 0.f, cw = 0.f;  // bar_U = s lam - cu U;  bar_W = bar_U + cw W
    if (p.rownorm) {
        nn = wsum(nn);
        mm = wsum(mm);
        ul = wsum(ul);
        if (mm > 0.f) {
            const float n = sqrtf(nn), m = sqrtf(mm);
            s = n / m;
            cu = ul * n / (m * m * m);
            cw = (nn > 0.f) ? ul / (m * n) : 0.f;
        }
    }
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        const int col = lane + 64 * e;
        if (col < len) {
            const float bu = s * lv[e] - cu * uv[e];
            p.lam[off + col] = bu + cw * wv[e];
            const long lo = (long)p.NH * 3 * n13;
            put_pair(p.gam, lo, off + col, -bu);
            put_pair(p.wcb, lo, off + col, wv[e]);
        }
    }
}

// fp32 weights (W1, W3 [hid][d], W2 [d][hid] per head) -> bf16 pairs [2][NH][3][hid d]
__global__ __launch_bounds__(256) void lbk_cvt(const float *w1, const float *w2, const float *w3,
                                               bf16 *dst, int NH, long n13)
{
    const long total = (long)NH * 3 * n13;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int h = (int)(i / (3 * n13));
        const long r = i % (3 * n13);
        const int which = (int)(r / n13);
        const long e = r % n13;
        const float *src = which == 0 ? w1 : which == 1 ? w3 : w2;
        put_pair(dst, total, i, src[(long)h * n13 + e]);
    }
}

// fp32 [NH][3][hid d] in the update's order -> the caller's W1, W2, W3 layouts
__global__ __launch_bounds__(256) void lbk_split(const float *lam, float *d1, float *d2, float *d3,
                                                 int NH, long n13)
{
    const long total = (long)NH * 3 * n13;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int h = (int)(i / (3 * n13));
        const long r = i % (3 * n13);
        const int which = (int)(r / n13);
        const long e = r % n13;
        float *dst = which == 0 ? d1 : which == 1 ? d3 : d2;
        dst[(long)h * n13 + e] = lam[i];
    }
}

// the caller's d_w_final (or zero) -> lam [NH][3][hid d]
__global__ __launch_bounds__(256) void lbk_lam_init(const float *d1, const float *d2, const float *d3,
                                                    float *lam, int NH, long n13)
{
    const long total = (long)NH * 3 * n13;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int h = (int)(i / (3 * n13));
        const long r = i % (3 * n13);
        const int which = (int)(r / n13);
        const long e = r % n13;
        const float *src = which == 0 ? d1 : which == 1 ? d3 : d2;
        lam[i] = src ? src[(long)h * n13 + e] : 0.f;
    }
}

// dY = -eta V of a chunk, bf16 pairs [2][NH][rpad][d]; rows past the chunk are zero
__global__ __launch_bounds__(256) void lbk_dy(const bf16 *v, const float *eta, bf16 *dy, int NH, int Tkv,
                                              int c0, int clen, int rpad, int d)
{
    const long total = (long)NH * rpad * d;
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int h = (int)(i / ((long)rpad * d));
        const int t = (int)((i / d) % rpad);
        const int o = (int)(i % d);
        float x = 0.f;
        if (t < clen) {
            const long tk = (long)h * Tkv + c0 + t;
            x = -eta[tk] * (float)v[tk * d + o];
        }
        put_pair(dy, total, i, x);
    }
}

__device__ __forceinline__ void silu_terms(float z, float &a, float &a1, float &a2)
{
    const float s = 1.f / (1.f + __expf(-z));
    a = z * s;
    a1 = s * (1.f + z * (1.f - s));
    a2 = s * (1.f - s) * (2.f + z * (1.f - 2.f * s));
}

// D's reverse, elementwise over [rows][hid] per head (f: H1, H3, dG, P1, P3,
// P2 in fp32; e: dH1, dH3, G, bar_dG, bar_H1, bar_H3 as bf16 pairs, hi in
// planes 0..5, lo in planes 6..11); rows >= rows_valid are written as zero.
__global__ __launch_bounds__(256) void lbk_elem_vjp(const float *f, bf16 *e, long plane, int rpad, int hid,
                                                    int rows_valid, long total)
{
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int t = (int)((i / hid) % rpad);
        float v[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (t < rows_valid) {
            const float h1 = f[i], h3 = f[plane + i], dg = f[2 * plane + i];
            const float p1 = f[3 * plane + i], p3 = f[4 * plane + i], p2 = f[5 * plane + i];
            float a, a1, a2;
            silu_terms(h1, a, a1, a2);
            v[0] = dg * h3 * a1;                                // dH1
            v[1] = dg * a;                                      // dH3
            v[2] = a * h3;                                      // G
            v[3] = p1 * h3 * a1 + p3 * a;                       // bar_dG
            v[4] = p1 * dg * h3 * a2 + (p3 * dg + p2 * h3) * a1;  // bar_H1
            v[5] = p1 * dg * a1 + p2 * a;                       // bar_H3
        }
#pragma unroll
        for (int k = 0; k < 6; ++k) put_pair(e, 6 * plane, k * plane + i, v[k]);
    }
}

// the apply's reverse, elementwise (f: H1, H3, bar_G in fp32 planes 0..2; e:
// G -> plane 2, bar_H1 -> plane 4, bar_H3 -> plane 5, as the GEMMs read them)
__global__ __launch_bounds__(256) void lbk_elem_apply(const float *f, bf16 *e, long plane, int rpad, int hid,
                                                      int rows_valid, long total)
{
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
        const int t = (int)((i / hid) % rpad);
        float g = 0.f, b1 = 0.f, b3 = 0.f;
        if (t < rows_valid) {
            const float h1 = f[i], h3 = f[plane + i], bg = f[2 * plane + i];
            float a, a1, a2;
            silu_terms(h1, a, a1, a2);
            g = a * h3;
            b1 = bg * h3 * a1;
            b3 = bg * a;
        }
        put_pair(e, 6 * plane, 2 * plane + i, g);
        put_pair(e, 6 * plane, 4 * plane + i, b1);
        put_pair(e, 6 * plane, 5 * plane + i, b3);
    }
}

// d_v = -eta bar_dY (bf16) and d_eta = -sum_o bar_dY V (fp32), one wave per token
__global__ __launch_bounds__(256) void lbk_tok(const float *bdy, const bf16 *v, const float *eta, bf16 *dv,
                                               float *deta, int NH, int Tkv, int c0, int clen, int rpad, int d)
{
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (gw >= NH * clen) return;
    const int h = gw / clen, t = gw % clen;
    const long tk = (long)h * Tkv + c0 + t;
    const float e = eta[tk];
    const float *row = bdy + ((long)h * rpad + t) * d;
    float s = 0.f;
    for (int o = lane; o < d; o += 64) {
        const float b = row[o];
        s += b * (float)v[tk * d + o];
        dv[tk * d + o] = (bf16)(-e * b);
    }
    s = wsum(s);
    if (lane == 0) deta[tk] = -s;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static size_t al256b(size_t x) { return (x + 255) / 256 * 256; }

// split-K limits: contractions over tokens (the weight adjoints) into at most
// 16 token ranges, the ones over the hidden units (token-side adjoints) into
// at most 4 groups of segments
constexpr int BWD_KS_W = 16, BWD_KS_T = 4;

LactBwdPlan lact_bwd_plan(const LactShape &s)
{
    LactBwdPlan pl{};
    LactShape f = s;
    f.Tq = 0;  // the replay runs no applies
    pl.fwd = lact_plan(f);
    const int chunk = pl.fwd.off[15] ? (int)pl.fwd.off[15] : s.chunk;
    const size_t cpad = pl.fwd.off[12];
    const size_t qrows = (s.order == 1) ? (size_t)((s.Tq + 127) / 128 * 128) : cpad;
    pl.rpad = (int)(cpad > qrows ? cpad : qrows);
    pl.chunk = chunk;
    const size_t NH = s.NH, n13 = (size_t)s.hid * s.d, nc = pl.fwd.nchunks;
    size_t off = al256b(pl.fwd.bytes);
    auto take = [&](size_t &o, size_t bytes) {
        o = off;
        off = al256b(off + bytes);
    };
    take(pl.o_save_w, nc * NH * 3 * n13 * 4);
    take(pl.o_save_d, nc * NH * 3 * n13 * 4);
    take(pl.o_wfin, 3 * NH * n13 * 4);
    take(pl.o_lam, NH * 3 * n13 * 4);
    take(pl.o_gam, 2 * NH * 3 * n13 * 2);                      // hi, lo
    take(pl.o_wcb, 2 * NH * 3 * n13 * 2);                      // hi, lo
    take(pl.o_f, 6 * NH * (size_t)pl.rpad * s.hid * 4);
    take(pl.o_e, 12 * NH * (size_t)pl.rpad * s.hid * 2);       // 6 planes, hi then lo
    take(pl.o_dy, 2 * NH * cpad * s.d * 2);                    // hi, lo
    take(pl.o_bdy, NH * (size_t)pl.rpad * s.d * 4);
    const size_t pw = (size_t)BWD_KS_W * NH * 3 * n13, pt = (size_t)BWD_KS_T * NH * pl.rpad * s.d;
    take(pl.o_part, 4 * (pw > pt ? pw : pt));
    pl.bytes = off;
    return pl;
}

template <bool AT, bool BT>
static void run_gemm(const BwdGemm &j, int NH, hipStream_t st)
{
    const int grid = NH * ((j.M + 127) / 128) * ((j.N + 127) / 128) * j.ksplit;
    if (grid > 0 && j.nseg > 0) lbk_gemm<AT, BT><<<dim3(grid), dim3(256), 0, st>>>(j);
}

// Token-range split of a contraction over ntok tokens (both operands
// k-major): enough splits to give about one workgroup per compute unit, each
// a whole number of 64-token steps, at most BWD_KS_W.  Returns the split count.
static int split_tokens(BwdGemm &j, int NH, int ntok)
{
    const int tiles = NH * ((j.M + 127) / 128) * ((j.N + 127) / 128);
    int ks = 256 / (tiles > 0 ? tiles : 1);
    ks = ks < 1 ? 1 : (ks > BWD_KS_W ? BWD_KS_W : ks);
    const int kper = ((ntok + ks - 1) / ks + 63) / 64 * 64;
    j.ksplit = (ntok + kper - 1) / kper;
    j.split_rows = 1;
    j.kper = kper;
    return j.ksplit;
}

static unsigned ew_grid(long n) { return (unsigned)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192); }
// grid of the four-element reductions
static unsigned ew_grid4(long n) { return ew_grid((n + 3) / 4); }

static BwdGemm gemm_job(int M, int N, int kseg, int kvalid, long lda, long a_hs, long ldb, long b_hs)
{
    BwdGemm j{};
    j.M = M;
    j.N = N;
    j.kseg = kseg;
    j.nseg = 0;
    j.ksplit = 1;
    j.kvalid = kvalid;
    j.lda = lda;
    j.a_hs = a_hs;
    j.ldb = ldb;
    j.b_hs = b_hs;
    return j;
}

// Adds the product A B to a job as its segments: A and B are hi parts, alo and
// blo their lo parts (null for an exact bf16 operand): hi*hi + lo*hi + hi*lo.
static void add_prod(BwdGemm &j, const bf16 *a, const bf16 *alo, const bf16 *b, const bf16 *blo)
{
    j.A[j.nseg] = a;
    j.B[j.nseg++] = b;
    if (alo) {
        j.A[j.nseg] = alo;
        j.B[j.nseg++] = b;
    }
    if (blo) {
        j.A[j.nseg] = a;
        j.B[j.nseg++] = blo;
    }
}

struct BwdBufs {
    const bf16 *wcb, *wcb_lo;   // bf16 pairs of the weights the step reads, [NH][3][hid d] each
    float *lam, *F;
    bf16 *E;                    // 6 planes hi, then 6 planes lo
    long plane;
    float *part;                // split-K partials
};

// The three weight-adjoint GEMMs of a phase (W1, W3: hid x d; W2: d x hid) add
// into lam: split over token ranges when that fills the chip (partials, then
// one ordered reduction for all three), else added directly.
static void weight_adjoints(BwdGemm (&jobs)[3], const BwdBufs &b, int NH, long n13, int ntok, hipStream_t st)
{
    int ks = 1;
    for (int x = 0; x < 3; ++x) ks = split_tokens(jobs[x], NH, ntok);
    for (int x = 0; x < 3; ++x) {
        BwdGemm &j = jobs[x];
        if (ks > 1) {
            j.P = b.part + (x == 2 ? 2 : x) * n13;
            j.p_ss = (long)NH * 3 * n13;
            j.p_hs = 3 * n13;
        } else {
            j.ksplit = 1;
        }
        run_gemm<true, true>(j, NH, st);
    }
    if (ks > 1) {
        const long n = (long)NH * 3 * n13;
        lbk_red_add<<<dim3(ew_grid4(n)), dim3(256), 0, st>>>(b.part, ks, n, b.lam, n);
    }
}

// A token-side product over the hidden units (its segments in groups of three,
// one group per product), split into one group per workgroup; the ordered sum
// goes to bf16 rows of an output [NH][.][d] (ob, head stride o_hs) or to fp32
// rows [NH][rpad][d] (of).
template <bool BT>
static void token_side(BwdGemm &j, const BwdBufs &b, const LactBwdPlan &pl, int NH, int rows, int d, bf16 *ob,
                       long o_hs, float *of, hipStream_t st)
{
    // every product here has two bf16-pair operands: three segments each
    j.ksplit = (j.nseg % 3 == 0 && j.nseg / 3 <= BWD_KS_T) ? j.nseg / 3 : 1;
    j.split_rows = 0;
    j.P = b.part;
    j.p_hs = (long)pl.rpad * d;
    j.p_ss = (long)NH * pl.rpad * d;
    j.ldc = d;
    run_gemm<false, BT>(j, NH, st);
    const long n = (long)NH * rows * d;
    lbk_red_rows<<<dim3(ew_grid4(n)), dim3(256), 0, st>>>(b.part, j.ksplit, j.p_ss, NH, rows, pl.rpad, d, ob, o_hs,
                                                         of);
}

// The apply's reverse for rows X (x0 .. x0 + rows of q, upstream dout) at the
// weights whose bf16 pairs are in b.wcb: d_q rows, and the weight adjoints
// added into lam.  F planes 0..2 and E planes 2, 4, 5 are used as scratch.
static void apply_bwd(const LactShape &s, const LactBwdPlan &pl, const BwdBufs &b, const bf16 *q,
                      const bf16 *dout, bf16 *dq, int x0, int rows, hipStream_t st)
{
    const int NH = s.NH, d = s.d, hid = s.hid;
    const long n13 = (long)hid * d, plane = b.plane;
    const long x_hs = (long)s.Tq * d, f_hs = (long)pl.rpad * hid, w_hs = 3 * n13;
    const bf16 *X = q + (long)x0 * d, *DO = dout + (long)x0 * d;
    const bf16 *E = b.E, *El = b.E + 6 * plane;
    // H1 = X W1^T, H3 = X W3^T, bar_G = dO W2
    for (int k = 0; k < 3; ++k) {
        const long wo = (k == 0 ? 0 : k == 1 ? n13 : 2 * n13);
        BwdGemm j = gemm_job(rows, hid, d, d, d, x_hs, k == 2 ? hid : d, w_hs);
        add_prod(j, k == 2 ? DO : X, nullptr, b.wcb + wo, b.wcb_lo + wo);
        j.C = b.F + k * plane;
        j.c_hs = f_hs;
        j.ldc = hid;
        j.out = 0;
        if (k == 2) run_gemm<false, true>(j, NH, st);
        else run_gemm<false, false>(j, NH, st);
    }
    const long tot = (long)NH * pl.rpad * hid;
    lbk_elem_apply<<<dim3((unsigned)((tot + 255) / 256 < 8192 ? (tot + 255) / 256 : 8192)), dim3(256), 0, st>>>(
        b.F, b.E, plane, pl.rpad, hid, rows, tot);
    const int kseg = (rows + 63) / 64 * 64;
    // lam_W1 += bar_H1^T X, lam_W3 += bar_H3^T X, lam_W2 += dO^T G
    BwdGemm wj[3];
    for (int k = 0; k < 3; ++k) {
        const bool w2 = k == 2;
        BwdGemm &j = wj[k];
        j = gemm_job(w2 ? d : hid, w2 ? hid : d, kseg, rows, w2 ? d : hid, w2 ? x_hs : f_hs, w2 ? hid : d,
                     w2 ? f_hs : x_hs);
        if (w2)
            add_prod(j, DO, nullptr, E + 2 * plane, El + 2 * plane);
        else
            add_prod(j, E + (k == 0 ? 4 : 5) * plane, El + (k == 0 ? 4 : 5) * plane, X, nullptr);
        j.C = b.lam + (w2 ? 2 : k) * n13;
        j.c_hs = w_hs;
        j.ldc = w2 ? hid : d;
        j.out = 1;
    }
    weight_adjoints(wj, b, NH, n13, rows, st);
    // d_q = bar_H1 W1 + bar_H3 W3
    BwdGemm j = gemm_job(rows, d, hid, hid, hid, f_hs, d, w_hs);
    add_prod(j, E + 4 * plane, El + 4 * plane, b.wcb, b.wcb_lo);
    add_prod(j, E + 5 * plane, El + 5 * plane, b.wcb + n13, b.wcb_lo + n13);
    token_side<true>(j, b, pl, NH, rows, d, dq + (long)x0 * d, x_hs, nullptr, st);
}

hipError_t lact_bwd_launch(const LactShape &s, const LactBwdPlan &pl, const void *q, const void *k,
                           const void *v, const float *eta, const float *w1, const float *w2, const float *w3,
                           const void *dout, const float *dw1f, const float *dw2f, const float *dw3f, void *dq,
                           void *dk, void *dv, float *deta, float *dw1, float *dw2, float *dw3, void *ws,
                           hipStream_t st)
{
    char *base = (char *)ws;
    const int NH = s.NH, d = s.d, hid = s.hid;
    const long n13 = (long)hid * d, wtot = (long)NH * 3 * n13;
    float *save_w = (float *)(base + pl.o_save_w), *save_d = (float *)(base + pl.o_save_d);
    float *wfin = (float *)(base + pl.o_wfin);
    float *lam = (float *)(base + pl.o_lam);
    bf16 *gam = (bf16 *)(base + pl.o_gam), *wcb = (bf16 *)(base + pl.o_wcb);
    const bf16 *gam_lo = gam + wtot, *wcb_lo = wcb + wtot;
    float *F = (float *)(base + pl.o_f);
    bf16 *E = (bf16 *)(base + pl.o_e);
    bf16 *DY = (bf16 *)(base + pl.o_dy);
    float *BDY = (float *)(base + pl.o_bdy);
    const bf16 *Q = (const bf16 *)q, *K = (const bf16 *)k, *V = (const bf16 *)v, *DO = (const bf16 *)dout;
    const long plane = (long)NH * pl.rpad * hid, f_hs = (long)pl.rpad * hid, w_hs = 3 * n13;
    const bf16 *El = E + 6 * plane;
    const int cpad = (int)pl.fwd.off[12];
    const unsigned wgrid = (unsigned)((wtot + 255) / 256 < 4096 ? (wtot + 255) / 256 : 4096);
    const BwdBufs bufs{wcb, wcb_lo, lam, F, E, plane, (float *)(base + pl.o_part)};

    // 1. the forward again (no applies), saving W_c and D_c of every chunk;
    //    its final weights land in wfin ([W1 all heads][W3 all heads][W2 all heads])
    LactShape f = s;
    f.Tq = 0;
    f.save_w = save_w;
    f.save_d = save_d;
    hipError_t e = lact_launch(f, pl.fwd, nullptr, k, v, eta, w1, w2, w3, nullptr, wfin, wfin + 2 * NH * n13,
                               wfin + NH * n13, base, st, nullptr);
    if (e != hipSuccess) return e;
    const float *wf1 = wfin, *wf3 = wfin + NH * n13, *wf2 = wfin + 2 * NH * n13;

    // 2. lam = d_w_final (or 0)
    lbk_lam_init<<<dim3(wgrid), dim3(256), 0, st>>>(dw1f, dw2f, dw3f, lam, NH, n13);

    // 3. non-causal: the queries read the final weights
    if (s.order == 1 && s.Tq > 0) {
        lbk_cvt<<<dim3(wgrid), dim3(256), 0, st>>>(wf1, wf2, wf3, wcb, NH, n13);
        apply_bwd(s, pl, bufs, Q, DO, (bf16 *)dq, 0, s.Tq, st);
    }

    // 4. chunks in reverse
    const int urows = NH * (2 * hid + d);
    for (int c = pl.fwd.nchunks - 1; c >= 0; --c) {
        const int c0 = c * pl.chunk;
        const int clen = (c0 + pl.chunk <= s.Tkv) ? pl.chunk : s.Tkv - c0;
        BwdStep sp{save_w + (long)c * NH * 3 * n13, save_d + (long)c * NH * 3 * n13, lam, gam, wcb, NH, d, hid,
                   s.rownorm};
        lbk_step<<<dim3((urows + 3) / 4), dim3(256), 0, st>>>(sp);
        const long dyt = (long)NH * cpad * d;
        lbk_dy<<<dim3((unsigned)((dyt + 255) / 256 < 8192 ? (dyt + 255) / 256 : 8192)), dim3(256), 0, st>>>(
            V, eta, DY, NH, s.Tkv, c0, clen, cpad, d);
        const bf16 *DYl = DY + dyt;
        const bf16 *Kc = K + (long)c0 * d;
        const long k_hs = (long)s.Tkv * d, dy_hs = (long)cpad * d;
        // H1, H3, dG, P1, P3, P2 (contractions over d)
        for (int x = 0; x < 6; ++x) {
            const bool onk = (x == 0 || x == 1 || x == 3 || x == 4);  // A = K, else A = dY
            const long wo = (x % 3 == 0 ? 0 : x % 3 == 1 ? n13 : 2 * n13);
            const bf16 *Bh = (x < 3 ? wcb : gam) + wo, *Bl = (x < 3 ? wcb_lo : gam_lo) + wo;
            BwdGemm j = gemm_job(clen, hid, d, d, d, onk ? k_hs : dy_hs, onk ? d : hid, w_hs);
            add_prod(j, onk ? Kc : DY, onk ? nullptr : DYl, Bh, Bl);
            j.C = F + x * plane;
            j.c_hs = f_hs;
            j.ldc = hid;
            j.out = 0;
            if (onk) run_gemm<false, false>(j, NH, st);
            else run_gemm<false, true>(j, NH, st);
        }
        const long tot = (long)NH * pl.rpad * hid;
        lbk_elem_vjp<<<dim3((unsigned)((tot + 255) / 256 < 8192 ? (tot + 255) / 256 : 8192)), dim3(256), 0, st>>>(
            F, E, plane, pl.rpad, hid, clen, tot);
        // lam_W1 += bar_H1^T K, lam_W3 += bar_H3^T K, lam_W2 += dY^T bar_dG
        const int kseg = (clen + 63) / 64 * 64;
        BwdGemm wj[3];
        for (int x = 0; x < 3; ++x) {
            const bool w2m = x == 2;
            BwdGemm &j = wj[x];
            j = gemm_job(w2m ? d : hid, w2m ? hid : d, kseg, clen, w2m ? d : hid, w2m ? dy_hs : f_hs,
                         w2m ? hid : d, w2m ? f_hs : k_hs);
            if (w2m)
                add_prod(j, DY, DYl, E + 3 * plane, El + 3 * plane);
            else
                add_prod(j, E + (x == 0 ? 4 : 5) * plane, El + (x == 0 ? 4 : 5) * plane, Kc, nullptr);
            j.C = lam + (w2m ? 2 : x) * n13;
            j.c_hs = w_hs;
            j.ldc = w2m ? hid : d;
            j.out = 1;
        }
        weight_adjoints(wj, bufs, NH, n13, clen, st);
        // d_k = dH1 Gam1 + dH3 Gam3 + bar_H1 W1 + bar_H3 W3 (this chunk's rows)
        {
            BwdGemm j = gemm_job(clen, d, hid, hid, hid, f_hs, d, w_hs);
            add_prod(j, E, El, gam, gam_lo);
            add_prod(j, E + plane, El + plane, gam + n13, gam_lo + n13);
            add_prod(j, E + 4 * plane, El + 4 * plane, wcb, wcb_lo);
            add_prod(j, E + 5 * plane, El + 5 * plane, wcb + n13, wcb_lo + n13);
            token_side<true>(j, bufs, pl, NH, clen, d, (bf16 *)dk + (long)c0 * d, k_hs, nullptr, st);
        }
        // bar_dY = G Gam2^T + bar_dG W2^T, then d_v and d_eta
        {
            BwdGemm j = gemm_job(clen, d, hid, hid, hid, f_hs, hid, w_hs);
            add_prod(j, E + 2 * plane, El + 2 * plane, gam + 2 * n13, gam_lo + 2 * n13);
            add_prod(j, E + 3 * plane, El + 3 * plane, wcb + 2 * n13, wcb_lo + 2 * n13);
            token_side<false>(j, bufs, pl, NH, clen, d, nullptr, 0, BDY, st);
            lbk_tok<<<dim3((NH * clen + 3) / 4), dim3(256), 0, st>>>(BDY, V, eta, (bf16 *)dv, deta, NH, s.Tkv, c0,
                                                                     clen, pl.rpad, d);
        }
        // causal: the chunk's queries read W_c
        if (s.order == 0 && c0 < s.Tq) {
            const int rows = (c0 + clen <= s.Tq) ? clen : s.Tq - c0;
            apply_bwd(s, pl, bufs, Q, DO, (bf16 *)dq, c0, rows, st);
        }
    }
    // 5. d_w_init = lam
    lbk_split<<<dim3(wgrid), dim3(256), 0, st>>>(lam, dw1, dw2, dw3, NH, n13);
    return hipGetLastError();
}

}  // namespace tttk
