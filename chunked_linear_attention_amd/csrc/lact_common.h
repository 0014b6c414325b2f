// Pieces shared by the LaCT SwiGLU forward (lact_swiglu.hip) and backward
// (lact_swiglu_bwd.hip) kernels: 16-byte vector helpers, the bf16 MFMA wrapper,
// the generic GEMM tile and the parameter block of a LaCT call.
#pragma once

#include "ttt_device.h"

namespace tttk {

typedef __bf16 bf16;
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

// 16 bytes = 8 bf16
struct alignas(16) B8 {
    u32x4v v;
};

__device__ __forceinline__ B8 ld16(const bf16 *p) { return B8{*reinterpret_cast<const u32x4v *>(p)}; }
__device__ __forceinline__ void st16(bf16 *p, B8 x) { *reinterpret_cast<u32x4v *>(p) = x.v; }
__device__ __forceinline__ B8 zero16() { return B8{u32x4v{0u, 0u, 0u, 0u}}; }
__device__ __forceinline__ bf16x8 as_bf8(B8 x) { return __builtin_bit_cast(bf16x8, x.v); }

__device__ __forceinline__ f32x4 mfma32(f32x4 acc, bf16x8 a, bf16x8 b)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// logistic function with the hardware reciprocal (about 1 ulp; the results are
// rounded to bf16): 1 + e^-z = inf gives 0, e^-z = 0 gives 1
__device__ __forceinline__ float sigmoidf_(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }


// ---------------------------------------------------------------------------
// Generic GEMM tile: C[m][n] = sum_k A[m][k] B[n][k] (bf16), block tile
// BM x 128 with BM = 32 MB, 4 waves as 2 x 2 of (16 MB) x 64, k step 64, K a
// multiple of 64.  MB = 4 is the 128 x 128 tile; MB = 8 (256 x 128, wave tiles
// of 128 x 64) reads half as many LDS bytes per multiply-add from the A side;
// MB = 2 (64 x 128) gives small products twice the workgroups.
// An operand is stored either k-contiguous (row m of A at A + m * lda,
// 128-byte rows per stage) or, with AT / BT, k-major (row k at A + k * lda,
// holding M contiguous elements: a token-major tensor read as its transpose),
// whose fragments come from the transposing LDS read.  Rows of A past M and
// rows of B past N read as zero, and so do rows k >= kvalid of a k-major
// operand.  The epilogue gets the wave's MB x 4 accumulator tiles: tile (i, q)
// holds C at rows mbase + 16 i + 4 g + (0..3), column nbase + 16 q + (lane & 15).
// ---------------------------------------------------------------------------
constexpr int GBK = 64;
constexpr int GPITCH = GBK + 8;  // LDS row pitch (bf16): 16-byte fragment reads hit distinct banks per 8 lanes
constexpr int GTPITCH = 128 + 16;  // k-major stage rows: transposing reads of 8 rows hit distinct banks
constexpr int GPD = 2;           // register stages in flight (even: LDS buffer = stage parity)

// Row of a k-major stage that holds k row k (see the fragment reads).
__device__ __forceinline__ int kperm(int k)
{
    const int r = k & 31;
    return (k & ~31) | ((r & 4) ? 16 : 0) | ((r >> 3) << 2) | (r & 3);
}

template <int BM> struct GemmLdsT {
    // at BM = 64 the k-major A stage (64 k rows of BM + 16) needs 72 rows
    static constexpr int AR = BM < 72 ? 72 : BM;
    bf16 a[2][AR][GPITCH];
    bf16 b[2][128][GPITCH];
};
using GemmLds = GemmLdsT<128>;
static_assert(sizeof(bf16[GBK][GTPITCH]) <= sizeof(bf16[128][GPITCH]), "k-major stage fits the buffer");
static_assert(sizeof(bf16[GBK][256 + 16]) <= sizeof(bf16[256][GPITCH]), "k-major stage fits the buffer");
static_assert(sizeof(bf16[GBK][64 + 16]) <= sizeof(bf16[GemmLdsT<64>::AR][GPITCH]), "k-major stage fits the buffer");

// K is cut into nseg segments of kseg (a multiple of 64); segment s reads A
// from As[s] and B from Bs[s] (same leading dimensions; As and Bs are arrays
// of pointers or anything indexable by the segment number).  This sums
// products of split operands (hi and lo bf16 parts) in one accumulation.
// Core of the tile: accumulates the k steps [st_lo, st_lo + nlive) of the
// product into acc, running nloop steps (a multiple of GPD; steps past nlive
// compute zeros) so that wave groups with different ranges meet the same
// barriers.  tid: the thread's index within its group of 256.
template <bool AT, bool BT, int MB, typename PA, typename PB>
__device__ __forceinline__ void gemm_tile_core(GemmLdsT<32 * MB> &L, const PA &As, long lda,
                                               const PB &Bs, long ldb, int M, int N, int kseg,
                                               int nseg, int m0, int n0, int kvalid, int st_lo, int nlive,
                                               int nloop, int tid, f32x4 (&acc)[MB][4])
{
    static_assert(MB == 2 || MB == 4 || MB == 8, "block rows 64, 128 or 256");
    constexpr int NP = MB > 4 ? MB : 4;  // pieces per thread and side, at most
    constexpr int BM = 32 * MB;
    constexpr int TPA = BM + 16;        // k-major A stage pitch
    constexpr int AKT = BM / 8;         // threads per k-major A row (8 elements each)
    const int K = kseg * nseg;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, mm = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;
    // Pieces of 16 bytes per thread: MB for A, 4 for B.  k-contiguous: rows
    // tid/8 + 32 i, 8 columns each.  k-major: k rows tid/(BM/8) + (2048/BM) i
    // of A (tid/16 + 16 i of B), 8 of the row's elements each.
    int lrow[NP], lcol, krow[4], kcol, akrow[MB], akcol;
#pragma unroll
    for (int i = 0; i < NP; ++i) lrow[i] = (tid >> 3) + 32 * i;
#pragma unroll
    for (int i = 0; i < MB; ++i) akrow[i] = tid / AKT + (256 / AKT) * i;
#pragma unroll
    for (int i = 0; i < 4; ++i) krow[i] = (tid >> 4) + 16 * i;
    lcol = (tid & 7) * 8;
    kcol = (tid & 15) * 8;
    akcol = (tid % AKT) * 8;
    bool aok[MB], bok[4];
#pragma unroll
    for (int i = 0; i < MB; ++i) aok[i] = m0 + lrow[i] < M;
#pragma unroll
    for (int i = 0; i < 4; ++i) bok[i] = n0 + lrow[i] < N;
    const int nst = K / GBK;
    const int ngroups = nloop / GPD;
    B8 ra[GPD][MB], rb[GPD][4];
    auto issue = [&](int s, int st) {
        const int kk = min(st_lo + st, nst - 1) * GBK;
        const int sg = kk / kseg, kin = kk - sg * kseg;
        const bf16 *A = As[sg], *B = Bs[sg];
        // A piece i, then B piece i (the order of the 128-row tile)
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            if (i < MB) {
                if constexpr (AT)
                    ra[s][i] = ld16(A + (long)min(kin + akrow[i], kvalid - 1) * lda + m0 + akcol);
                else
                    ra[s][i] = ld16(A + (long)min(m0 + lrow[i], M - 1) * lda + kin + lcol);
            }
            if (i < 4) {
                if constexpr (BT)
                    rb[s][i & 3] = ld16(B + (long)min(kin + krow[i & 3], kvalid - 1) * ldb + n0 + kcol);
                else
                    rb[s][i & 3] = ld16(B + (long)min(n0 + lrow[i], N - 1) * ldb + kin + lcol);
            }
        }
    };
    // Past the last k step the stage holds zeros, so every step computes (the
    // loads, LDS writes and MFMAs of a step stay in one basic block).
    auto commit = [&](int s, int buf, int st) {
        const bool live = st < nlive;
        const int kin = (min(st_lo + st, nst - 1) * GBK) % kseg;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            if (i < MB) {
                if constexpr (AT) {
                    bf16(*T)[TPA] = reinterpret_cast<bf16(*)[TPA]>(&L.a[buf][0][0]);
                    st16(&T[kperm(akrow[i])][akcol], (live && kin + akrow[i] < kvalid) ? ra[s][i] : zero16());
                } else {
                    st16(&L.a[buf][lrow[i]][lcol], (live && aok[i]) ? ra[s][i] : zero16());
                }
            }
            if (i < 4) {
                if constexpr (BT) {
                    bf16(*T)[GTPITCH] = reinterpret_cast<bf16(*)[GTPITCH]>(&L.b[buf][0][0]);
                    st16(&T[kperm(krow[i & 3])][kcol], (live && kin + krow[i & 3] < kvalid) ? rb[s][i & 3] : zero16());
                } else {
                    st16(&L.b[buf][lrow[i]][lcol], (live && bok[i & 3]) ? rb[s][i & 3] : zero16());
                }
            }
        }
    };
    // fragment of row r (m or n) for the 32-wide half kh, k = 8g + (0..7)
    // (tp: the k-major stage's row pitch).  A k-major stage stores k row
    // 8g + j of each 32-row block at row kperm: 4g + j for j < 4, 16 + 4g +
    // j - 4 otherwise, so the two transposing reads (rows 4g + j and 16 + 4g
    // + j) return the same natural k order as one 16-byte read of a
    // k-contiguous row.
    auto frag = [&](const bf16 (*X)[GPITCH], bool kmajor, int tp, int r, int kh) {
        if (!kmajor) return as_bf8(ld16(&X[r][32 * kh + 8 * g]));
        const bf16 *T = &X[0][0];
        const int rb0 = r - mm;  // first row of the 16-row block
        const bf16x4 x0 = lds_read_tr(T + (32 * kh + 4 * g + (mm >> 2)) * tp + rb0 + 4 * (mm & 3));
        const bf16x4 x1 = lds_read_tr(T + (32 * kh + 16 + 4 * g + (mm >> 2)) * tp + rb0 + 4 * (mm & 3));
        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = zero4();

    // per 32-wide half: MB x 4 MFMAs, MB + 4 loads (or LDS writes) between them
    constexpr int NMF = 4 * MB, NLD = MB + 4;
    constexpr int RDS = (AT ? 2 : 1) * MB + (BT ? 2 : 1) * 4;  // LDS reads per half
#pragma unroll
    for (int s = 0; s < GPD; ++s) {
        issue(s, s);
        __builtin_amdgcn_sched_barrier(0);
    }
    commit(0, 0, 0);
    lds_barrier();
    for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
        for (int j = 0; j < GPD; ++j) {
            const int st = gi * GPD + j;
            const int buf = j & 1;
            // per 32-wide half: its fragments, then its MFMAs with the next
            // steps' loads (first half) or LDS writes (second half) between them
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                bf16x8 af[MB], bfr[4];
#pragma unroll
                for (int i = 0; i < MB; ++i) af[i] = frag(L.a[buf], AT, TPA, wm * (16 * MB) + 16 * i + mm, kh);
#pragma unroll
                for (int i = 0; i < 4; ++i) bfr[i] = frag(L.b[buf], BT, GTPITCH, wn * 64 + 16 * i + mm, kh);
                if (kh == 0)
                    issue(j, st + GPD);
                else
                    commit((j + 1) % GPD, (j + 1) & 1, st + 1);
#pragma unroll
                for (int i = 0; i < MB; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) acc[i][q] = mfma32(acc[i][q], af[i], bfr[q]);
                __builtin_amdgcn_sched_group_barrier(0x100, RDS, 0);
#pragma unroll
                for (int x = 0; x < NLD; ++x) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    if (kh == 0)
                        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                    else
                        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                }
                if constexpr (NMF > 2 * NLD) __builtin_amdgcn_sched_group_barrier(0x008, NMF - 2 * NLD, 0);
            }
            lds_barrier();
        }
    }
}

template <bool AT = false, bool BT = false, int MB = 4, typename PA, typename PB, typename Epi>
__device__ __forceinline__ void gemm_nt_tile(GemmLdsT<32 * MB> &L, const PA &As, long lda,
                                             const PB &Bs, long ldb, int M, int N,
                                             int kseg, int nseg, int m0, int n0, int kvalid, Epi &&epi)
{
    const int nst = kseg * nseg / GBK;
    f32x4 acc[MB][4];
    gemm_tile_core<AT, BT, MB>(L, As, lda, Bs, ldb, M, N, kseg, nseg, m0, n0, kvalid, 0, nst,
                               (nst + GPD - 1) / GPD * GPD, threadIdx.x, acc);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    epi(acc, m0 + (wave >> 1) * (16 * MB), n0 + (wave & 1) * 64, lane >> 4, lane & 15);
}

// The same 128 x 128 tile with eight waves (512 threads): waves 4-7 take the
// second half of the k steps in their own LDS buffers, so each SIMD runs two
// waves of one tile and one hides the other's load and LDS latency (for
// launches with one workgroup per CU).  Their sums are handed to waves 0-3
// through LDS; waves 4-7 then leave the kernel, and waves 0-3 run the
// epilogue as in the four-wave tile.  The epilogue must therefore not use a
// workgroup barrier, and the call must end the kernel.
template <bool AT = false, bool BT = false, typename PA, typename PB, typename Epi>
__device__ __forceinline__ void gemm_nt_tile_kg2(GemmLds (&L)[2], const PA &As, long lda,
                                                 const PB &Bs, long ldb, int M, int N, int kseg,
                                                 int nseg, int m0, int n0, int kvalid, Epi &&epi)
{
    const int nst = kseg * nseg / GBK;
    const int half = (nst + 1) / 2;
    const int grp = threadIdx.x >> 8, tid = threadIdx.x & 255;
    f32x4 acc[4][4];
    gemm_tile_core<AT, BT, 4>(L[grp], As, lda, Bs, ldb, M, N, kseg, nseg, m0, n0, kvalid, grp ? half : 0,
                              grp ? nst - half : half, (half + GPD - 1) / GPD * GPD, tid, acc);
    // hand-off: lane-linear f32x4 slots in group 1's buffer (64 KB)
    f32x4 *x = reinterpret_cast<f32x4 *>(&L[1]) + (tid >> 6) * 16 * 64 + (tid & 63);
    static_assert(sizeof(f32x4) * 4 * 16 * 64 <= sizeof(GemmLds), "hand-off fits the buffer");
    if (grp) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) x[(4 * i + q) * 64] = acc[i][q];
    }
    lds_barrier();
    if (grp) return;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] += x[(4 * i + q) * 64];
    const int lane = tid & 63, wave = tid >> 6;
    epi(acc, m0 + (wave >> 1) * 64, n0 + (wave & 1) * 64, lane >> 4, lane & 15);
}

// ---------------------------------------------------------------------------
// parameters shared by the kernels
// ---------------------------------------------------------------------------
struct LactParams {
    const bf16 *q, *k, *v;
    const float *eta;
    const float *w1i, *w2i, *w3i;
    bf16 *out;
    float *w1, *w2, *w3;        // fp32 masters (the final-state buffers)
    int NH, Tq, Tkv, d, hid, chunk, nchunks, cpad, qpad, loss, order, rownorm, splitk;
    bf16 *dy;      // [NH][cpad][d]    dY token-major (MSE)
    bf16 *w13b;    // [nslots][NH][2 parts][2 hid][d]  W1/W3 rows interleaved by 16; part 0 =
                   //   bf16(W) (nearest), part 1 = bf16(W - part 0)
    bf16 *w2b;     // [nslots][NH][2 parts][d][hid]
    bf16 *gt;      // [NH][hid][cpad]  G^T of the current chunk
    bf16 *dh1t;    // [NH][hid][cpad]
    bf16 *dh3t;    // [NH][hid][cpad]
    bf16 *gq;      // [NH][2 parts][qpad][hid]  G of the queries (or of the keys, MSE), hi/lo
    float *part;   // [splitk][NH][3][hid * d] gradient partials; under Muon split 0 then
                   //   holds the momentum-step direction and the Newton-Schulz iterate (fp32)
    int nslots;
    int rule;      // 0 gradient descent, 1 momentum, 2 Muon
    float beta, lr;
    float *m1, *m2, *m3;   // momentum buffers (like w1, w2, w3), or null
    bf16 *nsb;     // [2][NH][3][hid * d] bf16 copies of the iterate (ping-pong)
    bf16 *gram;    // [NH][3][d][d] bf16 Gram matrix of the iterate
    float *diag;   // [NH][3][d] fp32 diagonal of the first Gram matrix
    // Backward's forward replay: when set, the update of chunk save_c also
    // writes the chunk-start weights and the step direction it subtracts,
    // [chunk][NH][3][hid * d] fp32 each (W1, W3 as [hid][d], W2 as [d][hid]).
    float *save_w = nullptr, *save_d = nullptr;
    int save_c = 0;
};

// Row of W1 (which = 0) or W3 (which = 1) hidden unit h inside the packed
// [2 hid][d] copy: blocks of 16 W1 rows and 16 W3 rows alternate, so one
// wave's 64-row tile of a product with the packed copy holds matching
// W1 and W3 rows.
__device__ __forceinline__ int packed_row(int h, int which) { return 32 * (h >> 4) + 16 * which + (h & 15); }

__device__ __forceinline__ long slot_off13(const LactParams &p, int slot, int h, int part = 0)
{
    return (((long)slot * p.NH + h) * 2 + part) * 2 * p.hid * p.d;
}
__device__ __forceinline__ long slot_off2(const LactParams &p, int slot, int h, int part = 0)
{
    return (((long)slot * p.NH + h) * 2 + part) * (long)p.d * p.hid;
}
// w = hi + lo: hi = bf16(w) (nearest), lo = bf16(w - hi) (w - hi is exact in fp32).
__device__ __forceinline__ void split1(float w, bf16 &hi, bf16 &lo)
{
    hi = (bf16)w;
    lo = (bf16)(w - (float)hi);
}

}  // namespace tttk
