// Causal sliding-window softmax attention on gfx950 (bf16 MFMA, fp32 softmax).
//
// What is computed ("LaCT: Test-Time Training Done Right", sections 3.1 and
// 4: a window attention over nearby tokens sits beside the large-chunk fast
// weight, on the same Q, K, V, and the outputs are combined): for every
// (batch, head) and query t,
//     o_t = sum_{t - W < s <= t} softmax_s(scale * q_t . k_s) v_s
// optionally added to what `out` already holds.
//
// One workgroup = 128 queries of one head, eight waves of 16 (at head dim 256
// a wave then needs about 200 registers, so two waves share each SIMD and one
// wave's softmax and barrier latency hides behind the other's matrix work;
// four waves of 32 need nearly 500 and run one per SIMD).  Key/value blocks
// of 64 tokens are staged in LDS (double-buffered, the next block's global
// loads in flight during the current block's math).  Each wave computes the
// transposed scores S^T = K Q^T (rows = keys, columns = its queries), so the
// score accumulators, rounded to bf16, are directly the B operand of
// O^T += V^T P^T; V^T fragments come from LDS with transposing reads.  The
// softmax is the streaming one (running max and sum per query, the output
// rescaled when the max grows), in base 2 with the scale folded in.  Blocks
// entirely outside a wave's window are skipped by that wave; masks are
// applied only on blocks that straddle a window edge or the sequence end.
#include "ttt_device.h"
#include "ttt_internal.h"

#include <hip/hip_runtime.h>

namespace tttk {
namespace {

typedef __bf16 bf16;
typedef uint32_t u32x4w __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4w ldg16(const bf16 *p) { return *reinterpret_cast<const u32x4w *>(p); }
__device__ __forceinline__ void sts16(bf16 *p, u32x4w x) { *reinterpret_cast<u32x4w *>(p) = x; }

__device__ __forceinline__ f32x4 mfma32b(f32x4 acc, bf16x8 a, bf16x8 b)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

struct WinParams {
    const bf16 *q, *k, *v;
    bf16 *out;
    int NH, T, window, accumulate;
    float scale_log2;  // scale * log2(e)
};

constexpr int QB = 128;       // queries per workgroup
constexpr int KB = 64;        // keys per block

template <int D> struct WinLds {
    static constexpr int KP = D + 8;    // K rows: 16-byte fragment reads hit distinct banks
    static constexpr int VP = D + 16;   // V rows: transposing reads of 8 rows hit distinct banks
    bf16 k[2][KB][KP];
    bf16 v[2][KB][VP];
};

// NW waves per workgroup, each owning QB / NW queries (NU query tiles of 16).
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void window_attn_fwd(WinParams p)
{
    constexpr int NT = 64 * NW;
    constexpr int WQ = QB / NW;   // queries per wave
    constexpr int NU = WQ / 16;   // 16-query tiles per wave
    constexpr int NKS = D / 32;   // 32-deep k steps over the head dim
    constexpr int NDT = D / 16;   // 16-row output tiles over the head dim
    constexpr int LPT = KB * D / 8 / NT;  // 16-byte pieces per thread per operand and block
    __shared__ WinLds<D> L;
    const int nqb = (p.T + QB - 1) / QB;
    const int bid = xcd_block(blockIdx.x, gridDim.x);
    const int h = bid / nqb, qb = bid % nqb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, mm = lane & 15;
    const int q0 = qb * QB;
    const int qw0 = q0 + wave * WQ;                    // this wave's first query
    const long hoff = (long)h * p.T * D;
    const bf16 *K = p.k + hoff, *V = p.v + hoff;

    // key blocks covering [q0 - W + 1, min(q0 + QB, T))
    const int klo = max(0, q0 - p.window + 1);
    const int kb0 = klo / KB * KB;
    const int khi = min(q0 + QB, p.T);
    const int nblk = (khi - kb0 + KB - 1) / KB;

    // Q^T fragments (B operand, column = query): 8 consecutive head-dim elements
    bf16x8 qf[NU][NKS];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int t = min(qw0 + 16 * u + mm, p.T - 1);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            qf[u][ks] = __builtin_bit_cast(bf16x8, ldg16(p.q + hoff + (long)t * D + 32 * ks + 8 * g));
    }

    // block loader: piece i * NT + tid covers row piece / (D / 8), 8 columns, so
    // each load instruction of the workgroup reads NT x 16 bytes of consecutive rows
    u32x4w rk[LPT], rv[LPT];
    auto issue = [&](int kb) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int piece = i * NT + tid;
            const int r = piece / (D / 8), c = (piece % (D / 8)) * 8;
            const long row = min(kb + r, p.T - 1);
            rk[i] = ldg16(K + row * D + c);
            rv[i] = ldg16(V + row * D + c);
        }
    };
    auto commit = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int piece = i * NT + tid;
            const int r = piece / (D / 8), c = (piece % (D / 8)) * 8;
            sts16(&L.k[buf][r][c], rk[i]);
            sts16(&L.v[buf][r][c], rv[i]);
        }
    };

    f32x4 o[NDT][NU];
    float mrun[NU], lrun[NU];   // running max (base-2 scaled scores) and this lane's share of the sum
#pragma unroll
    for (int u = 0; u < NU; ++u) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt][u] = zero4();
        mrun[u] = -1e30f;
        lrun[u] = 0.f;
    }

    issue(kb0);
    commit(0);
    __syncthreads();
    for (int n = 0; n < nblk; ++n) {
        const int kb = kb0 + n * KB;
        if (n + 1 < nblk) issue(kb + KB);
        const int buf = n & 1;
        // does this block meet the wave's windows at all, and does it need a mask?
        const int qlast = min(qw0 + WQ - 1, p.T - 1);
        const bool live = qw0 < p.T && kb <= qlast && kb + KB - 1 > qw0 - p.window;
        const bool full = kb + KB - 1 <= qw0 && kb > qlast - p.window && kb + KB <= p.T;
        if (live) {
            f32x4 s[4][NU];
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int u = 0; u < NU; ++u) s[kt][u] = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4w *>(
                                                                    &L.k[buf][16 * kt + mm][32 * ks + 8 * g]));
#pragma unroll
                    for (int u = 0; u < NU; ++u) s[kt][u] = mfma32b(s[kt][u], a, qf[u][ks]);
                }
            }
            // s[kt][u][j] = score of key kb + 16 kt + 4 g + j for query qw0 + 16 u + mm
            bf16x8 pf[2][NU];
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int qi = qw0 + 16 * u + mm;
                float mx = -1e30f;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float x = s[kt][u][j] * p.scale_log2;
                        if (!full) {
                            const int ki = kb + 16 * kt + 4 * g + j;
                            if (ki > qi || ki <= qi - p.window || ki >= p.T) x = -INFINITY;
                        }
                        s[kt][u][j] = x;
                        mx = fmaxf(mx, x);
                    }
                mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
                // The running max moves only when a score exceeds it by more
                // than 2^8 (base 2): numerator and denominator share the stale
                // max, so the result is unchanged, the probabilities stay below
                // 256, and most blocks skip rescaling the output accumulators.
                const bool grow = mx > mrun[u] + 8.f;
                const float mnew = grow ? mx : mrun[u];
                const float alpha = __builtin_amdgcn_exp2f(mrun[u] - mnew);
                mrun[u] = mnew;
                float ls = 0.f;
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float e = __builtin_amdgcn_exp2f(s[kt][u][j] - mnew);
                        s[kt][u][j] = e;
                        ls += e;
                    }
                lrun[u] = lrun[u] * alpha + ls;
                if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) o[dt][u] *= alpha;
                }
#pragma unroll
                for (int pp = 0; pp < 2; ++pp)
                    pf[pp][u] = __builtin_shufflevector(to_bf16x4(s[2 * pp][u]), to_bf16x4(s[2 * pp + 1][u]),
                                                        0, 1, 2, 3, 4, 5, 6, 7);
            }
            // O^T += V^T P^T; V^T fragments by transposing reads (k = 4g + j, 16 + 4g + j)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
                for (int pp = 0; pp < 2; ++pp) {
                    const bf16x4 x0 = lds_read_tr(&L.v[buf][32 * pp + 4 * g + (mm >> 2)][16 * dt + 4 * (mm & 3)]);
                    const bf16x4 x1 = lds_read_tr(&L.v[buf][32 * pp + 16 + 4 * g + (mm >> 2)][16 * dt + 4 * (mm & 3)]);
                    const bf16x8 a = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int u = 0; u < NU; ++u) o[dt][u] = mfma32b(o[dt][u], a, pf[pp][u]);
                }
            }
        }
        if (n + 1 < nblk) commit(buf ^ 1);
        __syncthreads();
    }

    // finish: divide by the row sums (the four g lanes of a column hold shares)
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        float l = lrun[u];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const int qi = qw0 + 16 * u + mm;
        if (qi >= p.T) continue;
        const float inv = 1.f / l;
        bf16 *orow = p.out + hoff + (long)qi * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            f32x4 y = o[dt][u] * inv;
            bf16 *dst = orow + 16 * dt + 4 * g;
            if (p.accumulate) y += to_f32x4(load4<bf16>(dst));
            store4<bf16>(dst, to_bf16x4(y));
        }
    }
}

}  // namespace

#ifndef WIN_NW
#define WIN_NW 8  // waves per workgroup: 8 waves of 16 queries (two waves per SIMD)
#endif

hipError_t window_attn_launch(int NH, int T, int d, int window, float scale, int accumulate,
                              const void *q, const void *k, const void *v, void *out,
                              hipStream_t st)
{
    WinParams p{static_cast<const bf16 *>(q), static_cast<const bf16 *>(k),
                static_cast<const bf16 *>(v), static_cast<bf16 *>(out), NH, T, window, accumulate,
                scale * 1.4426950408889634f};
    const dim3 grid(NH * ((T + QB - 1) / QB));
    switch (d) {
    case 64: window_attn_fwd<64, WIN_NW><<<grid, dim3(64 * WIN_NW), 0, st>>>(p); break;
    case 128: window_attn_fwd<128, WIN_NW><<<grid, dim3(64 * WIN_NW), 0, st>>>(p); break;
    default: window_attn_fwd<256, WIN_NW><<<grid, dim3(64 * WIN_NW), 0, st>>>(p); break;
    }
    return hipGetLastError();
}

}  // namespace tttk
