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
// So the work runs in four launches: the state recursion and the G recursion
// with one workgroup per (head, 16 columns) and their operands staged in LDS
// a batch of chunks at a time, and between and after them two
// launches with one workgroup per (head, chunk) for everything else (the
// G-free terms and R_c first, then the terms that need G_{c+1}), exchanging
// per-chunk matrices through the workspace.  Everything is fp32 FMA in LDS.
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

// four consecutive floats of an LDS row (16-byte aligned)
__device__ __forceinline__ f32x4 lds4(const float *x) { return *reinterpret_cast<const f32x4 *>(x); }

// Serial passes: the operands of NB chunks at a time are loaded into registers
// while the previous NB chunks compute out of LDS, and written to LDS once per
// batch, so no chunk step waits for memory (a step only reads LDS and stores).
template <int D, int B> struct Batch {
    static constexpr int NB = (B <= 16 ? 8 : 4) * 64 / D;  // LDS: two batches of K and V / R_c
};

// Serial pass 1 (one workgroup per (head, 16 state columns); columns of the
// state never mix in the recursion W_{c+1} = W_c + K^T H (V - K W_c)):
// writes every chunk-start state.
template <int D, int B, typename E>
__global__ __launch_bounds__(256) void lbw_states(LinBwdParams p)
{
    constexpr int NB = Batch<D, B>::NB, NCB = D / CB, NK = B * D / 256, NV = B * CB / 256;
    // K rows padded to D + 4 floats; V and U stored transposed (token index
    // last), rows padded to B + 4: the dot products read four elements at a time
    constexpr int KP = D + 4, TP = B + 4, NE = D * CB / 256;
    __shared__ float W[D][CB + 1];
    __shared__ __align__(16) float Ks[2][NB][B][KP];
    __shared__ __align__(16) float Vt[2][NB][CB][TP];
    __shared__ __align__(16) float et[2][NB][B];
    __shared__ __align__(16) float Ut[CB][TP];
    const int h = blockIdx.x / NCB, j0 = (blockIdx.x % NCB) * CB, tid = threadIdx.x;
    const long tok0 = (long)h * p.T;
    const int nbat = (p.nchunks + NB - 1) / NB;
    float pk[NB][NK], pv[NB][NV], pe[NB];
    auto load = [&](int k) {
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const int c = k * NB + m;
            const int c0 = c * B, n = c < p.nchunks ? min(B, p.T - c0) : 0;
#pragma unroll
            for (int r = 0; r < NK; ++r) {
                const int e = tid + 256 * r, i = e / D, a = e % D;
                pk[m][r] = i < n ? ldf<E>(p.k, (tok0 + c0 + i) * D + a) : 0.f;
            }
#pragma unroll
            for (int r = 0; r < NV; ++r) {
                const int e = tid + 256 * r, i = e / CB, j = e % CB;
                pv[m][r] = i < n ? ldf<E>(p.v, (tok0 + c0 + i) * D + j0 + j) : 0.f;
            }
            pe[m] = (tid < n) ? p.eta[tok0 + c0 + tid] : 0.f;
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int m = 0; m < NB; ++m) {
#pragma unroll
            for (int r = 0; r < NK; ++r) Ks[buf][m][(tid + 256 * r) / D][(tid + 256 * r) % D] = pk[m][r];
#pragma unroll
            for (int r = 0; r < NV; ++r) Vt[buf][m][(tid + 256 * r) % CB][(tid + 256 * r) / CB] = pv[m][r];
            if (tid < B) et[buf][m][tid] = pe[m];
        }
    };
    for (int e = tid; e < D * CB; e += 256) W[e / CB][e % CB] = p.w0[(long)h * D * D + (e / CB) * D + j0 + e % CB];
    load(0);
    store(0);
    __syncthreads();
    for (int k = 0; k < nbat; ++k) {
        const int buf = k & 1;
        if (k + 1 < nbat) load(k + 1);
        for (int m = 0; m < NB; ++m) {
            const int c = k * NB + m;
            if (c >= p.nchunks) break;
            float *dst = p.states + ((long)h * p.nchunks + c) * D * D;
            for (int e = tid; e < D * CB; e += 256) dst[(e / CB) * D + j0 + e % CB] = W[e / CB][e % CB];
            const float(*Kc)[KP] = Ks[buf][m];
            const float(*Vc)[TP] = Vt[buf][m];
            const float(*Uc)[TP] = Vc;
            if (p.loss == 1) {  // U = V - K W
                for (int e = tid; e < B * CB; e += 256) {
                    const int i = e / CB, j = e % CB;
                    float sacc = 0.f;
#pragma unroll
                    for (int a = 0; a < D; a += 4) {
                        const f32x4 kv = lds4(&Kc[i][a]);
#pragma unroll
                        for (int x = 0; x < 4; ++x) sacc += kv[x] * W[a + x][j];
                    }
                    Ut[j][i] = Vc[j][i] - sacc;
                }
                lds_barrier();
                Uc = Ut;
            }
            {
                // thread elements (tid / CB + (256 / CB) r, tid % CB): one column j,
                // so each read of U^T and eta serves all of them
                const int j = tid % CB, ab = tid / CB;
                float sacc[NE];
#pragma unroll
                for (int r = 0; r < NE; ++r) sacc[r] = 0.f;
#pragma unroll
                for (int i = 0; i < B; i += 4) {
                    const f32x4 uv = lds4(&Uc[j][i]);
                    const f32x4 ev = lds4(&et[buf][m][i]);
#pragma unroll
                    for (int r = 0; r < NE; ++r)
#pragma unroll
                        for (int x = 0; x < 4; ++x) sacc[r] += Kc[i + x][ab + (256 / CB) * r] * ev[x] * uv[x];
                }
#pragma unroll
                for (int r = 0; r < NE; ++r) W[ab + (256 / CB) * r][j] += sacc[r];
            }
            lds_barrier();
        }
        if (k + 1 < nbat) {
            store(buf ^ 1);
            __syncthreads();
        }
    }
    if (p.order == 1)
        for (int e = tid; e < D * CB; e += 256) p.wfinal[(long)h * D * D + (e / CB) * D + j0 + e % CB] = W[e / CB][e % CB];
}

// Parallel pass 2, one workgroup per (head, chunk): every term that does not
// need G.  Writes dQ, d_eta's first part and the chunk's U, S~, dK part, R_c.
template <int D, int B, typename E>
// Three waves per SIMD (three workgroups per CU at d = 64, chunk 16; the LDS
// allows it): the register cap costs a few spilled values and still measured
// ~3.5% faster on the whole backward than two waves per SIMD.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 8))) void lbw_local(LinBwdParams p)
{
    __shared__ float Wc[D][D + 1];
    // token rows padded to D + 4 floats: 16-byte aligned, so the loops below read
    // four consecutive elements of a row (the same row for the whole wave) at once
    constexpr int P = D + 4;
    __shared__ __align__(16) float Qs[B][P], Ks[B][P], dOs[B][P], Us[B][P], Ss[B][P];
    __shared__ float As[B][B + 1], dAs[B][B + 1];
    __shared__ float et[B];
    constexpr int NBD = B * D / 256;
    constexpr int RS = 256 / D;  // row stride of one thread's outputs (rows i0 + RS r)
    const int h = blockIdx.x / p.nchunks, c = blockIdx.x % p.nchunks, tid = threadIdx.x;
    const long tok0 = (long)h * p.T;
    const int c0 = c * B, n = min(B, p.T - c0);
    const long cb = ((long)h * p.nchunks + c);
    const float *src = p.states + cb * D * D;
    for (int e = tid; e < D * D; e += 256) Wc[e / D][e % D] = src[e];
    for (int e = tid; e < B * D; e += 256) {
        const int i = e / D, j = e % D;
        const bool ok = i < n;
        const long g = (tok0 + c0 + i) * D + j;
        Qs[i][j] = ok ? ldf<E>(p.q, g) : 0.f;
        Ks[i][j] = ok ? ldf<E>(p.k, g) : 0.f;
        Us[i][j] = ok ? ldf<E>(p.v, g) : 0.f;
        dOs[i][j] = ok ? ldf<E>(p.dout, g) : 0.f;
    }
    if (tid < B) et[tid] = tid < n ? p.eta[tok0 + c0 + tid] : 0.f;
    __syncthreads();
    const long row0 = (long)h * p.nchunks * B + (long)c * B;  // this chunk's rows in the per-token buffers
    if (p.loss == 1) {
        float u[NBD];
        {
            const int i0 = tid / D, j = tid % D;  // outputs (i0 + RS r, j)
#pragma unroll
            for (int r = 0; r < NBD; ++r) u[r] = 0.f;
            #pragma unroll 2
            for (int a = 0; a < D; a += 4) {
                const float w0 = Wc[a][j], w1 = Wc[a + 1][j], w2 = Wc[a + 2][j], w3 = Wc[a + 3][j];
#pragma unroll
                for (int r = 0; r < NBD; ++r) {
                    const f32x4 kv = lds4(&Ks[i0 + RS * r][a]);
                    u[r] += kv[0] * w0;
                    u[r] += kv[1] * w1;
                    u[r] += kv[2] * w2;
                    u[r] += kv[3] * w3;
                }
            }
#pragma unroll
            for (int r = 0; r < NBD; ++r) u[r] = Us[i0 + RS * r][j] - u[r];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < NBD; ++r) {
            const int e = tid + 256 * r;
            Us[e / D][e % D] = u[r];
            p.ub[(row0 + e / D) * D + e % D] = u[r];
        }
    }
    for (int e = tid; e < B * B; e += 256) {
        const int t = e / B, i = e % B;
        float s = 0.f;
        if (i <= t)
            for (int a = 0; a < D; ++a) s += Qs[t][a] * Ks[i][a];
        As[t][i] = s;
    }
    __syncthreads();
    // S~ = S^T dO (S = A H);  dS = (dO U^T) * M
    {
        const int i0 = tid / D, j = tid % D;
        float sv[NBD];
#pragma unroll
        for (int r = 0; r < NBD; ++r) sv[r] = 0.f;
        for (int t = 0; t < B; ++t) {
            const float x = dOs[t][j];
#pragma unroll
            for (int r = 0; r < NBD; ++r) sv[r] += As[t][i0 + RS * r] * x;  // A is zero for t < i
        }
#pragma unroll
        for (int r = 0; r < NBD; ++r) {
            const int i = i0 + RS * r;
            Ss[i][j] = et[i] * sv[r];
            p.st[(row0 + i) * D + j] = et[i] * sv[r];
        }
    }
    for (int e = tid; e < B * B; e += 256) {
        const int t = e / B, i = e % B;
        float s = 0.f;
        if (i <= t)
            for (int a = 0; a < D; ++a) s += dOs[t][a] * Us[i][a];
        dAs[t][i] = s;
    }
    __syncthreads();
    if (tid < 64) {  // d_eta, the G-free part: sum_t dS[t][i] A[t][i]
        for (int i = 0; i < B; ++i) {
            float s = 0.f;
            for (int t = tid; t < B; t += 64) s += dAs[t][i] * As[t][i];
            for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
            if (tid == 0 && i < n) p.deta[tok0 + c0 + i] = s;
        }
    }
    __syncthreads();
    for (int e = tid; e < B * B; e += 256) dAs[e / B][e % B] *= et[e % B];
    __syncthreads();
    // dQ = dO Wc^T + dA K;  dK part = dA^T Q [- S~ Wc^T]
    {
        const int i0 = tid / D, a = tid % D;  // outputs (i0 + RS r, a)
        float sq[NBD], sk[NBD];
#pragma unroll
        for (int r = 0; r < NBD; ++r) sq[r] = sk[r] = 0.f;
        #pragma unroll 2
        for (int j = 0; j < D; j += 4) {
            const float w[4] = {Wc[a][j], Wc[a][j + 1], Wc[a][j + 2], Wc[a][j + 3]};
#pragma unroll
            for (int r = 0; r < NBD; ++r) {
                const f32x4 ov = lds4(&dOs[i0 + RS * r][j]);
#pragma unroll
                for (int x = 0; x < 4; ++x) sq[r] += ov[x] * w[x];
                if (p.loss == 1) {
                    const f32x4 sv4 = lds4(&Ss[i0 + RS * r][j]);
#pragma unroll
                    for (int x = 0; x < 4; ++x) sk[r] -= sv4[x] * w[x];
                }
            }
        }
        for (int t = 0; t < B; ++t) {
            const float kk = Ks[t][a], qq = Qs[t][a];
#pragma unroll
            for (int r = 0; r < NBD; ++r) {
                sq[r] += dAs[i0 + RS * r][t] * kk;
                sk[r] += dAs[t][i0 + RS * r] * qq;
            }
        }
#pragma unroll
        for (int r = 0; r < NBD; ++r) {
            const int i = i0 + RS * r;
            if (i < n) stf<E>(p.dq, (tok0 + c0 + i) * D + a, sq[r]);
            p.dkl[(row0 + i) * D + a] = sk[r];
        }
    }
    // R_c = Q^T dO [- K^T S~]
    float *R = p.rc + cb * D * D;
    {
        constexpr int NR = D * D / 256;
        const int a0 = (tid / D) * NR, j = tid % D;  // outputs (a0 + r, j)
        float sr[NR];
#pragma unroll
        for (int r = 0; r < NR; ++r) sr[r] = 0.f;
        #pragma unroll 2
        for (int i = 0; i < B; ++i) {
            const float x = dOs[i][j], y = Ss[i][j];
#pragma unroll
            for (int r = 0; r < NR; r += 4) {
                const f32x4 qv = lds4(&Qs[i][a0 + r]);
#pragma unroll
                for (int e = 0; e < 4; ++e) sr[r + e] += qv[e] * x;
                if (p.loss == 1) {
                    const f32x4 kv = lds4(&Ks[i][a0 + r]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) sr[r + e] -= kv[e] * y;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) R[(long)(a0 + r) * D + j] = sr[r];
    }
}

// Serial pass 3 (one workgroup per (head, 16 columns of G); G's columns never
// mix either): G_c = G_{c+1} + R_c [- K^T H K G_{c+1}], storing every G_{c+1};
// the last G is d_w_init.  Chunks run last to first, in batches as above.
template <int D, int B, typename E>
__global__ __launch_bounds__(256) void lbw_grad(LinBwdParams p)
{
    constexpr int NB = Batch<D, B>::NB, NCB = D / CB, NK = B * D / 256, NR = D * CB / 256;
    // K rows padded to D + 4 floats and (H K G) stored transposed, rows padded
    // to B + 4: both dot products read four consecutive elements at a time
    constexpr int KP = D + 4, TP = B + 4, NE = D * CB / 256;
    __shared__ float G[D][CB + 1];
    __shared__ __align__(16) float KGt[CB][TP];
    __shared__ float Rs[2][NB][D][CB + 1];
    __shared__ __align__(16) float Ks[2][NB][B][KP];
    __shared__ float et[2][NB][B];
    const int h = blockIdx.x / NCB, j0 = (blockIdx.x % NCB) * CB, tid = threadIdx.x;
    const long tok0 = (long)h * p.T;
    const int last = p.nchunks - 1;
    const int nbat = (p.nchunks + NB - 1) / NB;
    float pk[NB][NK], pr[NB][NR], pe[NB];
    auto load = [&](int k) {  // batch k = chunks last - k NB - m, m < NB
#pragma unroll
        for (int m = 0; m < NB; ++m) {
            const int c = last - (k * NB + m);
            const bool ok = c >= 0;
            const int c0 = c * B, n = ok ? min(B, p.T - c0) : 0;
            const float *R = p.rc + ((long)h * p.nchunks + (ok ? c : 0)) * D * D;
            const bool hasr = ok && p.order == 0;  // the update-then-apply order has no R_c
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int e = tid + 256 * r;
                pr[m][r] = hasr ? R[(long)(e / CB) * D + j0 + e % CB] : 0.f;
            }
            if (p.loss == 1) {
#pragma unroll
                for (int r = 0; r < NK; ++r) {
                    const int e = tid + 256 * r, i = e / D, a = e % D;
                    pk[m][r] = i < n ? ldf<E>(p.k, (tok0 + c0 + i) * D + a) : 0.f;
                }
                pe[m] = (tid < n) ? p.eta[tok0 + c0 + tid] : 0.f;
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int m = 0; m < NB; ++m) {
#pragma unroll
            for (int r = 0; r < NR; ++r) Rs[buf][m][(tid + 256 * r) / CB][(tid + 256 * r) % CB] = pr[m][r];
            if (p.loss == 1) {
#pragma unroll
                for (int r = 0; r < NK; ++r) Ks[buf][m][(tid + 256 * r) / D][(tid + 256 * r) % D] = pk[m][r];
                if (tid < B) et[buf][m][tid] = pe[m];
            }
        }
    };
    const float *g0 = p.order == 1 ? p.ginit : p.dwf;
    for (int e = tid; e < D * CB; e += 256)
        G[e / CB][e % CB] = g0 ? g0[(long)h * D * D + (e / CB) * D + j0 + e % CB] : 0.f;
    load(0);
    store(0);
    __syncthreads();
    for (int k = 0; k < nbat; ++k) {
        const int buf = k & 1;
        if (k + 1 < nbat) load(k + 1);
        for (int m = 0; m < NB; ++m) {
            const int c = last - (k * NB + m);
            if (c < 0) break;
            float *gdst = p.gnext + ((long)h * p.nchunks + c) * D * D;
            for (int e = tid; e < D * CB; e += 256) gdst[(e / CB) * D + j0 + e % CB] = G[e / CB][e % CB];
            const float(*Kc)[KP] = Ks[buf][m];
            if (p.loss == 1) {
                for (int e = tid; e < B * CB; e += 256) {
                    const int i = e / CB, j = e % CB;
                    float sacc = 0.f;
#pragma unroll
                    for (int a = 0; a < D; a += 4) {
                        const f32x4 kv = lds4(&Kc[i][a]);
#pragma unroll
                        for (int x = 0; x < 4; ++x) sacc += kv[x] * G[a + x][j];
                    }
                    KGt[j][i] = et[buf][m][i] * sacc;
                }
                lds_barrier();
            }
            {
                // thread elements (tid / CB + (256 / CB) r, tid % CB): one column j,
                // so each read of (H K G)^T serves all of them
                const int j = tid % CB, ab = tid / CB;
                float sacc[NE];
#pragma unroll
                for (int r = 0; r < NE; ++r) sacc[r] = Rs[buf][m][ab + (256 / CB) * r][j];
                if (p.loss == 1) {
#pragma unroll
                    for (int i = 0; i < B; i += 4) {
                        const f32x4 kg = lds4(&KGt[j][i]);
#pragma unroll
                        for (int r = 0; r < NE; ++r)
#pragma unroll
                            for (int x = 0; x < 4; ++x) sacc[r] -= Kc[i + x][ab + (256 / CB) * r] * kg[x];
                    }
                }
#pragma unroll
                for (int r = 0; r < NE; ++r) G[ab + (256 / CB) * r][j] += sacc[r];
            }
            lds_barrier();
        }
        if (k + 1 < nbat) {
            store(buf ^ 1);
            __syncthreads();
        }
    }
    __syncthreads();
    for (int e = tid; e < D * CB; e += 256) p.dw0[(long)h * D * D + (e / CB) * D + j0 + e % CB] = G[e / CB][e % CB];
}

// Parallel pass 4, one workgroup per (head, chunk): the terms that need
// G = G_{c+1}:  KG = K G,  dV = dU = S~ + H KG,
// dK = part + H (U G^T [- KG Wc^T]),  d_eta += rowsum(KG * U).
template <int D, int B, typename E>
__global__ __launch_bounds__(256) void lbw_dep(LinBwdParams p)
{
    __shared__ float Gn[D][D + 1], Wc[D][D + 1];
    // token rows padded to D + 4 floats (16-byte aligned: four elements per read)
    constexpr int P = D + 4;
    __shared__ __align__(16) float Ks[B][P], Us[B][P], KGs[B][P];
    __shared__ float et[B];
    constexpr int NBD = B * D / 256;
    const int h = blockIdx.x / p.nchunks, c = blockIdx.x % p.nchunks, tid = threadIdx.x;
    const long tok0 = (long)h * p.T;
    const int c0 = c * B, n = min(B, p.T - c0);
    const long cb = ((long)h * p.nchunks + c);
    const long row0 = (long)h * p.nchunks * B + (long)c * B;
    for (int e = tid; e < D * D; e += 256) {
        Gn[e / D][e % D] = p.gnext[cb * D * D + e];
        if (p.loss == 1) Wc[e / D][e % D] = p.states[cb * D * D + e];
    }
    const bool nc = p.order == 1;  // no outputs per chunk: U from here, no G-free parts
    for (int e = tid; e < B * D; e += 256) {
        const int i = e / D, j = e % D;
        const bool ok = i < n;
        Ks[i][j] = ok ? ldf<E>(p.k, (tok0 + c0 + i) * D + j) : 0.f;
        Us[i][j] = (p.loss == 1 && !nc) ? p.ub[(row0 + i) * D + j]
                                        : (ok ? ldf<E>(p.v, (tok0 + c0 + i) * D + j) : 0.f);
    }
    if (tid < B) et[tid] = tid < n ? p.eta[tok0 + c0 + tid] : 0.f;
    __syncthreads();
    if (nc && p.loss == 1) {  // U = V - K W_c
        float u[NBD];
#pragma unroll
        for (int r = 0; r < NBD; ++r) {
            const int e = tid + 256 * r, i = e / D, j = e % D;
            float sacc = 0.f;
            for (int a = 0; a < D; ++a) sacc += Ks[i][a] * Wc[a][j];
            u[r] = Us[i][j] - sacc;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < NBD; ++r) Us[(tid + 256 * r) / D][(tid + 256 * r) % D] = u[r];
        __syncthreads();
    }
    // thread outputs (i0 + RS r, j): the wave shares its rows, so row reads are
    // broadcasts and each column element of G is read once for all rows
    constexpr int RS = 256 / D;
    const int i0 = tid / D, jl = tid % D;
    {
        float sg[NBD];
#pragma unroll
        for (int r = 0; r < NBD; ++r) sg[r] = 0.f;
#pragma unroll 2
        for (int a = 0; a < D; a += 4) {
            const float g0 = Gn[a][jl], g1 = Gn[a + 1][jl], g2 = Gn[a + 2][jl], g3 = Gn[a + 3][jl];
#pragma unroll
            for (int r = 0; r < NBD; ++r) {
                const f32x4 kv = lds4(&Ks[i0 + RS * r][a]);
                sg[r] += kv[0] * g0;
                sg[r] += kv[1] * g1;
                sg[r] += kv[2] * g2;
                sg[r] += kv[3] * g3;
            }
        }
#pragma unroll
        for (int r = 0; r < NBD; ++r) {
            const int i = i0 + RS * r;
            KGs[i][jl] = sg[r];
            if (i < n) stf<E>(p.dv, (tok0 + c0 + i) * D + jl, (nc ? 0.f : p.st[(row0 + i) * D + jl]) + et[i] * sg[r]);
        }
    }
    __syncthreads();
    if (tid < 64) {
        for (int i = 0; i < n; ++i) {
            float s = 0.f;
            for (int a = tid; a < D; a += 64) s += KGs[i][a] * Us[i][a];
            for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
            if (tid == 0) p.deta[tok0 + c0 + i] = (nc ? 0.f : p.deta[tok0 + c0 + i]) + s;
        }
    }
    {
        const int a = jl;  // outputs (i0 + RS r, a)
        float sk[NBD];
#pragma unroll
        for (int r = 0; r < NBD; ++r) sk[r] = 0.f;
#pragma unroll 2
        for (int j = 0; j < D; j += 4) {
            const float g[4] = {Gn[a][j], Gn[a][j + 1], Gn[a][j + 2], Gn[a][j + 3]};
            float w[4] = {0.f, 0.f, 0.f, 0.f};
            if (p.loss == 1) {
#pragma unroll
                for (int x = 0; x < 4; ++x) w[x] = Wc[a][j + x];
            }
#pragma unroll
            for (int r = 0; r < NBD; ++r) {
                const f32x4 uv = lds4(&Us[i0 + RS * r][j]);
                if (p.loss == 1) {
                    const f32x4 kg = lds4(&KGs[i0 + RS * r][j]);
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        sk[r] += uv[x] * g[x];
                        sk[r] -= kg[x] * w[x];
                    }
                } else {
#pragma unroll
                    for (int x = 0; x < 4; ++x) sk[r] += uv[x] * g[x];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < NBD; ++r) {
            const int i = i0 + RS * r;
            if (i < n) stf<E>(p.dk, (tok0 + c0 + i) * D + a, (nc ? 0.f : p.dkl[(row0 + i) * D + a]) + et[i] * sk[r]);
        }
    }
}

// Update-then-apply order, the apply's adjoint: G_final = dW_final + Q^T dO
// (one workgroup per (head, 16 columns), queries in tiles of 64) ...
template <int D, typename E>
__global__ __launch_bounds__(256) void lbw_nc_g(LinBwdParams p)
{
    __shared__ float Qs[64][D + 1], dOs[64][CB + 1];
    constexpr int NCB = D / CB;
    const int h = blockIdx.x / NCB, j0 = (blockIdx.x % NCB) * CB, tid = threadIdx.x;
    const long q0 = (long)h * p.Tq;
    float acc[D * CB / 256];
#pragma unroll
    for (int r = 0; r < D * CB / 256; ++r) {
        const int e = tid + 256 * r;
        acc[r] = p.dwf ? p.dwf[(long)h * D * D + (e / CB) * D + j0 + e % CB] : 0.f;
    }
    for (int t0 = 0; t0 < p.Tq; t0 += 64) {
        const int n = min(64, p.Tq - t0);
        for (int e = tid; e < 64 * D; e += 256) {
            const int t = e / D, a = e % D;
            Qs[t][a] = t < n ? ldf<E>(p.q, (q0 + t0 + t) * D + a) : 0.f;
        }
        for (int e = tid; e < 64 * CB; e += 256) {
            const int t = e / CB, j = e % CB;
            dOs[t][j] = t < n ? ldf<E>(p.dout, (q0 + t0 + t) * D + j0 + j) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < D * CB / 256; ++r) {
            const int e = tid + 256 * r, a = e / CB, j = e % CB;
            float sacc = 0.f;
            for (int t = 0; t < 64; ++t) sacc += Qs[t][a] * dOs[t][j];
            acc[r] += sacc;
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < D * CB / 256; ++r) {
        const int e = tid + 256 * r;
        p.ginit[(long)h * D * D + (e / CB) * D + j0 + e % CB] = acc[r];
    }
}

// ... and dQ = dO W_final^T (one workgroup per (head, 64 queries)).
template <int D, typename E>
__global__ __launch_bounds__(256) void lbw_nc_dq(LinBwdParams p)
{
    __shared__ float Wf[D][D + 1], dOs[64][D + 1];
    const int nqt = (p.Tq + 63) / 64;
    const int h = blockIdx.x / nqt, t0 = (blockIdx.x % nqt) * 64, tid = threadIdx.x;
    const long q0 = (long)h * p.Tq;
    const int n = min(64, p.Tq - t0);
    for (int e = tid; e < D * D; e += 256) Wf[e / D][e % D] = p.wfinal[(long)h * D * D + e];
    for (int e = tid; e < 64 * D; e += 256) {
        const int t = e / D, j = e % D;
        dOs[t][j] = t < n ? ldf<E>(p.dout, (q0 + t0 + t) * D + j) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < 64 * D; e += 256) {
        const int t = e / D, a = e % D;
        float sacc = 0.f;
        for (int j = 0; j < D; ++j) sacc += dOs[t][j] * Wf[a][j];
        if (t < n) stf<E>(p.dq, (q0 + t0 + t) * D + a, sacc);
    }
}

}  // namespace

size_t linear_bwd_workspace(int NH, int Tkv, int d, int chunk)
{
    const size_t nch = (Tkv + chunk - 1) / chunk;
    // states, G_{c+1}, R_c (d x d per chunk) and U, S~, dK part (chunk x d per chunk), plus
    // the final state and dL/dW_final (update-then-apply order), fp32
    return (size_t)NH * (nch * (3 * (size_t)d * d + 3 * (size_t)chunk * d) + 2 * (size_t)d * d) *
           sizeof(float);
}

template <int D, int B, typename E>
static void lbw_run(const LinBwdParams &p, int NH, hipStream_t st)
{
    const dim3 b(256);
    lbw_states<D, B, E><<<dim3(NH * (D / CB)), b, 0, st>>>(p);
    if (p.order == 0) {
        lbw_local<D, B, E><<<dim3(NH * p.nchunks), b, 0, st>>>(p);
    } else {
        lbw_nc_g<D, E><<<dim3(NH * (D / CB)), b, 0, st>>>(p);
        if (p.Tq > 0) lbw_nc_dq<D, E><<<dim3(NH * ((p.Tq + 63) / 64)), b, 0, st>>>(p);
    }
    lbw_grad<D, B, E><<<dim3(NH * (D / CB)), b, 0, st>>>(p);
    lbw_dep<D, B, E><<<dim3(NH * p.nchunks), b, 0, st>>>(p);
}

hipError_t linear_bwd_launch(int NH, int Tq, int Tkv, int d, int chunk, int loss, int order,
                             int bf16, const void *q, const void *k, const void *v,
                             const float *eta, const float *w0, const void *dout, const float *dwf,
                             void *dq, void *dk, void *dv, float *deta, float *dw0, void *ws,
                             hipStream_t st)
{
    const int nch = (Tkv + chunk - 1) / chunk;
    float *base = static_cast<float *>(ws);
    const size_t dd = (size_t)NH * nch * d * d, bd = (size_t)NH * nch * chunk * d;
    float *tail = base + 3 * dd + 3 * bd;
    LinBwdParams p{q, k, v, dout, eta, w0, dwf, dq, dk, dv, deta, dw0, base, base + dd,
                   base + 2 * dd, base + 3 * dd, base + 3 * dd + bd, base + 3 * dd + 2 * bd, Tkv,
                   nch, loss, order, Tq, tail, tail + (size_t)NH * d * d};
    if (d == 128) {  // chunk 16 only (LDS of the dependent pass)
        if (bf16) lbw_run<128, 16, __bf16>(p, NH, st);
        else lbw_run<128, 16, float>(p, NH, st);
    } else if (chunk == 16) {
        if (bf16) lbw_run<64, 16, __bf16>(p, NH, st);
        else lbw_run<64, 16, float>(p, NH, st);
    } else {
        if (bf16) lbw_run<64, 32, __bf16>(p, NH, st);
        else lbw_run<64, 32, float>(p, NH, st);
    }
    return hipGetLastError();
}

}  // namespace tttk
