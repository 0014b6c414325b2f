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
// and the sweep runs over the chunks in reverse, one workgroup per (batch,
// head), with the chunk-start states written by a forward pass of the same
// recursion.  Everything is fp32 FMA in LDS: the chain over chunks is serial
// per head, so this version parallelises over heads only.
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
    float *states;  // [NH][nchunks][D][D]
    int T, nchunks, loss;
};

template <typename E> __device__ __forceinline__ float ldf(const void *p, long i)
{
    return (float)static_cast<const E *>(p)[i];
}
template <typename E> __device__ __forceinline__ void stf(void *p, long i, float x)
{
    static_cast<E *>(p)[i] = (E)x;
}

// forward recursion over the chunks, writing each chunk-start state
template <int D, int B, typename E>
__global__ __launch_bounds__(256) void lin_bwd_states(LinBwdParams p)
{
    __shared__ float W[D][D + 1];
    __shared__ float Ks[B][D + 1], Us[B][D + 1];
    __shared__ float et[B];
    const int h = blockIdx.x, tid = threadIdx.x;
    const long tok0 = (long)h * p.T;
    for (int e = tid; e < D * D; e += 256) W[e / D][e % D] = p.w0[(long)h * D * D + e];
    __syncthreads();
    for (int c = 0; c < p.nchunks; ++c) {
        const int c0 = c * B, n = min(B, p.T - c0);
        float *dst = p.states + ((long)h * p.nchunks + c) * D * D;
        for (int e = tid; e < D * D; e += 256) dst[e] = W[e / D][e % D];
        for (int e = tid; e < B * D; e += 256) {
            const int i = e / D, j = e % D;
            Ks[i][j] = i < n ? ldf<E>(p.k, (tok0 + c0 + i) * D + j) : 0.f;
            Us[i][j] = i < n ? ldf<E>(p.v, (tok0 + c0 + i) * D + j) : 0.f;
        }
        if (tid < B) et[tid] = tid < n ? p.eta[tok0 + c0 + tid] : 0.f;
        __syncthreads();
        if (p.loss == 1) {
            float u[(B * D + 255) / 256];
#pragma unroll
            for (int r = 0; r < (B * D + 255) / 256; ++r) {
                const int e = tid + 256 * r;
                u[r] = 0.f;
                if (e < B * D) {
                    const int i = e / D, j = e % D;
                    float s = 0.f;
                    for (int a = 0; a < D; ++a) s += Ks[i][a] * W[a][j];
                    u[r] = Us[i][j] - s;
                }
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < (B * D + 255) / 256; ++r) {
                const int e = tid + 256 * r;
                if (e < B * D) Us[e / D][e % D] = u[r];
            }
            __syncthreads();
        }
        for (int e = tid; e < D * D; e += 256) {
            const int a = e / D, j = e % D;
            float s = 0.f;
            for (int i = 0; i < B; ++i) s += Ks[i][a] * et[i] * Us[i][j];
            W[a][j] += s;
        }
        __syncthreads();
    }
}

template <int D, int B, typename E>
__global__ __launch_bounds__(256) void lin_bwd_sweep(LinBwdParams p)
{
    __shared__ float Wc[D][D + 1], G[D][D + 1];
    __shared__ float Qs[B][D + 1], Ks[B][D + 1], dOs[B][D + 1], Us[B][D + 1], dUs[B][D + 1],
        KGs[B][D + 1];
    __shared__ float As[B][B + 1], dAs[B][B + 1];
    __shared__ float et[B];
    constexpr int NBD = (B * D + 255) / 256;
    const int h = blockIdx.x, tid = threadIdx.x;
    const long tok0 = (long)h * p.T;
    for (int e = tid; e < D * D; e += 256)
        G[e / D][e % D] = p.dwf ? p.dwf[(long)h * D * D + e] : 0.f;
    for (int c = p.nchunks - 1; c >= 0; --c) {
        const int c0 = c * B, n = min(B, p.T - c0);
        const float *src = p.states + ((long)h * p.nchunks + c) * D * D;
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
        // U (MSE), K G, A
        float u[NBD], kg[NBD];
#pragma unroll
        for (int r = 0; r < NBD; ++r) {
            const int e = tid + 256 * r;
            u[r] = kg[r] = 0.f;
            if (e < B * D) {
                const int i = e / D, j = e % D;
                float s = 0.f, t = 0.f;
                for (int a = 0; a < D; ++a) {
                    s += Ks[i][a] * Wc[a][j];
                    t += Ks[i][a] * G[a][j];
                }
                u[r] = Us[i][j] - s;
                kg[r] = t;
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
#pragma unroll
        for (int r = 0; r < NBD; ++r) {
            const int e = tid + 256 * r;
            if (e < B * D) {
                if (p.loss == 1) Us[e / D][e % D] = u[r];
                KGs[e / D][e % D] = kg[r];
            }
        }
        __syncthreads();
        // dU = S^T dO + H (K G);  dS = (dO U^T) * M,  dA = dS H
#pragma unroll
        for (int r = 0; r < NBD; ++r) {
            const int e = tid + 256 * r;
            if (e < B * D) {
                const int i = e / D, j = e % D;
                float s = 0.f;
                for (int t = i; t < B; ++t) s += As[t][i] * dOs[t][j];
                dUs[i][j] = et[i] * (s + KGs[i][j]);
            }
        }
        for (int e = tid; e < B * B; e += 256) {
            const int t = e / B, i = e % B;
            float s = 0.f;
            if (i <= t)
                for (int a = 0; a < D; ++a) s += dOs[t][a] * Us[i][a];
            dAs[t][i] = s;  // dS for now
        }
        __syncthreads();
        // deta (one wave): sum_t dS[t][i] A[t][i] + (K G)_i . U_i
        if (tid < 64) {
            for (int i = 0; i < B; ++i) {
                float s = 0.f;
                for (int t = tid; t < B; t += 64) s += dAs[t][i] * As[t][i];
                for (int a = tid; a < D; a += 64) s += KGs[i][a] * Us[i][a];
                for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
                if (tid == 0 && i < n) p.deta[tok0 + c0 + i] = s;
            }
        }
        __syncthreads();
        for (int e = tid; e < B * B; e += 256) dAs[e / B][e % B] *= et[e % B];
        __syncthreads();
        // dQ = dO Wc^T + dA K;  dK = dA^T Q + H U G^T - dU Wc^T (MSE);  dV = dU
#pragma unroll
        for (int r = 0; r < NBD; ++r) {
            const int e = tid + 256 * r;
            if (e < B * D) {
                const int i = e / D, a = e % D;
                float sq = 0.f, sk = 0.f, ug = 0.f;
                for (int j = 0; j < D; ++j) {
                    sq += dOs[i][j] * Wc[a][j];
                    ug += Us[i][j] * G[a][j];
                    if (p.loss == 1) sk -= dUs[i][j] * Wc[a][j];
                }
                for (int t = 0; t < B; ++t) {
                    sq += dAs[i][t] * Ks[t][a];
                    sk += dAs[t][i] * Qs[t][a];
                }
                sk += et[i] * ug;
                if (i < n) {
                    const long g = (tok0 + c0 + i) * D + a;
                    stf<E>(p.dq, g, sq);
                    stf<E>(p.dk, g, sk);
                    stf<E>(p.dv, g, dUs[i][a]);
                }
            }
        }
        __syncthreads();
        // G <- G + Q^T dO - K^T dU (MSE)
        for (int e = tid; e < D * D; e += 256) {
            const int a = e / D, j = e % D;
            float s = 0.f;
            for (int i = 0; i < B; ++i) {
                s += Qs[i][a] * dOs[i][j];
                if (p.loss == 1) s -= Ks[i][a] * dUs[i][j];
            }
            G[a][j] += s;
        }
        __syncthreads();
    }
    for (int e = tid; e < D * D; e += 256) p.dw0[(long)h * D * D + e] = G[e / D][e % D];
}

}  // namespace

size_t linear_bwd_workspace(int NH, int T, int d, int chunk)
{
    const long nchunks = (T + chunk - 1) / chunk;
    return (size_t)NH * nchunks * d * d * sizeof(float);
}

hipError_t linear_bwd_launch(int NH, int T, int d, int chunk, int loss, int bf16, const void *q,
                             const void *k, const void *v, const float *eta, const float *w0,
                             const void *dout, const float *dwf, void *dq, void *dk, void *dv,
                             float *deta, float *dw0, void *ws, hipStream_t st)
{
    LinBwdParams p{q, k, v, dout, eta, w0, dwf, dq, dk, dv, deta, dw0, static_cast<float *>(ws),
                   T, (T + chunk - 1) / chunk, loss};
    const dim3 g(NH), b(256);
    if (chunk == 16) {
        if (bf16) {
            lin_bwd_states<64, 16, __bf16><<<g, b, 0, st>>>(p);
            lin_bwd_sweep<64, 16, __bf16><<<g, b, 0, st>>>(p);
        } else {
            lin_bwd_states<64, 16, float><<<g, b, 0, st>>>(p);
            lin_bwd_sweep<64, 16, float><<<g, b, 0, st>>>(p);
        }
    } else {
        if (bf16) {
            lin_bwd_states<64, 32, __bf16><<<g, b, 0, st>>>(p);
            lin_bwd_sweep<64, 32, __bf16><<<g, b, 0, st>>>(p);
        } else {
            lin_bwd_states<64, 32, float><<<g, b, 0, st>>>(p);
            lin_bwd_sweep<64, 32, float><<<g, b, 0, st>>>(p);
        }
    }
    return hipGetLastError();
}

}  // namespace tttk
