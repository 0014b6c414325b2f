// Single-token decode steps on a carried fast-weight state.
//
// A decode step reads a whole state per (batch, head) for one token, so it is
// a batched matrix-vector product: 2 flops per 4-byte state element read.  It
// is bound by HBM bandwidth, not by the matrix cores, and runs on fp32 vector
// FMAs with every state element read (and, for TTT-Linear, written) once by
// one thread in 16-byte accesses.
//
// TTT-Linear ("Test-Time Training (TTT)", "TTT definition": one gradient step
// per token, output read after the step; examples 1 and 2 for the gradients;
// "Mini-batch gradient descent" for the chunk-start anchor):
//     u = v - k A  (MSE)  or  v  (inner product);   W <- W + eta k^T u;
//     y = q W = q W_old + eta (q . k) u
// with A = W (chunk size 1) or the chunk-start state held by the caller.
//
// LaCT ("LaCT: Test-Time Training Done Right", section 3.2 for the SwiGLU
// fast weight, section 4 for the causal order in which a chunk's queries read
// the chunk-start weights): y = W2 (silu(W1 q) * (W3 q)), in two launches
// (hidden activations, then the output rows), with the hidden vector of each
// head passed through the caller's workspace.
#include "ttt_device.h"
#include "ttt_internal.h"

#include <hip/hip_runtime.h>

namespace tttk {
namespace {

__device__ __forceinline__ float wave_sum(float s)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    return s;
}

__device__ __forceinline__ f32x4 lds4(const float *p)
{
    return f32x4{p[0], p[1], p[2], p[3]};
}

// ---- TTT-Linear ---------------------------------------------------------------
struct LinDecodeParams {
    const void *q, *k, *v;
    const float *eta;
    float *w;
    float *anchor;
    void *out;
    int anchor_update;
};

// One workgroup of 256 threads per (batch, head).  Thread (rg, cg) owns the
// four columns 4cg..4cg+3 of the rows r = i*RG + rg, so one wave-wide load
// instruction reads 64 / CG whole consecutive rows (1 KiB contiguous).
template <int D> struct LinDecodeTile {
    static constexpr int NT = 256;
    static constexpr int CG = D / 4;    // four-column groups per row
    static constexpr int RG = NT / CG;  // row groups (16 at d = 64, 8 at d = 128)
    static constexpr int RPT = D / RG;  // rows per thread (4 or 16)
};

template <int D, typename E, bool MSE, bool ANCHOR>
__global__ __launch_bounds__(256) void lin_decode(LinDecodeParams p)
{
    using T = LinDecodeTile<D>;
    __shared__ float sq[D], sk[D], sv[D], sqw[D], skw[D];
    __shared__ f32x4 red[2][T::RG][T::CG];
    __shared__ float sqk;
    const int h = blockIdx.x;
    const int tid = threadIdx.x;
    const int cg = tid % T::CG, rg = tid / T::CG;
    const size_t tok = (size_t)h * D;
    float *W = p.w + (size_t)h * D * D;
    const float *A = ANCHOR ? p.anchor + (size_t)h * D * D : nullptr;

    if (tid < D) {
        sq[tid] = (float)static_cast<const E *>(p.q)[tok + tid];
        sk[tid] = (float)static_cast<const E *>(p.k)[tok + tid];
        sv[tid] = (float)static_cast<const E *>(p.v)[tok + tid];
    }
    const float eta = p.eta[h];
    f32x4 wv[T::RPT];
#pragma unroll
    for (int i = 0; i < T::RPT; ++i)
        wv[i] = *reinterpret_cast<const f32x4 *>(W + (size_t)(i * T::RG + rg) * D + 4 * cg);
    __syncthreads();

    // partial q W and k A over this thread's rows
    f32x4 pq = zero4(), pk = zero4();
#pragma unroll
    for (int i = 0; i < T::RPT; ++i) {
        const int r = i * T::RG + rg;
        pq += sq[r] * wv[i];
        if constexpr (MSE && !ANCHOR) pk += sk[r] * wv[i];
    }
    if constexpr (MSE && ANCHOR) {
#pragma unroll
        for (int i = 0; i < T::RPT; ++i) {
            const int r = i * T::RG + rg;
            pk += sk[r] * *reinterpret_cast<const f32x4 *>(A + (size_t)r * D + 4 * cg);
        }
    }
    red[0][rg][cg] = pq;
    if constexpr (MSE) red[1][rg][cg] = pk;
    __syncthreads();
    if (tid < T::CG) {  // wave 0: q W
        f32x4 s = zero4();
#pragma unroll
        for (int j = 0; j < T::RG; ++j) s += red[0][j][tid];
#pragma unroll
        for (int e = 0; e < 4; ++e) sqw[4 * tid + e] = s[e];
    } else if (MSE && tid >= 64 && tid < 64 + T::CG) {  // wave 1: k A
        const int c = tid - 64;
        f32x4 s = zero4();
#pragma unroll
        for (int j = 0; j < T::RG; ++j) s += red[1][j][c];
#pragma unroll
        for (int e = 0; e < 4; ++e) skw[4 * c + e] = s[e];
    } else if (tid >= 128 && tid < 192) {  // wave 2: q . k
        const int l = tid - 128;
        float s = 0.f;
        for (int e = l; e < D; e += 64) s += sq[e] * sk[e];
        s = wave_sum(s);
        if (l == 0) sqk = s;
    }
    __syncthreads();

    f32x4 u = lds4(sv + 4 * cg);
    if constexpr (MSE) u -= lds4(skw + 4 * cg);
#pragma unroll
    for (int i = 0; i < T::RPT; ++i) {
        const int r = i * T::RG + rg;
        const f32x4 wn = wv[i] + (eta * sk[r]) * u;
        *reinterpret_cast<f32x4 *>(W + (size_t)r * D + 4 * cg) = wn;
        if constexpr (ANCHOR)
            if (p.anchor_update) *reinterpret_cast<f32x4 *>(p.anchor + (size_t)h * D * D + (size_t)r * D + 4 * cg) = wn;
    }
    if (rg == 0) {
        const f32x4 y = lds4(sqw + 4 * cg) + (eta * sqk) * u;
        store4<E>(static_cast<E *>(p.out) + tok + 4 * cg, out4<E>(y));
    }
}

template <int D, typename E>
hipError_t lin_decode_dispatch(int NH, bool mse, bool anchor, const LinDecodeParams &p,
                               hipStream_t st)
{
    const dim3 g(NH), b(256);
    if (mse) {
        if (anchor) lin_decode<D, E, true, true><<<g, b, 0, st>>>(p);
        else lin_decode<D, E, true, false><<<g, b, 0, st>>>(p);
    } else {
        if (anchor) lin_decode<D, E, false, true><<<g, b, 0, st>>>(p);
        else lin_decode<D, E, false, false><<<g, b, 0, st>>>(p);
    }
    return hipGetLastError();
}

// ---- LaCT SwiGLU ----------------------------------------------------------------
// Each wave owns 16 consecutive weight rows and accumulates one partial dot
// product per row in every lane; a butterfly over lane offsets 32, 16, 8, 4
// halves the rows held per lane at each step (17 cross-lane exchanges for 16
// rows instead of 6 per row), then offsets 2 and 1 finish the sums.  Lane l
// ends with the full sum of row
//     rev(l) = 8 * bit5(l) + 4 * bit4(l) + 2 * bit3(l) + bit2(l),
// held identically by the four lanes with the same l >> 2.
template <int N, int OFF>
__device__ __forceinline__ void fold_half(float (&acc)[16], int lane)
{
    const bool up = (lane & OFF) != 0;
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        const float send = up ? acc[j] : acc[j + N / 2];
        const float keep = up ? acc[j + N / 2] : acc[j];
        acc[j] = keep + __shfl_xor(send, OFF);
    }
}

__device__ __forceinline__ float rows16_reduce(float (&acc)[16], int lane)
{
    fold_half<16, 32>(acc, lane);
    fold_half<8, 16>(acc, lane);
    fold_half<4, 8>(acc, lane);
    fold_half<2, 4>(acc, lane);
    float s = acc[0];
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 1);
    return s;
}

__device__ __forceinline__ int rows16_row(int lane)
{
    return ((lane >> 5) & 1) * 8 + ((lane >> 4) & 1) * 4 + ((lane >> 3) & 1) * 2 + ((lane >> 2) & 1);
}

struct LactDecodeParams {
    const void *q;
    const float *w1, *w2, *w3;
    void *out;
    float *g;  // [NH][hid] workspace
    int d, hid;
};

// Hidden activations: block = (head, 64 hidden rows); g = silu(W1 q) * (W3 q).
template <typename E>
__global__ __launch_bounds__(256) void lact_decode_hidden(LactDecodeParams p)
{
    extern __shared__ float sx[];  // q of this head, fp32 [d]
    const int nrb = p.hid / 64;
    const int h = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < p.d; e += 256) sx[e] = (float)static_cast<const E *>(p.q)[(size_t)h * p.d + e];
    __syncthreads();
    const int r0 = rb * 64 + wave * 16;
    const float *W1 = p.w1 + ((size_t)h * p.hid + r0) * p.d;
    const float *W3 = p.w3 + ((size_t)h * p.hid + r0) * p.d;
    float a1[16], a3[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a1[i] = a3[i] = 0.f;
    const int n4 = p.d / 4;
    for (int e = lane; e < n4; e += 64) {
        const f32x4 x = lds4(sx + 4 * e);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const f32x4 u = *reinterpret_cast<const f32x4 *>(W1 + (size_t)i * p.d + 4 * e);
            const f32x4 w = *reinterpret_cast<const f32x4 *>(W3 + (size_t)i * p.d + 4 * e);
            a1[i] += u[0] * x[0] + u[1] * x[1] + u[2] * x[2] + u[3] * x[3];
            a3[i] += w[0] * x[0] + w[1] * x[1] + w[2] * x[2] + w[3] * x[3];
        }
    }
    const float z1 = rows16_reduce(a1, lane);
    const float z3 = rows16_reduce(a3, lane);
    if ((lane & 3) == 0) {
        const float s = 1.f / (1.f + expf(-z1));
        p.g[(size_t)h * p.hid + r0 + rows16_row(lane)] = z1 * s * z3;
    }
}

// Output rows: block = (head, 64 output rows); y = W2 g.
template <typename E>
__global__ __launch_bounds__(256) void lact_decode_out(LactDecodeParams p)
{
    extern __shared__ float sg[];  // g of this head, fp32 [hid]
    const int nrb = p.d / 64;
    const int h = blockIdx.x / nrb, rb = blockIdx.x % nrb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int e = tid; e < p.hid; e += 256) sg[e] = p.g[(size_t)h * p.hid + e];
    __syncthreads();
    const int r0 = rb * 64 + wave * 16;
    const float *W2 = p.w2 + ((size_t)h * p.d + r0) * p.hid;
    float a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = 0.f;
    const int n4 = p.hid / 4;
    for (int e = lane; e < n4; e += 64) {
        const f32x4 x = lds4(sg + 4 * e);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const f32x4 u = *reinterpret_cast<const f32x4 *>(W2 + (size_t)i * p.hid + 4 * e);
            a[i] += u[0] * x[0] + u[1] * x[1] + u[2] * x[2] + u[3] * x[3];
        }
    }
    const float y = rows16_reduce(a, lane);
    if ((lane & 3) == 0)
        static_cast<E *>(p.out)[(size_t)h * p.d + r0 + rows16_row(lane)] = (E)y;
}

}  // namespace

hipError_t linear_decode_launch(int NH, int d, int bf16, int loss, const void *q, const void *k,
                                const void *v, const float *eta, float *w, float *anchor,
                                int anchor_update, void *out, hipStream_t st)
{
    LinDecodeParams p{q, k, v, eta, w, anchor, out, anchor_update};
    const bool mse = loss == 1, an = anchor != nullptr;
    if (d == 64) return bf16 ? lin_decode_dispatch<64, __bf16>(NH, mse, an, p, st)
                             : lin_decode_dispatch<64, float>(NH, mse, an, p, st);
    return bf16 ? lin_decode_dispatch<128, __bf16>(NH, mse, an, p, st)
                : lin_decode_dispatch<128, float>(NH, mse, an, p, st);
}

size_t lact_decode_workspace(int NH, int hid) { return (size_t)NH * hid * sizeof(float); }

hipError_t lact_decode_launch(int NH, int d, int hid, int bf16, const void *q, const float *w1,
                              const float *w2, const float *w3, void *out, void *ws, hipStream_t st)
{
    LactDecodeParams p{q, w1, w2, w3, out, static_cast<float *>(ws), d, hid};
    const dim3 b(256);
    if (bf16) {
        lact_decode_hidden<__bf16><<<dim3(NH * (hid / 64)), b, d * sizeof(float), st>>>(p);
        lact_decode_out<__bf16><<<dim3(NH * (d / 64)), b, hid * sizeof(float), st>>>(p);
    } else {
        lact_decode_hidden<float><<<dim3(NH * (hid / 64)), b, d * sizeof(float), st>>>(p);
        lact_decode_out<float><<<dim3(NH * (d / 64)), b, hid * sizeof(float), st>>>(p);
    }
    return hipGetLastError();
}

}  // namespace tttk
