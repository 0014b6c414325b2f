// Measurement helpers (not part of the TTT path): a loop of independent bf16
// matrix-core products, from which a benchmark reads the dense bf16 MFMA
// rate this part reaches, to quote roofline fractions against a measured peak
// beside the published one; and the LaCT kernels' shared GEMM tile on its own,
// so its rate can be measured on plain products.
#include "../../include/ttt.h"
#include "lact_common.h"

namespace tttk {

// Every wave keeps four independent 32x32x16 accumulations in flight, so the
// matrix pipe never waits on a dependent result (on gfx950 this shape reaches
// about 1.6x the rate of the 16x16x32 one, measured with the same loop, so it
// is the one that shows the part's dense bf16 ceiling).  Operands come from
// the lane index (never zero, so nothing is folded away); the sum of the
// accumulators is written so the loop cannot be removed.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256) void probe_mfma_loop(float *out, int iters)
{
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (__bf16)(1.0f + 0.001f * (lane + j));
        b[j] = (__bf16)(1.0f - 0.001f * (lane + 2 * j));
    }
    f32x16 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// C[m][n] = sum_k A[m][k] B[n][k] on the shared (32 MB) x 128 tile, fp32 out;
// one workgroup per output tile.
template <bool AT, bool BT, int MB>
__global__ __launch_bounds__(256) void probe_gemm_tile(const bf16 *A, const bf16 *B, float *C, int M, int N, int K)
{
    __shared__ GemmLdsT<32 * MB> L;
    const int tn_n = N / 128;
    const int bid = xcd_block(blockIdx.x, gridDim.x);
    const int tm = bid / tn_n, tn = bid % tn_n;
    const bf16 *as[1] = {A}, *bs[1] = {B};
    gemm_nt_tile<AT, BT, MB>(L, as, AT ? M : K, bs, BT ? N : K, M, N, K, 1, tm * (32 * MB), tn * 128, K,
                             [&](f32x4 (&acc)[MB][4], int mb, int nb, int g, int mm) {
#pragma unroll
                                 for (int i = 0; i < MB; ++i)
#pragma unroll
                                     for (int q = 0; q < 4; ++q)
#pragma unroll
                                         for (int r = 0; r < 4; ++r)
                                             C[(long)(mb + 16 * i + 4 * g + r) * N + nb + 16 * q + mm] = acc[i][q][r];
                             });
}

// The eight-wave form of the 128 x 128 tile (two groups of waves splitting k).
template <bool AT, bool BT>
__global__ __launch_bounds__(512) void probe_gemm_tile_kg2(const bf16 *A, const bf16 *B, float *C, int M, int N,
                                                           int K)
{
    __shared__ GemmLds L[2];
    const int tn_n = N / 128;
    const int bid = xcd_block(blockIdx.x, gridDim.x);
    const int tm = bid / tn_n, tn = bid % tn_n;
    const bf16 *as[1] = {A}, *bs[1] = {B};
    gemm_nt_tile_kg2<AT, BT>(L, as, AT ? M : K, bs, BT ? N : K, M, N, K, 1, tm * 128, tn * 128, K,
                             [&](f32x4 (&acc)[4][4], int mb, int nb, int g, int mm) {
#pragma unroll
                                 for (int i = 0; i < 4; ++i)
#pragma unroll
                                     for (int q = 0; q < 4; ++q)
#pragma unroll
                                         for (int r = 0; r < 4; ++r)
                                             C[(long)(mb + 16 * i + 4 * g + r) * N + nb + 16 * q + mm] = acc[i][q][r];
                             });
}

template <int MB>
static void probe_gemm_launch(const bf16 *A, const bf16 *B, float *c, int M, int N, int K, int ak, int bk,
                              hipStream_t st)
{
    const dim3 grid((M / (32 * MB)) * (N / 128)), block(256);
    if (ak && bk)
        probe_gemm_tile<true, true, MB><<<grid, block, 0, st>>>(A, B, c, M, N, K);
    else if (ak)
        probe_gemm_tile<true, false, MB><<<grid, block, 0, st>>>(A, B, c, M, N, K);
    else if (bk)
        probe_gemm_tile<false, true, MB><<<grid, block, 0, st>>>(A, B, c, M, N, K);
    else
        probe_gemm_tile<false, false, MB><<<grid, block, 0, st>>>(A, B, c, M, N, K);
}

}  // namespace tttk

extern "C" ttt_status ttt_probe_gemm_bf16(const void *a, const void *b, float *c, int M, int N, int K, int a_kmajor,
                                          int b_kmajor, int block_rows, int wave_groups, void *stream)
{
    if (!a || !b || !c || (block_rows != 64 && block_rows != 128 && block_rows != 256)) return TTT_EINVAL;
    if (wave_groups != 1 && (wave_groups != 2 || block_rows != 128)) return TTT_EINVAL;
    if (M < block_rows || N < 128 || K < 64 || M % block_rows || N % 128 || K % 64) return TTT_EINVAL;
    if ((long long)(M / block_rows) * (N / 128) > (1 << 24)) return TTT_EUNSUPPORTED;
    const tttk::bf16 *A = (const tttk::bf16 *)a, *B = (const tttk::bf16 *)b;
    hipStream_t st = (hipStream_t)stream;
    if (wave_groups == 2) {
        const dim3 grid((M / 128) * (N / 128)), block(512);
        if (a_kmajor && b_kmajor)
            tttk::probe_gemm_tile_kg2<true, true><<<grid, block, 0, st>>>(A, B, c, M, N, K);
        else if (a_kmajor)
            tttk::probe_gemm_tile_kg2<true, false><<<grid, block, 0, st>>>(A, B, c, M, N, K);
        else if (b_kmajor)
            tttk::probe_gemm_tile_kg2<false, true><<<grid, block, 0, st>>>(A, B, c, M, N, K);
        else
            tttk::probe_gemm_tile_kg2<false, false><<<grid, block, 0, st>>>(A, B, c, M, N, K);
    } else if (block_rows == 256)
        tttk::probe_gemm_launch<8>(A, B, c, M, N, K, a_kmajor, b_kmajor, st);
    else if (block_rows == 64)
        tttk::probe_gemm_launch<2>(A, B, c, M, N, K, a_kmajor, b_kmajor, st);
    else
        tttk::probe_gemm_launch<4>(A, B, c, M, N, K, a_kmajor, b_kmajor, st);
    return hipGetLastError() == hipSuccess ? TTT_OK : TTT_EHIP;
}

extern "C" ttt_status ttt_probe_mfma_bf16(float *out, int blocks, int iters, void *stream)
{
    if (!out || blocks < 1 || iters < 1 || blocks > (1 << 20)) return TTT_EINVAL;
    tttk::probe_mfma_loop<<<dim3(blocks), dim3(256), 0, (hipStream_t)stream>>>(out, iters);
    return hipGetLastError() == hipSuccess ? TTT_OK : TTT_EHIP;
}
