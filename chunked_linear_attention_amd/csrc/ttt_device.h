// Device-side helpers shared by the gfx950 kernels: MFMA fragment types and
// wrappers, bf16 conversion, small vector loads.
//
// Wave-level fragment conventions (64 lanes, lane l, g = l >> 4, m = l & 15),
// for a 16 x 16 output tile C and a 16-deep slice of the contraction index k:
//   C tile  (f32x4 acc): acc[j] = C[4g + j][m]
//   A frag  (4 elements): a[j]  = A[m][4g + j]        (row m, k = 4g + j)
//   B frag  (4 elements): b[j]  = B[4g + j][m]        (k = 4g + j, column m)
// so an accumulator tile converted to bf16 is directly a B fragment (rows = k)
// and an A fragment of the transposed product.  A 32-deep product pairs two
// 16-deep fragments on both sides; the hardware k order inside the pair is a
// permutation applied identically to A and B, so the sum is unchanged.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tttk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename E> struct Frag;
template <> struct Frag<float> { typedef f32x4 type; };
template <> struct Frag<__bf16> { typedef bf16x4 type; };

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---- conversions -----------------------------------------------------------
// Round to nearest even; compiles to paired v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ f32x4 to_f32x4(bf16x4 x) { return __builtin_convertvector(x, f32x4); }

// x = hi + lo with hi = bf16(x) (nearest even) and lo = bf16(x - hi), where
// x - hi is exact in fp32: about 16 mantissa bits in two bf16 operands, and hi
// alone is the correctly rounded single operand.
__device__ __forceinline__ void split_bf16x4(f32x4 x, bf16x4 &hi, bf16x4 &lo)
{
    hi = to_bf16x4(x);
    const u32x2 hb = __builtin_bit_cast(u32x2, hi);
    f32x4 hf;
    hf[0] = __builtin_bit_cast(float, hb[0] << 16);
    hf[1] = __builtin_bit_cast(float, hb[0] & 0xFFFF0000u);
    hf[2] = __builtin_bit_cast(float, hb[1] << 16);
    hf[3] = __builtin_bit_cast(float, hb[1] & 0xFFFF0000u);
    lo = to_bf16x4(x - hf);
}
template <typename E> __device__ __forceinline__ typename Frag<E>::type to_frag(f32x4 x);
template <> __device__ __forceinline__ f32x4 to_frag<float>(f32x4 x) { return x; }
template <> __device__ __forceinline__ bf16x4 to_frag<__bf16>(f32x4 x) { return to_bf16x4(x); }
__device__ __forceinline__ f32x4 frag_to_f32(f32x4 x) { return x; }
__device__ __forceinline__ f32x4 frag_to_f32(bf16x4 x) { return to_f32x4(x); }

// ---- MFMA wrappers ---------------------------------------------------------
// acc += A(16x16 slice) * B(16x16 slice), contraction depth 16.
__device__ __forceinline__ f32x4 mma16(f32x4 acc, bf16x4 a, bf16x4 b)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f32x4 acc, f32x4 a, f32x4 b)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    return acc;
}
// Contraction depth 32 from two 16-deep fragment pairs.
__device__ __forceinline__ f32x4 mma32(f32x4 acc, bf16x4 a0, bf16x4 a1, bf16x4 b0, bf16x4 b1)
{
    bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(f32x4 acc, f32x4 a0, f32x4 a1, f32x4 b0, f32x4 b1)
{
    acc = mma16(acc, a0, b0);
    return mma16(acc, a1, b1);
}
// A single 16-deep product issued in the 32-deep shape (second half zero), so
// an accumulation chain never mixes MFMA shapes; a 16x16x16 bf16 MFMA costs
// as much as a 16x16x32 one on gfx950.  fp32 has no such shape change.
__device__ __forceinline__ f32x4 mma32z(f32x4 acc, bf16x4 a0, bf16x4 b0)
{
    const bf16x4 z = {(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
    return mma32(acc, a0, z, b0, z);
}
__device__ __forceinline__ f32x4 mma32z(f32x4 acc, f32x4 a0, f32x4 b0) { return mma16(acc, a0, b0); }

// Transposing read (16-bit elements): within each group of 16 lanes, lane i
// slot j receives the element that lane 4j + i/4 would read at slot i%4.
// Lane (m, g) pointing at row 4g + m/4, column c0 + 4(m%4) of a row-major
// tile therefore receives tile[4g + j][c0 + m], j = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16 *p)
{
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
    const v4bf r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) v4bf *)((__attribute__((address_space(3))) char *)p));
    return __builtin_bit_cast(bf16x4, r);
}

// ---- workgroup placement ------------------------------------------------------
// Workgroups are dealt to the 8 XCDs round-robin (XCD = block index mod 8),
// and each XCD has its own L2.  Renumber blocks so that logical blocks
// [x * n/8, (x + 1) * n/8) all run on XCD x: kernels order their logical
// index so that blocks sharing data are consecutive, and the data is then
// fetched into one L2 instead of eight.
__device__ __forceinline__ int xcd_block(int b, int n)
{
    return (n % 8) ? b : (b % 8) * (n / 8) + b / 8;
}

// ---- small vector memory helpers --------------------------------------------
// Four consecutive elements (8 bytes for bf16, 16 bytes for fp32).
template <typename E> struct Vec4;
template <> struct Vec4<float> {
    typedef f32x4 type;
};
template <> struct Vec4<__bf16> {
    typedef bf16x4 type;
};

template <typename E>
__device__ __forceinline__ typename Vec4<E>::type load4(const E *p)
{
    return *reinterpret_cast<const typename Vec4<E>::type *>(p);
}
template <typename E>
__device__ __forceinline__ void store4(E *p, typename Vec4<E>::type v)
{
    *reinterpret_cast<typename Vec4<E>::type *>(p) = v;
}

template <typename E> __device__ __forceinline__ typename Vec4<E>::type zero_vec4();
template <> __device__ __forceinline__ f32x4 zero_vec4<float>() { return zero4(); }
template <> __device__ __forceinline__ bf16x4 zero_vec4<__bf16>()
{
    return bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
}

// Output rounding to the storage type.
template <typename E> __device__ __forceinline__ typename Vec4<E>::type out4(f32x4 x);
template <> __device__ __forceinline__ f32x4 out4<float>(f32x4 x) { return x; }
template <> __device__ __forceinline__ bf16x4 out4<__bf16>(f32x4 x) { return to_bf16x4(x); }

// Workgroup barrier for LDS hand-offs only: waits for this wave's LDS
// operations (lgkmcnt = 0) and meets the other waves, but leaves global loads
// in flight (a plain __syncthreads() also drains every outstanding global
// load, which would defeat the prefetch ring).  The wavefront-scope fences
// only stop the compiler from moving memory operations across the barrier.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt = max, expcnt = max, lgkmcnt = 0
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace tttk
