// Device-side helpers shared by the gfx950 kernels of libbsp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage dtypes (values of bsp_dtype).
constexpr int kF32 = 0;
constexpr int kBF16 = 1;
constexpr int kFP8 = 2;
constexpr int kFP8V16 = 3;  // e4m3 Q and K, V widened to bf16

template <int DT> struct Storage;
template <> struct Storage<kF32> { static constexpr int bytes = 4; };
template <> struct Storage<kBF16> { static constexpr int bytes = 2; };
template <> struct Storage<kFP8> { static constexpr int bytes = 1; };

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// OCP e4m3fn code -> float, by the format: bias 7, 3 mantissa bits,
// exponent 0 subnormal; the NaN code never occurs in valid inputs.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return __uint_as_float(__float_as_uint(v) | s);
}

// Two OCP e4m3fn codes (bytes 0-1 of w if !hi, bytes 2-3 if hi) -> two
// floats / two bf16 (both exact: e4m3 has 4 significant bits), on the gfx950
// conversion units.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x2 e4m3x2_to_f32(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
            : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
  const bf16x2 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, true)
                      : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, false);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

// fp32 -> three bf16 planes, x = hi + mid + lo exactly: each plane is the
// bf16 rounding (to nearest even) of what the planes before it leave, every
// such remainder is exact in fp32, and the last one has at most 8
// significant bits.  A product of two planes is exact in fp32.  Pairs of
// elements share one conversion (v_cvt_pk_bf16_f32) and fill one register of
// each plane; a remainder x - plane is one v_dot2c_f32_bf16 of the packed
// plane with (-1, 0) or (0, -1) accumulated onto x (exact, as the difference
// is representable).  The two constants are kept opaque in registers: folded,
// (-1, 0) becomes the inline constant -1.0, which the hardware does not read
// as that bf16 pair (the scores came out wrong).  V is a bf16 vector of N
// elements.
template <int N, typename V>
__device__ __forceinline__ void split3(const float (&x)[N], V &hi, V &mi, V &lo) {
  static_assert(N % 2 == 0, "pairs of elements");
  uint32_t b0 = 0x0000bf80u, b1 = 0xbf800000u;  // bf16 pairs (-1, 0) and (0, -1)
  asm volatile("" : "+v"(b0), "+v"(b1));
  bf16x2 n0, n1;
  __builtin_memcpy(&n0, &b0, 4);
  __builtin_memcpy(&n1, &b1, 4);
#pragma unroll
  for (int e = 0; e < N; e += 2) {
    const bf16x2 h = __builtin_convertvector((f32x2{x[e], x[e + 1]}), bf16x2);
    const float r0 = __builtin_amdgcn_fdot2_f32_bf16(h, n0, x[e], false);
    const float r1 = __builtin_amdgcn_fdot2_f32_bf16(h, n1, x[e + 1], false);
    const bf16x2 m = __builtin_convertvector((f32x2{r0, r1}), bf16x2);
    const float s0 = __builtin_amdgcn_fdot2_f32_bf16(m, n0, r0, false);
    const float s1 = __builtin_amdgcn_fdot2_f32_bf16(m, n1, r1, false);
    const bf16x2 l = __builtin_convertvector((f32x2{s0, s1}), bf16x2);
    hi[e] = h[0], hi[e + 1] = h[1];
    mi[e] = m[0], mi[e + 1] = m[1];
    lo[e] = l[0], lo[e + 1] = l[1];
  }
}

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Buffer descriptor over [base, base + bytes): raw (stride 0), untyped
// 32-bit data format as gfx9-family untyped buffer loads expect.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16 bytes per lane from rsrc + soff + voff straight into LDS at ldst + 16 * lane
// (buffer_load_dwordx4 ... lds): no VGPR staging and no 64-bit address math.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                          void *ldst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)ldst, 16,
                                           voff, soff, 0, 0);
}

// Packed variable-length batch: the sequence whose query blocks
// cu_blocks[s] .. cu_blocks[s+1] contain batch block gb (binary search over
// the nseq + 1 nondecreasing offsets).
__device__ __forceinline__ int varlen_seq_of(const int32_t *cu_blocks, int nseq, int gb) {
  int lo = 0, hi = nseq;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cu_blocks[mid] <= gb) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace bsp
