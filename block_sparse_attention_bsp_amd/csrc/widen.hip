// e4m3 -> bf16 widening of a V tensor (FP8 inference of the FlashPrefill V2
// abstract, thelatestinai.com page: e4m3 operands).  The O = P V product runs
// on bf16 matrix cores with V in bf16 either way; widening V once before the
// attention launch, instead of inside every workgroup that reads a V tile,
// lets the tiles reach LDS by direct loads as for bf16 inputs.  The widening
// is exact (e4m3 has 4 significant bits and a range inside bf16's), so the
// attention result is bit-identical to the one on the codes.
//
// HBM-bound: every code is read once and every bf16 written once, 16 codes
// per lane per step with non-temporal 16-byte loads and 32-byte stores
// (nothing is reused in this pass).
#include "device.h"
#include "internal.h"

namespace bsp {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void widen_kernel(const uint8_t *__restrict__ src,
                                                    uint16_t *__restrict__ dst, long n) {
  const long nv = n >> 4;  // whole 16-code chunks
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < nv; i += stride) {
    const u32x4v w = __builtin_nontemporal_load((const u32x4v *)src + i);
    u32x4v lo, hi;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      lo[2 * j] = e4m3x2_to_bf16x2(w[j], false);
      lo[2 * j + 1] = e4m3x2_to_bf16x2(w[j], true);
      hi[2 * j] = e4m3x2_to_bf16x2(w[j + 2], false);
      hi[2 * j + 1] = e4m3x2_to_bf16x2(w[j + 2], true);
    }
    __builtin_nontemporal_store(lo, (u32x4v *)dst + 2 * i);
    __builtin_nontemporal_store(hi, (u32x4v *)dst + 2 * i + 1);
  }
  // the last n % 16 codes, one per lane of the first wavefront
  if (blockIdx.x == 0 && threadIdx.x < (n & 15)) {
    const long e = (nv << 4) + threadIdx.x;
    dst[e] = (uint16_t)(e4m3x2_to_bf16x2(src[e], false) & 0xFFFFu);
  }
}

hipError_t launch_widen(const void *src, void *dst, long n, hipStream_t st) {
  const long nv = n >> 4;
  // about eight resident wavefronts per SIMD over the 256 CUs, or fewer
  // workgroups for small tensors
  const long want = (nv + 255) / 256;
  const unsigned grid = (unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096);
  hipLaunchKernelGGL(widen_kernel, dim3(grid), dim3(256), 0, st, (const uint8_t *)src,
                     (uint16_t *)dst, n);
  return hipGetLastError();
}

}  // namespace bsp
