// Stage 1a: block mean pooling of Q and K (FlashPrefill summary page,
// section 3 "Instantaneous Pattern Discovery": average-pooled key blocks
// stand in for their tokens; Appendix B: key blocks are pre-pooled).
//
// HBM-bound: every byte of Q and K is read once, with non-temporal 16-byte
// loads (nothing is reused within this pass, and streaming past the caches
// raises the achieved read rate by about 15%).  One workgroup owns one
// (head, block) pair, a contiguous B x d slab (32 KiB for bf16 at
// B = d = 128): lane t reads 16-byte column chunk t % CH of rows t / CH,
// t / CH + RG, ...  Partial column sums meet in LDS.
#include "device.h"
#include "internal.h"

namespace bsp {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

template <int DT, int D, int BLK>
__global__ __launch_bounds__(256) void pool_kernel(const uint8_t *__restrict__ q,
                                                   const uint8_t *__restrict__ k,
                                                   const float *__restrict__ q_scale,
                                                   const float *__restrict__ k_scale,
                                                   float *__restrict__ q_pool,
                                                   float *__restrict__ k_pool, int hq, int seq,
                                                   int nb) {
  constexpr int ES = Storage<DT>::bytes;
  constexpr int VEC = 16 / ES;     // elements per 16-byte chunk
  constexpr int CH = D / VEC;      // chunks per row
  constexpr int RG = 256 / CH;     // row groups
  constexpr int ITER = BLK / RG;   // rows per thread for a full block
  static_assert(CH * RG == 256 && ITER * RG == BLK, "tiling");
  __shared__ float part[RG][D + 1];

  const int I = blockIdx.x;
  const int hh = blockIdx.y;
  const bool isq = hh < hq;
  const int h = isq ? hh : hh - hq;
  const int t0 = I * BLK;
  const int rows = min(BLK, seq - t0);
  const uint8_t *base = (isq ? q : k) + ((size_t)h * seq + t0) * D * ES;
  const int c = threadIdx.x % CH;
  const int r0 = threadIdx.x / CH;

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;

  uint4 w[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int r = r0 + it * RG;
    const u32x4v *src = (const u32x4v *)(base + ((size_t)r * D + c * VEC) * ES);
    const u32x4v t = r < rows ? __builtin_nontemporal_load(src) : u32x4v{0u, 0u, 0u, 0u};
    w[it] = make_uint4(t.x, t.y, t.z, t.w);
  }
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const uint32_t wd[4] = {w[it].x, w[it].y, w[it].z, w[it].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (DT == kF32) {
        acc[j] += __uint_as_float(wd[j]);
      } else if constexpr (DT == kBF16) {
        acc[2 * j] += bf16_bits_to_f32(wd[j] & 0xFFFFu);
        acc[2 * j + 1] += bf16_bits_to_f32(wd[j] >> 16);
      } else {
        const f32x2 lo = e4m3x2_to_f32(wd[j], false), hi = e4m3x2_to_f32(wd[j], true);
        acc[4 * j] += lo.x;
        acc[4 * j + 1] += lo.y;
        acc[4 * j + 2] += hi.x;
        acc[4 * j + 3] += hi.y;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < VEC; ++e) part[r0][c * VEC + e] = acc[e];
  __syncthreads();

  float scale = 1.f;
  if constexpr (DT == kFP8) scale = isq ? q_scale[h] : k_scale[h];
  float *out = (isq ? q_pool : k_pool) + ((size_t)h * nb + I) * D;
  const float inv = scale / (float)rows;
  for (int e = threadIdx.x; e < D; e += 256) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < RG; ++g) s += part[g][e];
    out[e] = s * inv;
  }
}

template <int DT, int D, int BLK>
static hipError_t launch_pool_t(const Shape &s, const void *q, const void *k, const float *qs,
                                const float *ks, float *qp, float *kp, hipStream_t st) {
  dim3 grid(s.nb, s.hq + s.hkv);
  hipLaunchKernelGGL((pool_kernel<DT, D, BLK>), grid, dim3(256), 0, st, (const uint8_t *)q,
                     (const uint8_t *)k, qs, ks, qp, kp, s.hq, s.seq, s.nb);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_pool_dt(const Shape &s, const void *q, const void *k, const float *qs,
                                 const float *ks, float *qp, float *kp, hipStream_t st) {
  if (s.d == 64 && s.block == 64) return launch_pool_t<DT, 64, 64>(s, q, k, qs, ks, qp, kp, st);
  if (s.d == 64 && s.block == 128) return launch_pool_t<DT, 64, 128>(s, q, k, qs, ks, qp, kp, st);
  if (s.d == 128 && s.block == 64) return launch_pool_t<DT, 128, 64>(s, q, k, qs, ks, qp, kp, st);
  return launch_pool_t<DT, 128, 128>(s, q, k, qs, ks, qp, kp, st);
}

hipError_t launch_pool(const Shape &s, const void *q, const void *k, const float *qs,
                       const float *ks, float *qp, float *kp, hipStream_t st) {
  if (s.dtype == kF32) return launch_pool_dt<kF32>(s, q, k, qs, ks, qp, kp, st);
  if (s.dtype == kBF16) return launch_pool_dt<kBF16>(s, q, k, qs, ks, qp, kp, st);
  return launch_pool_dt<kFP8>(s, q, k, qs, ks, qp, kp, st);
}

}  // namespace bsp
