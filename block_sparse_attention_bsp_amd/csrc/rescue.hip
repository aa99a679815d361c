// Rescue branch, radius pass (thelatestinai page, RBS-Attention abstract: a
// rescue branch built on the maximum key-block radius catches blocks whose
// centroid hides a relevant key).  r[g][J] = max over the valid keys k of
// block J of ||k - Kbar_J||, with Kbar_J from the pool kernel.
//
// HBM-bound like pooling: K is read once more, with non-temporal 16-byte
// loads, one wavefront per (kv head, block) slab.  Lane t holds the means of
// its column chunk t % CH; each row's squared distance is summed across the
// CH lanes that share it, the maximum over rows is a wavefront max.
#include "device.h"
#include "internal.h"

namespace bsp {

typedef unsigned int u32x4r __attribute__((ext_vector_type(4)));

template <int DT, int D, int BLK>
__global__ __launch_bounds__(256) void radius_kernel(const uint8_t *__restrict__ k,
                                                     const float *__restrict__ k_scale,
                                                     const float *__restrict__ k_pool,
                                                     float *__restrict__ k_radius, int seq, int nb,
                                                     int nslab) {
  constexpr int ES = Storage<DT>::bytes;
  constexpr int VEC = 16 / ES;     // elements per 16-byte chunk
  constexpr int CH = D / VEC;      // chunks per row
  constexpr int RPL = 64 / CH;     // rows covered by one wave-wide load
  constexpr int NLD = BLK / RPL;   // loads per lane for a whole slab
  constexpr int BATCH = NLD < 16 ? NLD : 16;
  static_assert(CH * RPL == 64 && NLD * RPL == BLK, "tiling");
  const int lane = threadIdx.x & 63;
  const int sl = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (sl >= nslab) return;  // whole wavefronts only
  const int g = sl / nb, J = sl - g * nb;
  const int t0 = J * BLK;
  const int rows = min(BLK, seq - t0);
  const uint8_t *base = k + ((size_t)g * seq + t0) * D * ES;
  const int c = lane % CH, r0 = lane / CH;
  const float scale = DT == kFP8 ? k_scale[g] : 1.f;

  float mean[VEC];
  {
    const float *m = k_pool + ((size_t)g * nb + J) * D + c * VEC;
#pragma unroll
    for (int e = 0; e < VEC; e += 4) {
      const float4 t = *(const float4 *)(m + e);
      mean[e] = t.x;
      mean[e + 1] = t.y;
      mean[e + 2] = t.z;
      mean[e + 3] = t.w;
    }
  }

  float best = 0.f;
#pragma unroll
  for (int b0 = 0; b0 < NLD; b0 += BATCH) {
    u32x4r w[BATCH];
#pragma unroll
    for (int it = 0; it < BATCH; ++it) {
      const int r = r0 + (b0 + it) * RPL;
      const u32x4r *src = (const u32x4r *)(base + ((size_t)r * D + c * VEC) * ES);
      w[it] = r < rows ? __builtin_nontemporal_load(src) : u32x4r{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < BATCH; ++it) {
      float x[VEC];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t wd = w[it][j];
        if constexpr (DT == kF32) {
          x[j] = __uint_as_float(wd);
        } else if constexpr (DT == kBF16) {
          x[2 * j] = bf16_bits_to_f32(wd & 0xFFFFu);
          x[2 * j + 1] = bf16_bits_to_f32(wd >> 16);
        } else {
          const f32x2 lo = e4m3x2_to_f32(wd, false), hi = e4m3x2_to_f32(wd, true);
          x[4 * j] = lo.x;
          x[4 * j + 1] = lo.y;
          x[4 * j + 2] = hi.x;
          x[4 * j + 3] = hi.y;
        }
      }
      float d2 = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float t = x[e] * scale - mean[e];
        d2 = fmaf(t, t, d2);
      }
      // the CH lanes of one row are consecutive: sum across them (all lanes
      // take part; rows past the end contribute 0)
#pragma unroll
      for (int o = 1; o < CH; o <<= 1) d2 += __shfl_xor(d2, o, 64);
      const int r = r0 + (b0 + it) * RPL;
      best = fmaxf(best, r < rows ? d2 : 0.f);
    }
  }
#pragma unroll
  for (int o = CH; o < 64; o <<= 1) best = fmaxf(best, __shfl_xor(best, o, 64));
  if (lane == 0) k_radius[(size_t)g * nb + J] = sqrtf(best);
}

template <int DT, int D, int BLK>
static hipError_t launch_radius_t(const Shape &s, const void *k, const float *ks, const float *kp,
                                  float *kr, hipStream_t st) {
  const int nslab = s.hkv * s.nb;
  hipLaunchKernelGGL((radius_kernel<DT, D, BLK>), dim3((nslab + 3) / 4), dim3(256), 0, st,
                     (const uint8_t *)k, ks, kp, kr, s.seq, s.nb, nslab);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_radius_dt(const Shape &s, const void *k, const float *ks,
                                   const float *kp, float *kr, hipStream_t st) {
  if (s.d == 64 && s.block == 64) return launch_radius_t<DT, 64, 64>(s, k, ks, kp, kr, st);
  if (s.d == 64 && s.block == 128) return launch_radius_t<DT, 64, 128>(s, k, ks, kp, kr, st);
  if (s.d == 128 && s.block == 64) return launch_radius_t<DT, 128, 64>(s, k, ks, kp, kr, st);
  return launch_radius_t<DT, 128, 128>(s, k, ks, kp, kr, st);
}

hipError_t launch_radius(const Shape &s, const void *k, const float *k_scale,
                         const float *k_pool, float *k_radius, hipStream_t st) {
  if (s.dtype == kF32) return launch_radius_dt<kF32>(s, k, k_scale, k_pool, k_radius, st);
  if (s.dtype == kBF16) return launch_radius_dt<kBF16>(s, k, k_scale, k_pool, k_radius, st);
  return launch_radius_dt<kFP8>(s, k, k_scale, k_pool, k_radius, st);
}

}  // namespace bsp
