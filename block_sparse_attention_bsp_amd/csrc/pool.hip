// Stage 1a: block mean pooling of Q and K (FlashPrefill summary page,
// section 3 "Instantaneous Pattern Discovery": average-pooled key blocks
// stand in for their tokens; Appendix B: key blocks are pre-pooled).
//
// HBM-bound: every byte of Q and K is read once, with non-temporal 16-byte
// loads (nothing is reused within this pass, and streaming past the caches
// raises the achieved read rate by about 15%).  One wavefront owns one
// (head, block) slab, a contiguous B x d region (32 KiB for bf16 at
// B = d = 128): lane t reads 16-byte column chunk t % CH of rows t / CH,
// t / CH + 64 / CH, ..., with all of a lane's loads for the slab in flight
// together.  The lanes that share a column chunk then combine their partial
// sums with cross-lane adds: no LDS and no barrier.
#include "device.h"
#include "internal.h"

namespace bsp {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// VL: a packed variable-length batch (seq = its tokens, nb = its query
// blocks); the query block of batch block I is block I - cu_blocks[s] of
// sequence s, and its keys are cache page page_table[s][that block], laid out
// [page][hkv][BLK][d].
template <int DT, int D, int BLK, bool VL>
__global__ __launch_bounds__(256) void pool_kernel(const uint8_t *__restrict__ q,
                                                   const uint8_t *__restrict__ k,
                                                   const float *__restrict__ q_scale,
                                                   const float *__restrict__ k_scale,
                                                   float *__restrict__ q_pool,
                                                   float *__restrict__ k_pool, int hq, int hkv,
                                                   int seq, int nb, int nslab, VarlenArgs vl) {
  constexpr int ES = Storage<DT>::bytes;
  constexpr int VEC = 16 / ES;     // elements per 16-byte chunk
  constexpr int CH = D / VEC;      // chunks per row (4..32)
  constexpr int RPL = 64 / CH;     // rows covered by one wave-wide load
  constexpr int NLD = BLK / RPL;   // loads per lane for a whole slab
  static_assert(CH * RPL == 64 && NLD * RPL == BLK, "tiling");
  const int lane = threadIdx.x & 63;
  const int sl = blockIdx.x * 4 + (threadIdx.x >> 6);  // one slab per wavefront
  if (sl >= nslab) return;
  const int hh = sl / nb, I = sl - hh * nb;
  const bool isq = hh < hq;
  const int h = isq ? hh : hh - hq;
  int rows;
  const uint8_t *base;
  if constexpr (VL) {
    const int sq = varlen_seq_of(vl.cu_blocks, vl.nseq, I);
    const int Il = I - vl.cu_blocks[sq], tok0 = vl.cu_seqlens[sq];
    rows = min(BLK, vl.cu_seqlens[sq + 1] - tok0 - Il * BLK);
    base = isq ? q + ((size_t)h * seq + tok0 + Il * BLK) * D * ES
               : k + ((size_t)vl.page_table[(size_t)sq * vl.max_pages + Il] * hkv + h) * BLK * D * ES;
  } else {
    const int t0 = I * BLK;
    rows = min(BLK, seq - t0);
    base = (isq ? q : k) + ((size_t)h * seq + t0) * D * ES;
  }
  const int c = lane % CH, r0 = lane / CH;

  float acc[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) acc[e] = 0.f;
  constexpr int BATCH = NLD < 16 ? NLD : 16;
#pragma unroll
  for (int b0 = 0; b0 < NLD; b0 += BATCH) {
    u32x4v w[BATCH];
#pragma unroll
    for (int it = 0; it < BATCH; ++it) {
      const int r = r0 + (b0 + it) * RPL;
      const u32x4v *src = (const u32x4v *)(base + ((size_t)r * D + c * VEC) * ES);
      w[it] = r < rows ? __builtin_nontemporal_load(src) : u32x4v{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < BATCH; ++it) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t wd = w[it][j];
        if constexpr (DT == kF32) {
          acc[j] += __uint_as_float(wd);
        } else if constexpr (DT == kBF16) {
          acc[2 * j] += bf16_bits_to_f32(wd & 0xFFFFu);
          acc[2 * j + 1] += bf16_bits_to_f32(wd >> 16);
        } else {
          const f32x2 lo = e4m3x2_to_f32(wd, false), hi = e4m3x2_to_f32(wd, true);
          acc[4 * j] += lo.x;
          acc[4 * j + 1] += lo.y;
          acc[4 * j + 2] += hi.x;
          acc[4 * j + 3] += hi.y;
        }
      }
    }
  }
  // lanes c, c + CH, ... hold partial sums of the same columns
#pragma unroll
  for (int o = CH; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], o, 64);
  if (lane < CH) {
    float scale = 1.f;
    if constexpr (DT == kFP8) scale = isq ? q_scale[h] : k_scale[h];
    const float inv = scale / (float)rows;
    float *out = (isq ? q_pool : k_pool) + ((size_t)h * nb + I) * D + c * VEC;
#pragma unroll
    for (int e = 0; e < VEC; e += 4)
      *(float4 *)(out + e) =
          make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
  }
}

template <int DT, int D, int BLK, bool VL>
static hipError_t launch_pool_t(const Shape &s, const void *q, const void *k, const float *qs,
                                const float *ks, float *qp, float *kp, const VarlenArgs &vl,
                                hipStream_t st) {
  const int nslab = (s.hq + s.hkv) * s.nb;
  hipLaunchKernelGGL((pool_kernel<DT, D, BLK, VL>), dim3((nslab + 3) / 4), dim3(256), 0, st,
                     (const uint8_t *)q, (const uint8_t *)k, qs, ks, qp, kp, s.hq, s.hkv, s.seq,
                     s.nb, nslab, vl);
  return hipGetLastError();
}

template <int DT, bool VL>
static hipError_t launch_pool_dt(const Shape &s, const void *q, const void *k, const float *qs,
                                 const float *ks, float *qp, float *kp, const VarlenArgs &vl,
                                 hipStream_t st) {
  if (s.d == 64 && s.block == 64)
    return launch_pool_t<DT, 64, 64, VL>(s, q, k, qs, ks, qp, kp, vl, st);
  if (s.d == 64 && s.block == 128)
    return launch_pool_t<DT, 64, 128, VL>(s, q, k, qs, ks, qp, kp, vl, st);
  if (s.d == 128 && s.block == 64)
    return launch_pool_t<DT, 128, 64, VL>(s, q, k, qs, ks, qp, kp, vl, st);
  return launch_pool_t<DT, 128, 128, VL>(s, q, k, qs, ks, qp, kp, vl, st);
}

template <bool VL>
static hipError_t launch_pool_any(const Shape &s, const void *q, const void *k, const float *qs,
                                  const float *ks, float *qp, float *kp, const VarlenArgs &vl,
                                  hipStream_t st) {
  if (s.dtype == kF32) return launch_pool_dt<kF32, VL>(s, q, k, qs, ks, qp, kp, vl, st);
  if (s.dtype == kBF16) return launch_pool_dt<kBF16, VL>(s, q, k, qs, ks, qp, kp, vl, st);
  return launch_pool_dt<kFP8, VL>(s, q, k, qs, ks, qp, kp, vl, st);
}

hipError_t launch_pool(const Shape &s, const void *q, const void *k, const float *qs,
                       const float *ks, float *qp, float *kp, hipStream_t st) {
  return launch_pool_any<false>(s, q, k, qs, ks, qp, kp, VarlenArgs{}, st);
}

hipError_t launch_pool_varlen(const Shape &s, const VarlenArgs &vl, const void *q,
                              const void *k_cache, const float *qs, const float *ks, float *qp,
                              float *kp, hipStream_t st) {
  return launch_pool_any<true>(s, q, k_cache, qs, ks, qp, kp, vl, st);
}

}  // namespace bsp
