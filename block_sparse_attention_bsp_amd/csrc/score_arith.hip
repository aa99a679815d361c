// Stage 1, per-query block approximation (FlashPrefill summary page, section 3
// "Instantaneous Pattern Discovery": pooled key blocks stand in for their
// tokens and a block's significance is averaged over its queries; "Block
// Approximation for Kernel Optimization": one fused pass that never forms
// the L x (L/B) matrix of per-token scores).  For query block I of head h:
//   P[h][I][J] = mean over the valid tokens i of block I of
//                softmax over J' <= I of (c * q_i . Kbar[g(h)][J'])  at J,
// 0 for J > I.  Kbar comes from the pool kernel.
//
// gfx950 design
//   * One workgroup per (q head, query block I), heaviest blocks first; each
//     wavefront owns 32 of the block's queries, whose Q fragments stay in
//     registers.  Key blocks are taken in tiles of 32.
//   * Exactness: Kbar is fp32, the MFMA operands bf16.  Each Kbar tile is
//     split in LDS into three bf16 planes hi + mid + lo that represent it to
//     within 2^-24 relatively; bf16 queries, and e4m3 codes widened to bf16,
//     are exact, so the three products are exact and only the fp32
//     accumulation rounds - the accuracy of an fp32 dot product.  fp32 inputs
//     use v_mfma_f32_32x32x2_f32 on the fp32 tile instead.
//   * Pass 1 computes S^T = Kbar Q^T: each lane holds one query and 16 key
//     blocks of a tile, so every query's softmax max and sum are in-lane plus
//     one exchange with the lane 32 away.  Pass 2 recomputes the tile as
//     S = Q Kbar^T - the same fragments with the operands swapped - so each
//     lane holds one key block and 16 queries: the average over queries is
//     in-lane, then one exchange, then the block's wavefronts meet in LDS.
#include "device.h"
#include "internal.h"

namespace bsp {

template <int DT, int D, int BLK>
struct ArithCfg {
  static constexpr int NW = BLK / 32;  // wavefronts: 32 queries each
  static constexpr int NT = NW * 64;
  static constexpr bool F32 = DT == kF32;
  static constexpr int KS = D / 16;    // bf16 k-steps (16 dimensions each)
  static constexpr int RSB = D * 2 + 16;  // padded bf16 plane row (bytes)
  static constexpr int RSF = D + 4;       // padded fp32 row (floats)
  static constexpr int PLANE = 32 * RSB;  // one bf16 plane (bytes)
  static constexpr int LDSB = F32 ? 32 * RSF * 4 : 3 * PLANE;
};

template <int DT, int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void score_arith_kernel(
    const uint8_t *__restrict__ q, const float *__restrict__ k_pool, float *__restrict__ P,
    const float *__restrict__ q_scale, int hq, int hkv, int seq, int nb, float c2) {
  using C = ArithCfg<DT, D, BLK>;
  constexpr int NW = C::NW, NT = C::NT, KS = C::KS, RSB = C::RSB, RSF = C::RSF;
  __shared__ __attribute__((aligned(16))) uint8_t ktb[2][C::LDSB];  // double-buffered tile
  __shared__ float qoff[BLK];         // per query: max + log2(sum) of pass 1
  __shared__ float part[2][NW][32];   // per wavefront: sum of p over its queries

  const int bid = blockIdx.x;
  const int I = nb - 1 - bid / hq, h = bid % hq;
  const int g = h / (hq / hkv);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int qi = I * BLK + w * 32 + l32;  // this lane's query in pass 1
  const int nvalid = min(BLK, seq - I * BLK);
  const int ntile = I / 32 + 1;
  const float scl = c2 * (DT == kFP8 ? q_scale[h] : 1.f);
  float *prow = P + ((size_t)h * nb + I) * nb;

  // ---- Q fragments (query qi, lane half selects the dimension group)
  bf16x8 qf[C::F32 ? 1 : KS];
  float qv[C::F32 ? D / 2 : 1];
  {
    const size_t row = (size_t)h * seq + min(qi, seq - 1);
    const bool ok = qi < seq;
    if constexpr (C::F32) {
      // step ks, lane half hh <-> dimension ks + (D/2)*hh
      const float *src = (const float *)q + row * D + (D / 2) * half;
#pragma unroll
      for (int i = 0; i < D / 2; i += 4) {
        const float4 t = *(const float4 *)(src + i);
        qv[i] = ok ? t.x : 0.f;
        qv[i + 1] = ok ? t.y : 0.f;
        qv[i + 2] = ok ? t.z : 0.f;
        qv[i + 3] = ok ? t.w : 0.f;
      }
    } else {
      // step ks: dimensions ks*16 + half*8 .. + 8
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (DT == kBF16) {
          uint4 a = *(const uint4 *)((const uint16_t *)q + row * D + ks * 16 + half * 8);
          if (!ok) a = make_uint4(0, 0, 0, 0);
          __builtin_memcpy(&qf[ks], &a, 16);
        } else {
          uint2 a = *(const uint2 *)(q + row * D + ks * 16 + half * 8);
          if (!ok) a = make_uint2(0, 0);
          const uint4 b = make_uint4(e4m3x2_to_bf16x2(a.x, false), e4m3x2_to_bf16x2(a.x, true),
                                     e4m3x2_to_bf16x2(a.y, false), e4m3x2_to_bf16x2(a.y, true));
          __builtin_memcpy(&qf[ks], &b, 16);
        }
      }
    }
  }

  // ---- Kbar tile jt -> LDS (fp32, or three bf16 planes), whole workgroup:
  //      the global loads of tile jt + 1 are issued before the MFMAs of tile
  //      jt, the split and the LDS stores follow them
  constexpr int FPT = 32 * D / 4 / NT;  // float4 per thread per tile
  static_assert(FPT * NT * 4 == 32 * D, "tile staging");
  float4 xr[FPT];
  auto stage_load = [&](int jt) {
    const float *src = k_pool + ((size_t)g * nb + jt * 32) * D;
    const int n = min(32, nb - jt * 32);
#pragma unroll
    for (int u = 0; u < FPT; ++u) {
      const int f = threadIdx.x + u * NT;
      xr[u] = f / (D / 4) < n ? *(const float4 *)(src + 4 * f) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto stage_store = [&](uint8_t *kt) {
#pragma unroll
    for (int u = 0; u < FPT; ++u) {
      const int f = threadIdx.x + u * NT;
      const int r = f / (D / 4), c4 = (f % (D / 4)) * 4;
      const float4 x = xr[u];
      if constexpr (C::F32) {
        *(float4 *)((float *)kt + r * RSF + c4) = x;
      } else {
        // hi + mid + lo, each the bf16 rounding (to nearest even) of what the
        // planes before it leave; every difference is exact in fp32 (split3)
        const float xs[4] = {x.x, x.y, x.z, x.w};
        bf16x4 hv, mv, lv;
        split3(xs, hv, mv, lv);
        uint8_t *base = kt + r * RSB + c4 * 2;
        __builtin_memcpy(base, &hv, 8);
        __builtin_memcpy(base + C::PLANE, &mv, 8);
        __builtin_memcpy(base + 2 * C::PLANE, &lv, 8);
      }
    }
  };

  // One 32 x 32 tile: kfirst ? S^T = Kbar Q^T : S = Q Kbar^T.  The Kbar
  // fragment of lane l is row l % 32 of the tile, the same for both orders.
  auto tile = [&](const uint8_t *kt, bool kfirst) -> f32x16 {
    f32x16 acc = f32x16{};
    if constexpr (C::F32) {
      const float *arow = (const float *)kt + l32 * RSF + (D / 2) * half;
#pragma unroll
      for (int i = 0; i < D / 2; i += 4) {
        const float4 a = *(const float4 *)(arow + i);
        const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc = kfirst ? __builtin_amdgcn_mfma_f32_32x32x2f32(av[e], qv[i + e], acc, 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_32x32x2f32(qv[i + e], av[e], acc, 0, 0, 0);
      }
    } else {
      const uint8_t *arow = kt + l32 * RSB + half * 16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int pl = 2; pl >= 0; --pl) {  // small planes first
          bf16x8 a;
          __builtin_memcpy(&a, arow + pl * C::PLANE + ks * 32, 16);
          acc = kfirst ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], acc, 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], a, acc, 0, 0, 0);
        }
      }
    }
    return acc;
  };

  // ---- pass 1: per query, max and sum of exp2 over the causal key blocks
  float m = -INFINITY, l = 0.f;
  stage_load(0);
  stage_store(ktb[0]);
  __syncthreads();
  for (int jt = 0; jt < ntile; ++jt) {
    if (jt + 1 < ntile) stage_load(jt + 1);
    const f32x16 acc = tile(ktb[jt & 1], true);
    float s[16], tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int J = jt * 32 + (r / 4) * 8 + half * 4 + (r % 4);
      s[r] = J <= I ? acc[r] * scl : -INFINITY;
      tmax = fmaxf(tmax, s[r]);
    }
    const float mn = fmaxf(m, tmax);
    if (mn != -INFINITY) {
      float a = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) a += __builtin_amdgcn_exp2f(s[r] - mn);
      l = l * __builtin_amdgcn_exp2f(m - mn) + a;
      m = mn;
    }
    if (jt + 1 < ntile) stage_store(ktb[(jt + 1) & 1]);
    __syncthreads();
  }
  {
    const float mo = __shfl_xor(m, 32, 64), lo = __shfl_xor(l, 32, 64);
    const float mn = fmaxf(m, mo);
    l = (m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f(m - mn)) +
        (mo == -INFINITY ? 0.f : lo * __builtin_amdgcn_exp2f(mo - mn));
    m = mn;
  }
  // a query past the end of the sequence gets +inf: its p is 0 in pass 2
  if (half == 0) qoff[w * 32 + l32] = qi < seq ? m + log2f(l) : INFINITY;
  stage_load(0);
  stage_store(ktb[0]);
  __syncthreads();
  // pass-2 rows of this lane: queries w*32 + (r/4)*8 + half*4 + r%4
  float off[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) off[r] = qoff[w * 32 + (r / 4) * 8 + half * 4 + (r % 4)];

  // ---- pass 2: p = exp2(s - off) summed over the block's queries; wave 0
  //      adds the wavefronts' sums of tile jt and writes them while tile
  //      jt + 1 is computed
  const float invn = 1.f / (float)nvalid;
  auto emit = [&](int jt) {
    const int J = jt * 32 + l32;
    if (w == 0 && half == 0 && J < nb) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) t += part[jt & 1][i][l32];
      prow[J] = J <= I ? t * invn : 0.f;
    }
  };
  for (int jt = 0; jt < ntile; ++jt) {
    if (jt + 1 < ntile) stage_load(jt + 1);
    const f32x16 acc = tile(ktb[jt & 1], false);
    const int J = jt * 32 + l32;
    float a = 0.f;
    if (J <= I) {
#pragma unroll
      for (int r = 0; r < 16; ++r) a += __builtin_amdgcn_exp2f(acc[r] * scl - off[r]);
    }
    a += __shfl_xor(a, 32, 64);
    if (half == 0) part[jt & 1][w][l32] = a;
    if (jt > 0) emit(jt - 1);
    if (jt + 1 < ntile) stage_store(ktb[(jt + 1) & 1]);
    __syncthreads();
  }
  emit(ntile - 1);
  // zeros past the causal tiles
  for (int J = ntile * 32 + threadIdx.x; J < nb; J += NT) prow[J] = 0.f;
}

template <int DT, int D, int BLK>
static hipError_t launch_arith_t(const Shape &s, float c, const void *q, const float *kp,
                                 float *S, const float *qs, hipStream_t st) {
  hipLaunchKernelGGL((score_arith_kernel<DT, D, BLK>), dim3((unsigned)(s.hq * s.nb)),
                     dim3(BLK * 2), 0, st, (const uint8_t *)q, kp, S, qs, s.hq, s.hkv, s.seq,
                     s.nb, c * kLog2e);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_arith_dt(const Shape &s, float c, const void *q, const float *kp,
                                  float *S, const float *qs, hipStream_t st) {
  if (s.d == 64 && s.block == 64) return launch_arith_t<DT, 64, 64>(s, c, q, kp, S, qs, st);
  if (s.d == 64 && s.block == 128) return launch_arith_t<DT, 64, 128>(s, c, q, kp, S, qs, st);
  if (s.d == 128 && s.block == 64) return launch_arith_t<DT, 128, 64>(s, c, q, kp, S, qs, st);
  return launch_arith_t<DT, 128, 128>(s, c, q, kp, S, qs, st);
}

hipError_t launch_score_arith(const Shape &s, float c, const void *q, const float *k_pool,
                              float *score, const float *q_scale, hipStream_t st) {
  if (s.dtype == kF32) return launch_arith_dt<kF32>(s, c, q, k_pool, score, q_scale, st);
  if (s.dtype == kBF16) return launch_arith_dt<kBF16>(s, c, q, k_pool, score, q_scale, st);
  return launch_arith_dt<kFP8>(s, c, q, k_pool, score, q_scale, st);
}

}  // namespace bsp
