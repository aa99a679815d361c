// Stage 1b: block scores and their row normalisation (FlashPrefill summary
// page, section 3 "Block Approximation for Kernel Optimization": scores live
// on the (L/B) x (L/B) block grid, never on an L x (L/B) intermediate;
// Appendix B: query tiles against causally valid pooled key blocks, then a
// global normalisation).
//
// Two passes over the causal block grid of a group of 32 query blocks:
//   pass 1  S^T tiles = Kbar Qbar^T (32 key blocks x 32 query blocks) on
//           v_mfma_f32_32x32x2_f32 - fp32 products and sums, so the
//           threshold downstream sees full-precision scores - reduced to the
//           running row max and sum of exp;
//   pass 2  after the row statistics meet, P = exp(S - max) / sum on the
//           causal part, zeros above it.
// Each lane owns one query block (a column of S^T), so the row reductions are
// in-lane plus one exchange with the lane 32 away; the wavefronts of a
// workgroup split the key-block tiles of the same 32 query blocks and merge
// their row statistics through LDS.  The grid launches the heaviest row
// groups of every head first.
//
// With a key-block radius r (rescue branch, thelatestinai page, RBS-Attention
// abstract) the same kernels compute c (Qbar_I . Kbar_J + |Qbar_I| r_J), an
// upper bound on the block's best per-key logit, and its row softmax.
//
// score_kernel_reg (rows of at most 1024 blocks): eight wavefronts with at
// most four tiles each keep their raw scores in registers, so P is written
// once, normalised, through an LDS transpose that makes every store cover
// whole 128-byte row runs.  score_kernel (longer rows): four wavefronts write
// the raw scores transposed the same way, then the workgroup sweeps its rows
// row-major with 16-byte accesses and normalises them in place.
#include "device.h"
#include "internal.h"

namespace bsp {

template <int D, bool RESC>
__global__ __launch_bounds__(256) void score_kernel(const float *__restrict__ q_pool,
                                                    const float *__restrict__ k_pool,
                                                    const float *__restrict__ k_radius,
                                                    float *__restrict__ P, int hq, int hkv, int nb,
                                                    float c2) {
  constexpr int KS = D / 2;  // k-steps; step ks, lane half h <-> dimension ks + KS*h
  __shared__ float red_m[4][32], red_l[4][32], row_m[32], row_inv[32];
  __shared__ __attribute__((aligned(16))) float kt_s[4 * 32 * (D + 4)];
  const int G = (nb + 31) / 32;
  const int grp = G - 1 - (int)blockIdx.y;
  const int h = blockIdx.x;
  const int g = h / (hq / hkv);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int I0 = grp * 32;
  const int rows = min(32, nb - I0);
  const int Il = I0 + l32;  // this lane's query block
  const bool row_ok = l32 < rows;
  const int ntc = (I0 + rows - 1) / 32 + 1;  // key-block tiles touching the causal part
  const bool vec = (nb & 3) == 0;             // rows of P are 16-byte aligned
  float *pgrp = P + ((size_t)h * nb + I0) * nb;

  // B operand (Qbar^T): lane holds Qbar[Il][ks + KS*half]
  float qb[KS];
  {
    const float *src = q_pool + ((size_t)h * nb + min(Il, nb - 1)) * D + KS * half;
#pragma unroll
    for (int i = 0; i < KS; i += 4) {
      const float4 t = *(const float4 *)(src + i);
      qb[i] = row_ok ? t.x : 0.f;
      qb[i + 1] = row_ok ? t.y : 0.f;
      qb[i + 2] = row_ok ? t.z : 0.f;
      qb[i + 3] = row_ok ? t.w : 0.f;
    }
  }
  // rescue branch: |Qbar_I| (the lane holds half of the dimensions)
  float qn = 0.f;
  if constexpr (RESC) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < KS; ++i) ss = fmaf(qb[i], qb[i], ss);
    qn = sqrtf(ss + __shfl_xor(ss, 32, 64));
  }
  const float *rad = RESC ? k_radius + (size_t)g * nb : nullptr;

  // S^T tile jt: element r of the lane is key block J0 + (r/4)*8 + half*4 + r%4.
  // The 32 Kbar rows of a tile are one contiguous block: each wave loads it
  // with coalesced 16-byte loads one tile ahead, stores it to its own padded
  // LDS slice (row stride D + 4 floats: conflict-free column reads) and reads
  // the A operand (row l32, dimensions ks + KS*half) back from there.  The
  // same slice then carries the tile's transpose for row-contiguous stores.
  constexpr int TF4 = 32 * D / 4 / 64;  // float4 per lane per tile
  constexpr int RS = D + 4;             // padded LDS row stride (floats)
  constexpr int TS = 33;                // transpose row stride (floats)
  float *kt_lds = kt_s + w * 32 * RS;
  typedef float4 stage_t[TF4];
  auto fetch = [&](int jt, stage_t &st) {
    const float *src = k_pool + ((size_t)g * nb + jt * 32) * D;
    const int n = min(32, nb - jt * 32);
#pragma unroll
    for (int i = 0; i < TF4; ++i) {
      const int f = lane + 64 * i;  // float4 index inside the tile
      st[i] = f / (D / 4) < n ? *(const float4 *)(src + 4 * f) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto stage = [&](const stage_t &st) {
#pragma unroll
    for (int i = 0; i < TF4; ++i) {
      const int f = lane + 64 * i;
      *(float4 *)(kt_lds + (f / (D / 4)) * RS + (f % (D / 4)) * 4) = st[i];
    }
  };
  auto mma = [&]() -> f32x16 {
    const float *arow = kt_lds + l32 * RS + KS * half;
    float4 a[KS / 4];
#pragma unroll
    for (int i = 0; i < KS / 4; ++i) a[i] = *(const float4 *)(arow + 4 * i);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int i = 0; i < KS / 4; ++i) {
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i].x, qb[4 * i], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i].y, qb[4 * i + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i].z, qb[4 * i + 2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i].w, qb[4 * i + 3], acc, 0, 0, 0);
    }
    return acc;
  };
  // Raw scores of tile jt -> P through the wave's LDS slice: written by
  // (row, key) = (l32, r), read back so that 8 lanes cover one row's 32 keys.
  auto put_tile = [&](int jt, const float (&s)[16]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) kt_lds[l32 * TS + (r / 4) * 8 + half * 4 + (r % 4)] = s[r];
    const int c4 = (lane & 7) * 4;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int rr = it * 8 + (lane >> 3);
      const float *t = kt_lds + rr * TS + c4;
      const int J = jt * 32 + c4;
      float *dst = pgrp + (size_t)rr * nb + J;
      if (rr < rows) {
        if (vec && J + 3 < nb) {
          *(float4 *)dst = make_float4(t[0], t[1], t[2], t[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (J + e < nb) dst[e] = t[e];
        }
      }
    }
  };

  // ---- pass 1: raw log2-domain scores to P, row max and sum of exp2
  float m = -INFINITY, l = 0.f;
  stage_t nxt;
  if (w < ntc) fetch(w, nxt);
  for (int jt = w; jt < ntc; jt += 4) {
    stage(nxt);
    if (jt + 4 < ntc) fetch(jt + 4, nxt);
    const f32x16 acc = mma();
    float s[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int J = jt * 32 + (r / 4) * 8 + half * 4 + (r % 4);
      const float add = RESC && J < nb ? qn * rad[J] : 0.f;
      s[r] = (J <= Il && J < nb) ? (acc[r] + add) * c2 : -INFINITY;
      tmax = fmaxf(tmax, s[r]);
    }
    put_tile(jt, s);
    const float mn = fmaxf(m, tmax);
    if (mn != -INFINITY) {
      float acc_l = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_l += exp2f(s[r] - mn);
      l = l * exp2f(m - mn) + acc_l;
      m = mn;
    }
  }
  // merge the two lane halves, then the four wavefronts
  {
    const float mo = __shfl_xor(m, 32, 64), lo = __shfl_xor(l, 32, 64);
    const float mn = fmaxf(m, mo);
    if (mn != -INFINITY) {
      l = (m == -INFINITY ? 0.f : l * exp2f(m - mn)) + (mo == -INFINITY ? 0.f : lo * exp2f(mo - mn));
      m = mn;
    }
  }
  if (half == 0) {
    red_m[w][l32] = m;
    red_l[w][l32] = l;
  }
  __syncthreads();
  if (w == 0 && half == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) M = fmaxf(M, red_m[i][l32]);
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (red_m[i][l32] != -INFINITY) L += red_l[i][l32] * exp2f(red_m[i][l32] - M);
    row_m[l32] = M;
    row_inv[l32] = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();

  // ---- pass 2: the group's rows of P, row-major and coalesced: causal
  // entries become exp2(s - M) / L from the raw scores of pass 1, the rest 0.
  const int jend = ntc * 32;  // raw scores exist for J < jend (-inf above the diagonal)
  if (vec) {
    // 8 rows per batch: all loads are issued before the first store
    for (int J = threadIdx.x * 4; J < nb; J += 1024) {
      for (int r0 = 0; r0 < rows; r0 += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int rr = r0 + u;
          v[u] = (rr < rows && J < jend) ? *(const float4 *)(pgrp + (size_t)rr * nb + J)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int rr = r0 + u;
          if (rr < rows) {
            if (J < jend) {
              const float M = row_m[rr], inv = row_inv[rr];
              v[u].x = exp2f(v[u].x - M) * inv;
              v[u].y = exp2f(v[u].y - M) * inv;
              v[u].z = exp2f(v[u].z - M) * inv;
              v[u].w = exp2f(v[u].w - M) * inv;
            }
            *(float4 *)(pgrp + (size_t)rr * nb + J) = v[u];
          }
        }
      }
    }
  } else {
    for (int rr = 0; rr < rows; ++rr) {
      const float M = row_m[rr], inv = row_inv[rr];
      float *prow = pgrp + (size_t)rr * nb;
      for (int J = threadIdx.x; J < nb; J += 256)
        prow[J] = J < jend ? exp2f(prow[J] - M) * inv : 0.f;
    }
  }
}

// Rows of at most 1024 key blocks: eight wavefronts split the key-block tiles
// of the group (at most four each) and keep their raw scores in registers,
// so P is written once, already normalised, and never read back.
template <int D, bool RESC>
__global__ __launch_bounds__(512) void score_kernel_reg(const float *__restrict__ q_pool,
                                                        const float *__restrict__ k_pool,
                                                        const float *__restrict__ k_radius,
                                                        float *__restrict__ P, int hq, int hkv,
                                                        int nb, float c2) {
  constexpr int KS = D / 2;   // k-steps; step ks, lane half h <-> dimension ks + KS*h
  constexpr int NWV = 8;      // wavefronts
  constexpr int MAXT = 4;     // tiles per wavefront
  __shared__ float red_m[NWV][32], red_l[NWV][32], row_m[32], row_inv[32];
  __shared__ __attribute__((aligned(16))) float kt_s[NWV * 32 * (D + 4)];
  const int G = (nb + 31) / 32;
  const int grp = G - 1 - (int)blockIdx.y;
  const int h = blockIdx.x;
  const int g = h / (hq / hkv);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int I0 = grp * 32;
  const int rows = min(32, nb - I0);
  const int Il = I0 + l32;  // this lane's query block
  const bool row_ok = l32 < rows;
  const int ntc = (I0 + rows - 1) / 32 + 1;  // key-block tiles touching the causal part
  const bool vec = (nb & 3) == 0;             // rows of P are 16-byte aligned
  float *pgrp = P + ((size_t)h * nb + I0) * nb;

  float qb[KS];
  {
    const float *src = q_pool + ((size_t)h * nb + min(Il, nb - 1)) * D + KS * half;
#pragma unroll
    for (int i = 0; i < KS; i += 4) {
      const float4 t = *(const float4 *)(src + i);
      qb[i] = row_ok ? t.x : 0.f;
      qb[i + 1] = row_ok ? t.y : 0.f;
      qb[i + 2] = row_ok ? t.z : 0.f;
      qb[i + 3] = row_ok ? t.w : 0.f;
    }
  }
  // rescue branch: |Qbar_I| (the lane holds half of the dimensions)
  float qn = 0.f;
  if constexpr (RESC) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < KS; ++i) ss = fmaf(qb[i], qb[i], ss);
    qn = sqrtf(ss + __shfl_xor(ss, 32, 64));
  }
  const float *rad = RESC ? k_radius + (size_t)g * nb : nullptr;

  constexpr int TF4 = 32 * D / 4 / 64;  // float4 per lane per tile
  constexpr int RS = D + 4;             // padded LDS row stride (floats)
  constexpr int TS = 33;                // transpose row stride (floats)
  float *kt_lds = kt_s + w * 32 * RS;
  // the tile goes global -> registers -> LDS in two halves (no prefetch:
  // the SIMD's other wavefront covers the load latency)
  auto load_stage = [&](int jt) {
    const float *src = k_pool + ((size_t)g * nb + jt * 32) * D;
    const int n = min(32, nb - jt * 32);
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float4 st[TF4 / 2];
#pragma unroll
      for (int i = 0; i < TF4 / 2; ++i) {
        const int f = lane + 64 * (hb * (TF4 / 2) + i);
        st[i] = f / (D / 4) < n ? *(const float4 *)(src + 4 * f) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int i = 0; i < TF4 / 2; ++i) {
        const int f = lane + 64 * (hb * (TF4 / 2) + i);
        *(float4 *)(kt_lds + (f / (D / 4)) * RS + (f % (D / 4)) * 4) = st[i];
      }
    }
  };
  auto mma = [&]() -> f32x16 {
    const float *arow = kt_lds + l32 * RS + KS * half;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int i = 0; i < KS / 4; ++i) {
      const float4 a = *(const float4 *)(arow + 4 * i);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, qb[4 * i], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, qb[4 * i + 1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, qb[4 * i + 2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, qb[4 * i + 3], acc, 0, 0, 0);
    }
    return acc;
  };

  // ---- pass 1: raw log2-domain scores held in registers, row max and sum
  float held[MAXT][16];
  float m = -INFINITY, l = 0.f;
#pragma unroll
  for (int t = 0; t < MAXT; ++t) {
    const int jt = w + t * NWV;
    if (jt < ntc) {
      load_stage(jt);
      const f32x16 acc = mma();
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int J = jt * 32 + (r / 4) * 8 + half * 4 + (r % 4);
        const float add = RESC && J < nb ? qn * rad[J] : 0.f;
        held[t][r] = (J <= Il && J < nb) ? (acc[r] + add) * c2 : -INFINITY;
        tmax = fmaxf(tmax, held[t][r]);
      }
      const float mn = fmaxf(m, tmax);
      if (mn != -INFINITY) {
        float acc_l = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc_l += exp2f(held[t][r] - mn);
        l = l * exp2f(m - mn) + acc_l;
        m = mn;
      }
    }
  }
  {
    const float mo = __shfl_xor(m, 32, 64), lo = __shfl_xor(l, 32, 64);
    const float mn = fmaxf(m, mo);
    if (mn != -INFINITY) {
      l = (m == -INFINITY ? 0.f : l * exp2f(m - mn)) + (mo == -INFINITY ? 0.f : lo * exp2f(mo - mn));
      m = mn;
    }
  }
  if (half == 0) {
    red_m[w][l32] = m;
    red_l[w][l32] = l;
  }
  __syncthreads();
  if (w == 0 && half == 0) {
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < NWV; ++i) M = fmaxf(M, red_m[i][l32]);
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < NWV; ++i)
      if (red_m[i][l32] != -INFINITY) L += red_l[i][l32] * exp2f(red_m[i][l32] - M);
    row_m[l32] = M;
    row_inv[l32] = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();

  // ---- pass 2: normalise the held tiles and write them through the wave's
  // LDS slice, so that 8 lanes cover one row's 32 keys of a tile
  {
    const float M = row_m[l32], inv = row_inv[l32];
    const int c4 = (lane & 7) * 4;
#pragma unroll
    for (int t = 0; t < MAXT; ++t) {
      const int jt = w + t * NWV;
      if (jt < ntc) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          kt_lds[l32 * TS + (r / 4) * 8 + half * 4 + (r % 4)] = exp2f(held[t][r] - M) * inv;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int rr = it * 8 + (lane >> 3);
          const float *tp = kt_lds + rr * TS + c4;
          const int J = jt * 32 + c4;
          float *dst = pgrp + (size_t)rr * nb + J;
          if (rr < rows) {
            if (vec && J + 3 < nb) {
              *(float4 *)dst = make_float4(tp[0], tp[1], tp[2], tp[3]);
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (J + e < nb) dst[e] = tp[e];
            }
          }
        }
      }
    }
  }
  // zeros above the causal tiles, all threads, row-major
  const int jend = ntc * 32;
  if (jend < nb) {
    if (vec) {
      const int n4 = (nb - jend) / 4;
      for (int e = threadIdx.x; e < rows * n4; e += 512) {
        const int rr = e / n4, J = jend + (e - rr * n4) * 4;
        *(float4 *)(pgrp + (size_t)rr * nb + J) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    } else {
      const int n1 = nb - jend;
      for (int e = threadIdx.x; e < rows * n1; e += 512) {
        const int rr = e / n1;
        pgrp[(size_t)rr * nb + jend + (e - rr * n1)] = 0.f;
      }
    }
  }
}

template <int D, bool RESC>
static hipError_t launch_score_t(const Shape &s, float c, const float *qp, const float *kp,
                                 const float *kr, float *S, hipStream_t st) {
  // heaviest row groups of every head first
  dim3 grid(s.hq, (s.nb + 31) / 32);
  if (s.nb <= 1024)
    hipLaunchKernelGGL((score_kernel_reg<D, RESC>), grid, dim3(512), 0, st, qp, kp, kr, S, s.hq,
                       s.hkv, s.nb, c * kLog2e);
  else
    hipLaunchKernelGGL((score_kernel<D, RESC>), grid, dim3(256), 0, st, qp, kp, kr, S, s.hq,
                       s.hkv, s.nb, c * kLog2e);
  return hipGetLastError();
}

// Packed variable-length batch: one wavefront per (q head, batch block gb)
// row, lane j taking the key blocks j, j + 64, ... of the row's own
// sequence.  Each score is an fp32 dot product of the (wave-uniform, hence
// scalar-loaded) Qbar row with the lane's Kbar row; a sequence has few
// blocks, so these rows are too short to fill matrix-core tiles.  Pass 1
// writes the log2-domain scores and keeps a per-lane running max and sum;
// after the wave combines them, pass 2 rewrites the row normalised.  Row gb
// has stride ld; its entries J < nb_s are written (0 for J > I).
template <int D>
__global__ __launch_bounds__(256) void score_vl_kernel(const float *__restrict__ q_pool,
                                                       const float *__restrict__ k_pool,
                                                       float *__restrict__ P, int hq, int hkv,
                                                       int nb, int ld, VarlenArgs vl, float c2) {
  const int lane = threadIdx.x & 63;
  const int row = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (row >= hq * nb) return;
  const int h = row / nb, gb = row - h * nb;
  const int g = h / (hq / hkv);
  const int sq = varlen_seq_of(vl.cu_blocks, vl.nseq, gb);
  // a row never writes past its stride, whatever the offsets say
  const int cb0 = vl.cu_blocks[sq], ncol = min(vl.cu_blocks[sq + 1] - cb0, ld);
  const int I = min(gb - cb0, ncol - 1);
  const float *qrow = q_pool + (size_t)row * D;
  const float *kbase = k_pool + ((size_t)g * nb + cb0) * D;
  float *prow = P + (size_t)row * ld;

  float m = -INFINITY, l = 0.f;
  for (int J = lane; J <= I; J += 64) {
    const float *krow = kbase + (size_t)J * D;
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int i = 0; i < D; i += 8) {
      const float4 k0 = *(const float4 *)(krow + i), k1 = *(const float4 *)(krow + i + 4);
      const float4 q0 = *(const float4 *)(qrow + i), q1 = *(const float4 *)(qrow + i + 4);
      a0 = fmaf(q0.x, k0.x, fmaf(q0.y, k0.y, fmaf(q0.z, k0.z, fmaf(q0.w, k0.w, a0))));
      a1 = fmaf(q1.x, k1.x, fmaf(q1.y, k1.y, fmaf(q1.z, k1.z, fmaf(q1.w, k1.w, a1))));
    }
    const float x = (a0 + a1) * c2;
    prow[J] = x;
    const float mn = fmaxf(m, x);
    l = l * exp2f(m - mn) + exp2f(x - mn);
    m = mn;
  }
  const float M = wave_max(m);
  float L = m == -INFINITY ? 0.f : l * exp2f(m - M);
  L = wave_sum(L);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  for (int J = lane; J < ncol; J += 64) prow[J] = J <= I ? exp2f(prow[J] - M) * inv : 0.f;
}

hipError_t launch_score_varlen(const Shape &s, const VarlenArgs &vl, float c, const float *q_pool,
                               const float *k_pool, float *S, hipStream_t st) {
  const int rows = s.hq * s.nb;
  if (s.d == 64)
    hipLaunchKernelGGL((score_vl_kernel<64>), dim3((rows + 3) / 4), dim3(256), 0, st, q_pool,
                       k_pool, S, s.hq, s.hkv, s.nb, vl.idx_stride, vl, c * kLog2e);
  else
    hipLaunchKernelGGL((score_vl_kernel<128>), dim3((rows + 3) / 4), dim3(256), 0, st, q_pool,
                       k_pool, S, s.hq, s.hkv, s.nb, vl.idx_stride, vl, c * kLog2e);
  return hipGetLastError();
}

hipError_t launch_score(const Shape &s, float c, const float *q_pool, const float *k_pool,
                        const float *k_radius, float *S, hipStream_t st) {
  if (k_radius) {
    if (s.d == 64) return launch_score_t<64, true>(s, c, q_pool, k_pool, k_radius, S, st);
    return launch_score_t<128, true>(s, c, q_pool, k_pool, k_radius, S, st);
  }
  if (s.d == 64) return launch_score_t<64, false>(s, c, q_pool, k_pool, nullptr, S, st);
  return launch_score_t<128, false>(s, c, q_pool, k_pool, nullptr, S, st);
}

}  // namespace bsp
