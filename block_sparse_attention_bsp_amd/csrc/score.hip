// Stage 1b: block scores and their row normalisation (FlashPrefill summary
// page, section 3 "Block Approximation for Kernel Optimization": scores live
// on the (L/B) x (L/B) block grid, never on an L x (L/B) intermediate;
// Appendix B: query tiles against causally valid pooled key blocks, then a
// global normalisation).
//
// One workgroup per group of 32 query blocks of a head, in two passes:
//   pass 1  S^T tiles = Kbar Qbar^T (32 key blocks x 32 query blocks), with
//           fp32-accurate products and sums so that the threshold downstream
//           sees full-precision scores, each computed once: its raw
//           log2-domain scores go to P, its rows into the running max and
//           sum of exp;
//   pass 2  after the row statistics meet, the workgroup rewrites its rows
//           of P in place, P = exp(S - max) / sum on the causal part, zeros
//           above it.
// Each lane owns one query block (a column of S^T), so the row reductions are
// in-lane plus one exchange with the lane 32 away; the wavefronts of a
// workgroup split the key-block tiles of the same 32 query blocks and merge
// their row statistics through LDS.  The grid launches the heaviest row
// groups of every head first.
//
// With a key-block radius r (rescue branch, thelatestinai page, RBS-Attention
// abstract) the same kernel computes c (Qbar_I . Kbar_J + |Qbar_I| r_J), an
// upper bound on the block's best per-key logit, and its row softmax.
#include "device.h"
#include "internal.h"
#include "kept_list.h"

namespace bsp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The dot products run on v_mfma_f32_32x32x16_bf16 over three bf16 planes of
// each operand: hi*hi + hi*mid + mid*hi + hi*lo + lo*hi + mid*mid leaves out
// only terms below 2^-24 of each product, every plane product is exact and
// the sums are fp32, so the scores are as accurate as fp32 products (the
// threshold downstream needs them to well under its 1e-4 band), at 1/2.7 of
// the matrix-core time of v_mfma_f32_32x32x2_f32.  The Qbar planes are made
// once and stay in registers; each Kbar tile is split as it is read.
//
// Kbar tiles reach LDS by direct-to-LDS buffer loads in two halves of the
// dimensions (each a wavefront's private buffer), the next half issued
// before the current one is computed.  Lane (r, kg) = (lane % 32, lane / 32)
// reads row r, dimensions D/2*kg + 8s .. + 8 at MFMA step s; a half holds
// steps [D/32 * hh, D/32 * (hh + 1)) as D/8 chunks of 16 bytes per row, in
// rows padded by one chunk: the odd row stride in 16-byte units puts the 16
// lanes of a ds_read_b128 phase on 16 distinct bank groups, and every read
// is the lane's row base plus an immediate offset.
template <int D>
struct ScoreStage {
  static constexpr int CPR = D / 8;                  // chunks per row of a half
  static constexpr int RS = (CPR + 1) * 16;          // padded row stride (bytes)
  static constexpr int NDMA = (32 * (CPR + 1) + 63) / 64;  // loads per half and wavefront
  static constexpr int HB = NDMA * 1024;             // bytes per half buffer
};

// The MFMA steps of one staged half hh: lane (l32, half) reads row l32 of
// the half buffer, splits it and accumulates the six plane products (the
// small ones into their own accumulator, unless ONE: the rescue variant needs
// those registers).  buf is restrict-qualified so that the compiler knows the
// loads in flight into the other half do not alias it.
template <int D, bool ONE>
__device__ __forceinline__ void score_half(const uint8_t *__restrict__ buf, int hh, int half,
                                           int l32, const bf16x8 (&qh)[D / 16],
                                           const bf16x8 (&qm)[D / 16], const bf16x8 (&ql)[D / 16],
                                           f32x16 &big, f32x16 &small) {
  constexpr int SU = D / 32;
  using S = ScoreStage<D>;
  const uint8_t *arow = buf + l32 * S::RS + half * (S::CPR / 2) * 16;
#pragma unroll
  for (int sl = 0; sl < SU; ++sl) {
    const int s = hh * SU + sl;
    const float4 a0 = *(const float4 *)(arow + 32 * sl);
    const float4 a1 = *(const float4 *)(arow + 32 * sl + 16);
    const float x[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    bf16x8 ah, am, al;
    split3(x, ah, am, al);
    f32x16 &sm = ONE ? big : small;
    sm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, qm[s], sm, 0, 0, 0);
    sm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, qh[s], sm, 0, 0, 0);
    sm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, ql[s], sm, 0, 0, 0);
    sm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, qh[s], sm, 0, 0, 0);
    sm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qm[s], sm, 0, 0, 0);
    big = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, qh[s], big, 0, 0, 0);
  }
}

// Any row length.  Pass 1 computes each tile once and stores its raw
// log2-domain scores into P while the row statistics accumulate; after the
// statistics meet, the workgroup rewrites its rows in place, normalised,
// with row-major 16-byte loads and stores, and fills the zeros above.  The
// rewrite reads back what pass 1 just wrote (mostly from the caches) instead
// of recomputing the products: at 2048 blocks per row a recomputing pass 2
// cost as much as pass 1.  Four wavefronts (72 KiB of staging) let two
// workgroups share a CU, so one's loads, barriers and stores overlap the
// other's products.
//
// FUSE (the threshold path of stage 2 in the same launch): pass 2 also
// decides and compacts the mask.  A row's largest P is exactly 1/L (its
// largest raw score gives exp2(0) = 1), so the threshold gamma * max P is
// known before the row is rewritten; each wavefront then takes whole rows,
// writes P, the row's block mask and its ascending kept list, with the same
// arithmetic as the mask kernel on the P it has just written, so nothing
// reads P back.
template <int D, bool RESC, bool VEC, bool FUSE>
__global__ __launch_bounds__(256, 2) void score_kernel(const float *__restrict__ q_pool,
                                                       const float *__restrict__ k_pool,
                                                       const float *__restrict__ k_radius,
                                                       float *__restrict__ P, int hq, int hkv,
                                                       int nb, float c2, FuseMask fz) {
  static_assert(!(RESC && FUSE), "the fused threshold serves the base scores");
  using S = ScoreStage<D>;
  constexpr int NWV = 4;      // wavefronts
  constexpr int NT = NWV * 64;
  constexpr int NS = D / 16;  // MFMA steps per tile (16 dimensions each)
  constexpr int CPR = S::CPR, NDMA = S::NDMA;
  __shared__ float red_m[NWV][32], red_l[NWV][32], row_m[32], row_inv[32];
  __shared__ __attribute__((aligned(16))) uint8_t stg0[NWV][S::HB];
  __shared__ __attribute__((aligned(16))) uint8_t stg1[NWV][S::HB];
  const int G = (nb + 31) / 32;
  const int grp = G - 1 - (int)blockIdx.y;
  const int h = blockIdx.x;
  const int g = h / (hq / hkv);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, half = lane >> 5, l32 = lane & 31;
  const int I0 = grp * 32;
  const int rows = min(32, nb - I0);
  const int Il = I0 + l32;  // this lane's query block
  const bool row_ok = l32 < rows;
  const int ntc = (I0 + rows - 1) / 32 + 1;              // key-block tiles touching the causal part
  const int nt = w < ntc ? (ntc - w + NWV - 1) / NWV : 0;  // this wave's tiles: w, w + NWV, ...
  constexpr bool vec = VEC;  // nb % 4 == 0: rows of P are 16-byte aligned
  float *pgrp = P + ((size_t)h * nb + I0) * nb;

  int vrow[NDMA];        // source row of each load
  uint32_t vdim[NDMA];   // its byte offset inside the row
#pragma unroll
  for (int it = 0; it < NDMA; ++it) {
    const int p = it * 64 + lane, c = p % (CPR + 1);
    const int cc = c < CPR ? c : 0;
    const int kg = cc / (CPR / 2), rem = cc % (CPR / 2);
    vrow[it] = min(p / (CPR + 1), 31);
    vdim[it] = (uint32_t)((D / 2) * kg + 4 * rem) * 4;
  }
  const __amdgpu_buffer_rsrc_t krs =
      make_rsrc(k_pool + (size_t)g * nb * D, (uint32_t)((size_t)nb * D * 4));
  // unit U (0 <= U < 2 nt) = half U % 2 of the wave's tile U / 2, into buffer U % 2
  auto issue = [&](int U) {
    const int jt = w + NWV * (U >> 1);
    const uint32_t soff = (uint32_t)(jt * 32 * D + (U & 1) * (D / 4)) * 4;
    uint8_t *dst = (U & 1) ? &stg1[w][0] : &stg0[w][0];
    const int last = nb - 1 - jt * 32;
#pragma unroll
    for (int it = 0; it < NDMA; ++it)
      lds_dma16(krs, (uint32_t)min(vrow[it], last) * (D * 4) + vdim[it], soff, dst + it * 1024);
  };
  if (nt > 0) issue(0);

  bf16x8 qh[NS], qm[NS], ql[NS];
  float qn = 0.f;  // rescue branch: |Qbar_I|
  {
    const float *src = q_pool + ((size_t)h * nb + min(Il, nb - 1)) * D + (D / 2) * half;
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const float4 t0 = *(const float4 *)(src + 8 * s), t1 = *(const float4 *)(src + 8 * s + 4);
      float x[8] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z, t1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = row_ok ? x[e] : 0.f;
        if constexpr (RESC) ss = fmaf(x[e], x[e], ss);
      }
      split3(x, qh[s], qm[s], ql[s]);
    }
    if constexpr (RESC) qn = sqrtf(ss + __shfl_xor(ss, 32, 64));
  }
  const float *rad = RESC ? k_radius + (size_t)g * nb : nullptr;

  // ---- pass 1: each tile once; raw scores to P (a tile's stores go out
  // during the next tile), row max and sum of exp2
  float m = -INFINITY, l = 0.f;
  float pv[16];
  int pjt = -1;  // tile whose raw scores pv holds
  // The stores are buffer stores, the same number on every call (4, or 16
  // for rows that are not 16-byte aligned): lanes without scores to write
  // drop out through the buffer's range check.  With no branch around them
  // the compiler's own waits before the next half's LDS reads count them
  // exactly and do not also wait for the loads issued before them.
  const __amdgpu_buffer_rsrc_t prs = make_rsrc(pgrp, (uint32_t)((size_t)rows * nb * 4));
  constexpr uint32_t kDrop = 0x80000000u;  // past any range
  auto store = [&]() {
    const bool ok = pjt >= 0 && row_ok;
    const uint32_t rb = (uint32_t)(l32 * nb) * 4;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int J = pjt * 32 + q4 * 8 + half * 4;
      if constexpr (VEC) {
        const u32x4 v = {__float_as_uint(pv[4 * q4]), __float_as_uint(pv[4 * q4 + 1]),
                         __float_as_uint(pv[4 * q4 + 2]), __float_as_uint(pv[4 * q4 + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, prs, ok && J < nb ? rb + J * 4 : kDrop, 0, 0);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(pv[4 * q4 + e]), prs,
                                                ok && J + e < nb ? rb + (J + e) * 4 : kDrop, 0, 0);
      }
    }
  };
  // rescue branch: the tile's key radii, loaded ahead of the next unit's
  // Kbar (the waits are in issue order, so a load issued after it and used
  // at once would also wait for the Kbar)
  float rv[RESC ? 16 : 1];
  auto load_rad = [&](int jt) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int J = jt * 32 + q4 * 8 + half * 4;
      if (vec && J < nb) {
        const float4 t4 = *(const float4 *)(rad + J);
        rv[4 * q4] = t4.x; rv[4 * q4 + 1] = t4.y; rv[4 * q4 + 2] = t4.z; rv[4 * q4 + 3] = t4.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) rv[4 * q4 + e] = J + e < nb ? rad[J + e] : 0.f;
      }
    }
  };
  for (int t = 0; t < nt; ++t) {
    const int jt = w + NWV * t;
    f32x16 big = f32x16{}, small = f32x16{};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int U = 2 * t + hh;
      // the previous half's products stay ahead of this wait (the compiler
      // would otherwise sink some of them past it, shortening the time the
      // loads in flight have to land)
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if constexpr (RESC)
        if (hh == 0) load_rad(jt);
      issue(U + 1 < 2 * nt ? U + 1 : U - 1);  // the last unit repeats one, never read
      if (hh == 1) store();
      __builtin_amdgcn_sched_barrier(0);
      score_half<D, RESC>(hh ? &stg1[w][0] : &stg0[w][0], hh, half, l32, qh, qm, ql, big, small);
    }
    const bool edge = jt * 32 + 31 > I0 || jt * 32 + 31 >= nb;
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int J = jt * 32 + (r / 4) * 8 + half * 4 + (r % 4);
      const float add = RESC && J < nb ? qn * rv[RESC ? r : 0] : 0.f;
      const float v = (big[r] + small[r] + add) * c2;
      pv[r] = (!edge || (J <= Il && J < nb)) ? v : -INFINITY;
      tmax = fmaxf(tmax, pv[r]);
    }
    const float mn = fmaxf(m, tmax);
    if (mn != -INFINITY) {
      float acc_l = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_l += __builtin_amdgcn_exp2f(pv[r] - mn);
      l = l * __builtin_amdgcn_exp2f(m - mn) + acc_l;
      m = mn;
    }
    pjt = jt;
  }
  store();
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // raw scores and the repeat load are done
  {
    const float mo = __shfl_xor(m, 32, 64), lo = __shfl_xor(l, 32, 64);
    const float mn = fmaxf(m, mo);
    if (mn != -INFINITY) {
      l = (m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f(m - mn)) +
          (mo == -INFINITY ? 0.f : lo * __builtin_amdgcn_exp2f(mo - mn));
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
      if (red_m[i][l32] != -INFINITY)
        L += red_l[i][l32] * __builtin_amdgcn_exp2f(red_m[i][l32] - M);
    row_m[l32] = M;
    row_inv[l32] = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();  // also orders every wave's raw stores before the reads below

  // ---- pass 2: the group's rows in place, row-major: P = exp2(raw - M) / L
  // on the causal tiles, zeros above them
  const int jc = min(ntc * 32, nb);  // columns written in pass 1
  if constexpr (FUSE) {
    // one wavefront per row; the staging buffers are idle now (every load
    // has landed), so a wave's kept-list ring lives in its own
    int32_t *ring = (int32_t *)&stg0[w][0];
    for (int rr = w; rr < rows; rr += NWV) {
      const int I = I0 + rr;
      const float M = row_m[rr], inv = row_inv[rr];
      const float thr = fz.gamma * inv;  // gamma times the row's largest P
      float *prow = pgrp + (size_t)rr * nb;
      const size_t orow = ((size_t)h * nb + I) * nb;
      KeptList kl;
      kl.init(ring, fz.idx + orow, lane, vec);
      for (int J0 = 0; J0 < nb; J0 += 2048) {
        float x[8][4];  // raw scores: a whole row of up to 2048 blocks in flight
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int J = J0 + c * 256 + 4 * lane;
          if (vec && J < jc) {  // jc % 4 == 0 here: J .. J + 3 all below it
            const float4 t = *(const float4 *)(prow + J);
            x[c][0] = t.x; x[c][1] = t.y; x[c][2] = t.z; x[c][3] = t.w;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[c][e] = J + e < jc ? prow[J + e] : -INFINITY;
          }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          if (J0 + c * 256 >= nb) break;
          const int J = J0 + c * 256 + 4 * lane;
          float pv4[4];
          bool keep[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int Je = J + e;
            pv4[e] = J + e < jc ? __builtin_amdgcn_exp2f(x[c][e] - M) * inv : 0.f;
            keep[e] = Je <= I && (pv4[e] >= thr || Je < fz.sink || I - Je < fz.local);
          }
          if (vec && J + 3 < nb) {
            *(float4 *)(prow + J) = make_float4(pv4[0], pv4[1], pv4[2], pv4[3]);
            if (fz.mask)
              *(uint32_t *)(fz.mask + orow + J) =
                  (uint32_t)keep[0] | ((uint32_t)keep[1] << 8) | ((uint32_t)keep[2] << 16) |
                  ((uint32_t)keep[3] << 24);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (J + e < nb) {
                prow[J + e] = pv4[e];
                if (fz.mask) fz.mask[orow + J + e] = keep[e] ? 1 : 0;
              }
          }
          kl.push(keep, J);
        }
      }
      const int n = kl.finish();
      if (lane == 0) fz.cnt[(size_t)h * nb + I] = n;
    }
  } else if (vec) {
    // one wavefront per row, 1 KiB per load instruction, up to 8 in flight
    const int n4 = nb / 4, c4 = jc / 4;
    constexpr int U = 8;
    for (int rr = w; rr < rows; rr += NWV) {
      const float M = row_m[rr], inv = row_inv[rr];
      float4 *prow = (float4 *)(pgrp + (size_t)rr * nb);
      for (int c0 = lane; c0 < n4; c0 += U * 64) {
        float4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
          const int c = c0 + k * 64;
          v[k] = c < c4 ? prow[c] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
          const int c = c0 + k * 64;
          if (c < n4)
            prow[c] = make_float4(__builtin_amdgcn_exp2f(v[k].x - M) * inv,
                                  __builtin_amdgcn_exp2f(v[k].y - M) * inv,
                                  __builtin_amdgcn_exp2f(v[k].z - M) * inv,
                                  __builtin_amdgcn_exp2f(v[k].w - M) * inv);
        }
      }
    }
  } else {
    for (int rr = w; rr < rows; rr += NWV) {
      const float M = row_m[rr], inv = row_inv[rr];
      float *prow = pgrp + (size_t)rr * nb;
      for (int J = lane; J < nb; J += 64)
        prow[J] = J < jc ? __builtin_amdgcn_exp2f(prow[J] - M) * inv : 0.f;
    }
  }
}

template <int D, bool RESC, bool FUSE>
static hipError_t launch_score_t(const Shape &s, float c, const float *qp, const float *kp,
                                 const float *kr, float *S, const FuseMask &fz, hipStream_t st) {
  // heaviest row groups of every head first
  const dim3 grid(s.hq, (s.nb + 31) / 32);
  if (s.nb % 4 == 0)
    hipLaunchKernelGGL((score_kernel<D, RESC, true, FUSE>), grid, dim3(256), 0, st, qp, kp, kr,
                       S, s.hq, s.hkv, s.nb, c * kLog2e, fz);
  else
    hipLaunchKernelGGL((score_kernel<D, RESC, false, FUSE>), grid, dim3(256), 0, st, qp, kp, kr,
                       S, s.hq, s.hkv, s.nb, c * kLog2e, fz);
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
  const FuseMask none{};
  if (k_radius) {
    if (s.d == 64) return launch_score_t<64, true, false>(s, c, q_pool, k_pool, k_radius, S, none, st);
    return launch_score_t<128, true, false>(s, c, q_pool, k_pool, k_radius, S, none, st);
  }
  if (s.d == 64) return launch_score_t<64, false, false>(s, c, q_pool, k_pool, nullptr, S, none, st);
  return launch_score_t<128, false, false>(s, c, q_pool, k_pool, nullptr, S, none, st);
}

hipError_t launch_score_mask(const Shape &s, float c, const float *q_pool, const float *k_pool,
                             float *S, const FuseMask &fz, hipStream_t st) {
  if (s.d == 64) return launch_score_t<64, false, true>(s, c, q_pool, k_pool, nullptr, S, fz, st);
  return launch_score_t<128, false, true>(s, c, q_pool, k_pool, nullptr, S, fz, st);
}

}  // namespace bsp
