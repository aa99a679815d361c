// Stage 2: max-based dynamic thresholding and block selection (FlashPrefill
// summary page, section 3 "Max-based Dynamic Thresholding": the pruning
// threshold comes from each query block's peak score, so no sort and no
// cumulative sum is needed; Appendix A: sink and local-window blocks are
// retained on top; Appendix B: score, sink, window and causal masks are
// combined, then the active-block indices are compressed).
//
// One wavefront per (head, query block) row; each lane covers 4 consecutive
// key blocks per step (128-bit score loads).  The row maximum is a wavefront
// max-reduction; the kept set is compacted in ascending order from four
// 64-wide ballots per step: a lane's slot is the popcount of the kept bits of
// lower lanes plus its own earlier kept elements.  The compacted indices are
// the kernel's largest output; they leave in whole 1 KiB runs (KeptList).
//
// Dual-branch form (rescue branch, thelatestinai page, RBS-Attention
// abstract: the two branches are thresholded independently and their masks
// combined): a block is kept when its base score reaches gamma times the
// row's base maximum, or its rescue score reaches gamma_r times the row's
// rescue maximum, or it is forced.
#include "device.h"
#include "internal.h"
#include "kept_list.h"

namespace bsp {

// VL: rows of a packed variable-length batch: row h * nb + gb (nb = the
// batch's query blocks) belongs to sequence s and is its query block
// I = gb - cu_blocks[s]; it has the sequence's nb_s columns and stride ld.
template <bool DUAL, bool VL>
__global__ __launch_bounds__(256) void mask_kernel(const float *__restrict__ P,
                                                   const float *__restrict__ Pr,
                                                   const uint8_t *__restrict__ user,
                                                   uint8_t *__restrict__ mask,
                                                   int32_t *__restrict__ kv_idx,
                                                   int32_t *__restrict__ kv_cnt, int rows, int nb,
                                                   float gamma, float gamma_r, int sink,
                                                   int local, int ld, VarlenArgs vl) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  int I = row % nb, ncol = nb;
  if constexpr (VL) {
    const int sq = varlen_seq_of(vl.cu_blocks, vl.nseq, I);
    // a row never reaches past its stride, whatever the offsets say
    ncol = min(vl.cu_blocks[sq + 1] - vl.cu_blocks[sq], ld);
    I = min(I - vl.cu_blocks[sq], ncol - 1);
  } else {
    ld = nb;
  }
  const size_t off = (size_t)row * ld;
  const bool vec = (ld & 3) == 0;  // rows are 16-byte aligned

  auto load4 = [&](const float *p, int J, float (&x)[4]) {
    if (vec && J + 3 < ncol) {
      const float4 t = *(const float4 *)(p + J);
      x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = J + e < ncol ? p[J + e] : 0.f;
    }
  };

  float thr = 0.f, thr_r = 0.f;
  if (!user) {
    float m = -INFINITY, mr = -INFINITY;
    for (int J0 = 4 * lane; J0 <= I; J0 += 256) {
      float x[4], y[4];
      load4(P + off, J0, x);
      if constexpr (DUAL) load4(Pr + off, J0, y);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (J0 + e <= I) {
          m = fmaxf(m, x[e]);
          if constexpr (DUAL) mr = fmaxf(mr, y[e]);
        }
    }
    thr = gamma * wave_max(m);
    if constexpr (DUAL) thr_r = gamma_r * wave_max(mr);
  }

  __shared__ __attribute__((aligned(16))) int32_t ring[4][512];
  KeptList kl;
  kl.init(ring[threadIdx.x >> 6], kv_idx + off, lane, vec);
  for (int J0 = 0; J0 < ncol; J0 += 256) {
    const int J = J0 + 4 * lane;
    bool keep[4] = {false, false, false, false};
    if (J <= I) {
      if (user) {
        if (vec && J + 3 < ncol) {
          const uint32_t u4 = *(const uint32_t *)(user + off + J);
#pragma unroll
          for (int e = 0; e < 4; ++e) keep[e] = ((u4 >> (8 * e)) & 0xFFu) != 0;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) keep[e] = J + e < ncol && user[off + J + e] != 0;
        }
      } else {
        float x[4], y[4];
        load4(P + off, J, x);
        if constexpr (DUAL) load4(Pr + off, J, y);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int Je = J + e;
          keep[e] = x[e] >= thr || (DUAL && y[e] >= thr_r) || Je < sink || I - Je < local;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) keep[e] = keep[e] && J + e <= I;
    }
    if (mask) {
      if (vec && J + 3 < ncol) {
        *(uint32_t *)(mask + off + J) = (uint32_t)keep[0] | ((uint32_t)keep[1] << 8) |
                                        ((uint32_t)keep[2] << 16) | ((uint32_t)keep[3] << 24);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (J + e < ncol) mask[off + J + e] = keep[e] ? 1 : 0;
      }
    }
    kl.push(keep, J);
  }
  const int n = kl.finish();
  if (lane == 0) kv_cnt[row] = n;
}

// Rows of at most 256 * NS blocks under the max-based threshold: the row of
// P is read from HBM once, all of a lane's loads in flight together, and kept
// in registers for the decision and the compaction.
template <int NS, bool DUAL>
__global__ __launch_bounds__(256) void mask_kernel_reg(const float *__restrict__ P,
                                                       const float *__restrict__ Pr,
                                                       uint8_t *__restrict__ mask,
                                                       int32_t *__restrict__ kv_idx,
                                                       int32_t *__restrict__ kv_cnt, int rows,
                                                       int nb, float gamma, float gamma_r, int sink,
                                                       int local) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int I = row % nb;
  const size_t off = (size_t)row * nb;
  const bool vec = (nb & 3) == 0;  // rows are 16-byte aligned

  auto row4 = [&](const float *src, int J, float (&v4)[4]) {
    if (J <= I) {
      if (vec && J + 3 < nb) {
        const float4 v = *(const float4 *)(src + off + J);
        v4[0] = v.x; v4[1] = v.y; v4[2] = v.z; v4[3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = J + e < nb ? src[off + J + e] : 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = 0.f;
    }
  };
  float x[NS][4], y[DUAL ? NS : 1][4];
  float m = -INFINITY, mr = -INFINITY;
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    row4(P, t * 256 + 4 * lane, x[t]);
    if constexpr (DUAL) row4(Pr, t * 256 + 4 * lane, y[t]);
  }
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (t * 256 + 4 * lane + e <= I) {
        m = fmaxf(m, x[t][e]);
        if constexpr (DUAL) mr = fmaxf(mr, y[t][e]);
      }
  const float thr = gamma * wave_max(m);
  const float thr_r = DUAL ? gamma_r * wave_max(mr) : 0.f;

  __shared__ __attribute__((aligned(16))) int32_t ring[4][512];
  KeptList kl;
  kl.init(ring[threadIdx.x >> 6], kv_idx + off, lane, vec);
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const int J = t * 256 + 4 * lane;
    if (t * 256 >= nb) break;
    bool keep[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int Je = J + e;
      keep[e] = Je <= I && (x[t][e] >= thr || (DUAL && y[DUAL ? t : 0][e] >= thr_r) ||
                            Je < sink || I - Je < local);
    }
    if (mask) {  // the block mask is optional (wave-uniform branch)
      if (vec && J + 3 < nb) {
        *(uint32_t *)(mask + off + J) = (uint32_t)keep[0] | ((uint32_t)keep[1] << 8) |
                                        ((uint32_t)keep[2] << 16) | ((uint32_t)keep[3] << 24);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (J + e < nb) mask[off + J + e] = keep[e] ? 1 : 0;
      }
    }
    kl.push(keep, J);
  }
  const int n = kl.finish();
  if (lane == 0) kv_cnt[row] = n;
}

template <bool DUAL>
static hipError_t launch_mask_t(const Shape &s, float gamma, float gamma_r, int sink, int local,
                                const float *score, const float *rescue, const uint8_t *user,
                                uint8_t *mask, int32_t *idx, int32_t *cnt, hipStream_t st) {
  const int rows = s.hq * s.nb;
  const dim3 grid((rows + 3) / 4), block(256);
#define BSP_MASK_REG(NS)                                                                       \
  hipLaunchKernelGGL((mask_kernel_reg<NS, DUAL>), grid, block, 0, st, score, rescue, mask, idx, \
                     cnt, rows, s.nb, gamma, gamma_r, sink, local)
  if (!user && s.nb <= 256)
    BSP_MASK_REG(1);
  else if (!user && s.nb <= 512)
    BSP_MASK_REG(2);
  else if (!user && s.nb <= 1024)
    BSP_MASK_REG(4);
  else if (!user && s.nb <= 2048)
    BSP_MASK_REG(8);
  else
    hipLaunchKernelGGL((mask_kernel<DUAL, false>), grid, block, 0, st, score, rescue, user, mask,
                       idx, cnt, rows, s.nb, gamma, gamma_r, sink, local, s.nb, VarlenArgs{});
#undef BSP_MASK_REG
  return hipGetLastError();
}

hipError_t launch_mask(const Shape &s, float gamma, int sink, int local, const float *score,
                       const uint8_t *user, uint8_t *mask, int32_t *idx, int32_t *cnt,
                       hipStream_t st, const float *rescue, float gamma_r) {
  if (rescue && !user)
    return launch_mask_t<true>(s, gamma, gamma_r, sink, local, score, rescue, nullptr, mask, idx,
                               cnt, st);
  return launch_mask_t<false>(s, gamma, 0.f, sink, local, score, nullptr, user, mask, idx, cnt, st);
}

hipError_t launch_mask_varlen(const Shape &s, const VarlenArgs &vl, float gamma, int sink,
                              int local, const float *score, const uint8_t *user, uint8_t *mask,
                              int32_t *idx, int32_t *cnt, hipStream_t st) {
  const int rows = s.hq * s.nb;
  hipLaunchKernelGGL((mask_kernel<false, true>), dim3((rows + 3) / 4), dim3(256), 0, st,
                     user ? nullptr : score, nullptr, user, mask, idx, cnt, rows, s.nb, gamma, 0.f,
                     sink, local, vl.idx_stride, vl);
  return hipGetLastError();
}

}  // namespace bsp
