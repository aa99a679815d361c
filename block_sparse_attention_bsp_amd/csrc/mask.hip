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
// lower lanes plus its own earlier kept elements.
#include "device.h"
#include "internal.h"

namespace bsp {

__global__ __launch_bounds__(256) void mask_kernel(const float *__restrict__ P,
                                                   const uint8_t *__restrict__ user,
                                                   uint8_t *__restrict__ mask,
                                                   int32_t *__restrict__ kv_idx,
                                                   int32_t *__restrict__ kv_cnt, int rows, int nb,
                                                   float gamma, int sink, int local) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int I = row % nb;
  const size_t off = (size_t)row * nb;
  const bool vec = (nb & 3) == 0;  // rows are 16-byte aligned

  auto load4 = [&](const float *p, int J, float (&x)[4]) {
    if (vec && J + 3 < nb) {
      const float4 t = *(const float4 *)(p + J);
      x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = J + e < nb ? p[J + e] : 0.f;
    }
  };

  float thr = 0.f;
  if (!user) {
    float m = -INFINITY;
    for (int J0 = 4 * lane; J0 <= I; J0 += 256) {
      float x[4];
      load4(P + off, J0, x);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (J0 + e <= I) m = fmaxf(m, x[e]);
    }
    thr = gamma * wave_max(m);
  }

  const uint64_t below = (1ull << lane) - 1ull;
  int n = 0;
  for (int J0 = 0; J0 < nb; J0 += 256) {
    const int J = J0 + 4 * lane;
    bool keep[4] = {false, false, false, false};
    if (J <= I) {
      if (user) {
        if (vec && J + 3 < nb) {
          const uint32_t u4 = *(const uint32_t *)(user + off + J);
#pragma unroll
          for (int e = 0; e < 4; ++e) keep[e] = ((u4 >> (8 * e)) & 0xFFu) != 0;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) keep[e] = J + e < nb && user[off + J + e] != 0;
        }
      } else {
        float x[4];
        load4(P + off, J, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int Je = J + e;
          keep[e] = x[e] >= thr || Je < sink || I - Je < local;
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) keep[e] = keep[e] && J + e <= I;
    }
    if (mask) {
      if (vec && J + 3 < nb) {
        *(uint32_t *)(mask + off + J) = (uint32_t)keep[0] | ((uint32_t)keep[1] << 8) |
                                        ((uint32_t)keep[2] << 16) | ((uint32_t)keep[3] << 24);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (J + e < nb) mask[off + J + e] = keep[e] ? 1 : 0;
      }
    }
    uint64_t bal[4];
    int before = 0, total = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bal[e] = __ballot(keep[e]);
      before += __popcll(bal[e] & below);
      total += __popcll(bal[e]);
    }
    int mine = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (keep[e]) kv_idx[off + n + before + mine] = J + e;
      mine += keep[e] ? 1 : 0;
    }
    n += total;
  }
  if (lane == 0) kv_cnt[row] = n;
}

// Rows of at most 256 * NS blocks under the max-based threshold: the row of
// P is read from HBM once, all of a lane's loads in flight together, and kept
// in registers for the decision and the compaction.
template <int NS>
__global__ __launch_bounds__(256) void mask_kernel_reg(const float *__restrict__ P,
                                                       uint8_t *__restrict__ mask,
                                                       int32_t *__restrict__ kv_idx,
                                                       int32_t *__restrict__ kv_cnt, int rows,
                                                       int nb, float gamma, int sink, int local) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int I = row % nb;
  const size_t off = (size_t)row * nb;
  const bool vec = (nb & 3) == 0;  // rows are 16-byte aligned

  float x[NS][4];
  float m = -INFINITY;
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const int J = t * 256 + 4 * lane;
    if (J <= I) {
      if (vec && J + 3 < nb) {
        const float4 v = *(const float4 *)(P + off + J);
        x[t][0] = v.x; x[t][1] = v.y; x[t][2] = v.z; x[t][3] = v.w;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[t][e] = J + e < nb ? P[off + J + e] : 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[t][e] = 0.f;
    }
  }
#pragma unroll
  for (int t = 0; t < NS; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (t * 256 + 4 * lane + e <= I) m = fmaxf(m, x[t][e]);
  const float thr = gamma * wave_max(m);

  const uint64_t below = (1ull << lane) - 1ull;
  int n = 0;
#pragma unroll
  for (int t = 0; t < NS; ++t) {
    const int J = t * 256 + 4 * lane;
    if (t * 256 >= nb) break;
    bool keep[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int Je = J + e;
      keep[e] = Je <= I && (x[t][e] >= thr || Je < sink || I - Je < local);
    }
    if (vec && J + 3 < nb) {
      *(uint32_t *)(mask + off + J) = (uint32_t)keep[0] | ((uint32_t)keep[1] << 8) |
                                      ((uint32_t)keep[2] << 16) | ((uint32_t)keep[3] << 24);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (J + e < nb) mask[off + J + e] = keep[e] ? 1 : 0;
    }
    uint64_t bal[4];
    int before = 0, total = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bal[e] = __ballot(keep[e]);
      before += __popcll(bal[e] & below);
      total += __popcll(bal[e]);
    }
    int mine = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (keep[e]) kv_idx[off + n + before + mine] = J + e;
      mine += keep[e] ? 1 : 0;
    }
    n += total;
  }
  if (lane == 0) kv_cnt[row] = n;
}

hipError_t launch_mask(const Shape &s, float gamma, int sink, int local, const float *score,
                       const uint8_t *user, uint8_t *mask, int32_t *idx, int32_t *cnt,
                       hipStream_t st) {
  const int rows = s.hq * s.nb;
  const dim3 grid((rows + 3) / 4), block(256);
  if (!user && s.nb <= 256)
    hipLaunchKernelGGL(mask_kernel_reg<1>, grid, block, 0, st, score, mask, idx, cnt, rows, s.nb,
                       gamma, sink, local);
  else if (!user && s.nb <= 512)
    hipLaunchKernelGGL(mask_kernel_reg<2>, grid, block, 0, st, score, mask, idx, cnt, rows, s.nb,
                       gamma, sink, local);
  else if (!user && s.nb <= 1024)
    hipLaunchKernelGGL(mask_kernel_reg<4>, grid, block, 0, st, score, mask, idx, cnt, rows, s.nb,
                       gamma, sink, local);
  else if (!user && s.nb <= 2048)
    hipLaunchKernelGGL(mask_kernel_reg<8>, grid, block, 0, st, score, mask, idx, cnt, rows, s.nb,
                       gamma, sink, local);
  else
    hipLaunchKernelGGL(mask_kernel, grid, block, 0, st, score, user, mask, idx, cnt, rows, s.nb,
                       gamma, sink, local);
  return hipGetLastError();
}

}  // namespace bsp
