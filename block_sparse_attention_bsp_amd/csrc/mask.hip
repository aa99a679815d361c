// Stage 2: max-based dynamic thresholding and block selection (FlashPrefill
// summary page, section 3 "Max-based Dynamic Thresholding": the pruning
// threshold comes from each query block's peak score, so no sort and no
// cumulative sum is needed; Appendix A: sink and local-window blocks are
// retained on top; Appendix B: score, sink, window and causal masks are
// combined, then the active-block indices are compressed).
//
// One wavefront per (head, query block) row.  The row maximum is a wavefront
// max-reduction; the kept set is compacted into ascending order with a
// 64-wide ballot and a popcount prefix per chunk of key blocks.
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
  float thr = 0.f;
  if (!user) {
    float m = -INFINITY;
    for (int J = lane; J <= I; J += 64) m = fmaxf(m, P[off + J]);
    thr = gamma * wave_max(m);
  }
  const uint64_t below = (1ull << lane) - 1ull;
  int n = 0;
  for (int J0 = 0; J0 < nb; J0 += 64) {
    const int J = J0 + lane;
    bool keep = false;
    if (J <= I) {
      if (user)
        keep = user[off + J] != 0;
      else
        keep = P[off + J] >= thr || J < sink || I - J < local;
    }
    if (mask && J < nb) mask[off + J] = keep ? 1 : 0;
    const uint64_t bal = __ballot(keep);
    if (keep) kv_idx[off + n + __popcll(bal & below)] = J;
    n += __popcll(bal);
  }
  if (lane == 0) kv_cnt[row] = n;
}

hipError_t launch_mask(const Shape &s, float gamma, int sink, int local, const float *score,
                       const uint8_t *user, uint8_t *mask, int32_t *idx, int32_t *cnt,
                       hipStream_t st) {
  const int rows = s.hq * s.nb;
  hipLaunchKernelGGL(mask_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, score, user, mask, idx,
                     cnt, rows, s.nb, gamma, sink, local);
  return hipGetLastError();
}

}  // namespace bsp
