// Stage 1b: block scores and their row normalisation (FlashPrefill summary
// page, section 3 "Block Approximation for Kernel Optimization": scores live
// on the (L/B) x (L/B) block grid, never on an L x (L/B) intermediate;
// Appendix B: query tiles against causally valid pooled key blocks, then a
// global normalisation).
//
//   score_logits_kernel   S[h][I][J] = c * q_pool[h][I] . k_pool[g][J], J <= I.
//       A causal fp32 GEMM on the pooled operands.  One workgroup owns 64 query
//       blocks of one head, keeps their pooled rows in LDS (d-major) and sweeps
//       64-wide key-block tiles up to its diagonal; each lane accumulates a 4x4
//       register tile.  fp32 throughout: the threshold compares scores, so the
//       pooled operands are not rounded to a narrower type.
//   score_softmax_kernel  one wavefront per row: max, sum of exp, normalise in
//       place, zero the entries above the diagonal.
#include "device.h"
#include "internal.h"

namespace bsp {

constexpr int kST = 64;  // query / key blocks per tile

template <int D>
__global__ __launch_bounds__(256) void score_logits_kernel(const float *__restrict__ q_pool,
                                                           const float *__restrict__ k_pool,
                                                           float *__restrict__ S, int hq, int hkv,
                                                           int nb, float c) {
  __shared__ float qt[D][kST + 4];
  __shared__ float kt[D][kST + 4];
  const int h = blockIdx.y;
  const int g = h / (hq / hkv);
  const int I0 = blockIdx.x * kST;
  const int tid = threadIdx.x;
  const int ty = tid / 16, tx = tid % 16;

  constexpr int F4 = D / 4;  // float4 per pooled row
  for (int e = tid; e < kST * F4; e += 256) {
    const int r = e / F4, d4 = (e % F4) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (I0 + r < nb) v = *(const float4 *)(q_pool + ((size_t)h * nb + I0 + r) * D + d4);
    qt[d4 + 0][r] = v.x;
    qt[d4 + 1][r] = v.y;
    qt[d4 + 2][r] = v.z;
    qt[d4 + 3][r] = v.w;
  }
  const int Ilast = min(I0 + kST, nb) - 1;
  for (int J0 = 0; J0 <= Ilast; J0 += kST) {
    __syncthreads();
    for (int e = tid; e < kST * F4; e += 256) {
      const int r = e / F4, d4 = (e % F4) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (J0 + r < nb) v = *(const float4 *)(k_pool + ((size_t)g * nb + J0 + r) * D + d4);
      kt[d4 + 0][r] = v.x;
      kt[d4 + 1][r] = v.y;
      kt[d4 + 2][r] = v.z;
      kt[d4 + 3][r] = v.w;
    }
    __syncthreads();
    float acc[4][4] = {};
#pragma unroll 8
    for (int d = 0; d < D; ++d) {
      const float4 a = *(const float4 *)&qt[d][ty * 4];
      const float4 b = *(const float4 *)&kt[d][tx * 4];
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int I = I0 + ty * 4 + i;
      if (I >= nb) continue;
      float *row = S + ((size_t)h * nb + I) * nb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int J = J0 + tx * 4 + j;
        if (J <= I) row[J] = acc[i][j] * c;
      }
    }
  }
}

__global__ __launch_bounds__(256) void score_softmax_kernel(float *__restrict__ S, int rows,
                                                            int nb) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int I = row % nb;
  float *p = S + (size_t)row * nb;
  float m = -INFINITY;
  for (int J = lane; J <= I; J += 64) m = fmaxf(m, p[J]);
  m = wave_max(m);
  float l = 0.f;
  for (int J = lane; J <= I; J += 64) l += expf(p[J] - m);
  l = wave_sum(l);
  const float inv = 1.f / l;
  for (int J = lane; J < nb; J += 64) p[J] = J <= I ? expf(p[J] - m) * inv : 0.f;
}

template <int D>
static hipError_t launch_score_t(const Shape &s, float c, const float *qp, const float *kp,
                                 float *S, hipStream_t st) {
  dim3 grid((s.nb + kST - 1) / kST, s.hq);
  hipLaunchKernelGGL(score_logits_kernel<D>, grid, dim3(256), 0, st, qp, kp, S, s.hq, s.hkv,
                     s.nb, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = s.hq * s.nb;
  hipLaunchKernelGGL(score_softmax_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, S, rows, s.nb);
  return hipGetLastError();
}

hipError_t launch_score(const Shape &s, float c, const float *qp, const float *kp, float *S,
                        hipStream_t st) {
  if (s.d == 64) return launch_score_t<64>(s, c, qp, kp, S, st);
  return launch_score_t<128>(s, c, qp, kp, S, st);
}

}  // namespace bsp
