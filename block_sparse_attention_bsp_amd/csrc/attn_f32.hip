// Stage 3 for fp32 inputs: block-sparse causal attention with an online
// softmax (FlashPrefill summary page, Appendix B "Block Sparse Attention":
// iterate only over the selected key blocks, causal masking where required,
// online softmax updates, final normalisation).
//
// fp32 FMA throughout (no MFMA): this path serves small fp32 problems and
// exactness checks.  One workgroup per (head, query block); 256 / B lanes
// share a query and split its d dimensions; keys stream through LDS in
// chunks of 32.
#include "device.h"
#include "internal.h"

namespace bsp {

template <int D, int BLK>
__global__ __launch_bounds__(256) void attn_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ kv_cnt, float *__restrict__ o,
    float *__restrict__ lse, int hq, int hkv, int seq, int nb, float scale2) {
  constexpr int TPQ = 256 / BLK;  // lanes per query
  constexpr int DP = D / TPQ;     // dims per lane
  constexpr int KC = 32;          // keys per LDS chunk
  __shared__ float ks[KC][D + 4];
  __shared__ float vs[KC][D + 4];

  const int bid = blockIdx.x;
  const int I = nb - 1 - bid / hq;
  const int h = bid % hq;
  const int g = h / (hq / hkv);
  const int tid = threadIdx.x;
  const int part = tid % TPQ;
  const int i = I * BLK + tid / TPQ;
  const size_t row = (size_t)h * nb + I;

  float qv[DP], acc[DP];
#pragma unroll
  for (int e = 0; e < DP; ++e) {
    qv[e] = i < seq ? q[((size_t)h * seq + i) * D + part * DP + e] : 0.f;
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int n = kv_idx ? min(kv_cnt[row], nb) : I + 1;
  for (int t = 0; t < n; ++t) {
    const int J = kv_idx ? kv_idx[row * nb + t] : t;
    if (J < 0 || J > I) continue;
    for (int c0 = 0; c0 < BLK; c0 += KC) {
      const int j0 = J * BLK + c0;
      __syncthreads();
      for (int e = tid; e < KC * D / 4; e += 256) {
        const int r = e / (D / 4), d4 = (e % (D / 4)) * 4;
        float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
        if (j0 + r < seq) {
          kk = *(const float4 *)(k + ((size_t)g * seq + j0 + r) * D + d4);
          vv = *(const float4 *)(v + ((size_t)g * seq + j0 + r) * D + d4);
        }
        *(float4 *)&ks[r][d4] = kk;
        *(float4 *)&vs[r][d4] = vv;
      }
      __syncthreads();
      float s[KC];
      float mx = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < KC; ++jj) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < DP; ++e) a = fmaf(qv[e], ks[jj][part * DP + e], a);
#pragma unroll
        for (int o2 = 1; o2 < TPQ; o2 <<= 1) a += __shfl_xor(a, o2, 64);
        a *= scale2;
        if (j0 + jj > i) a = -INFINITY;
        s[jj] = a;
        mx = fmaxf(mx, a);
      }
      const float mnew = fmaxf(m, mx);
      if (mnew == -INFINITY) continue;
      const float alpha = exp2f(m - mnew);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < DP; ++e) acc[e] *= alpha;
#pragma unroll
      for (int jj = 0; jj < KC; ++jj) {
        const float p = exp2f(s[jj] - mnew);
        l += p;
#pragma unroll
        for (int e = 0; e < DP; ++e) acc[e] = fmaf(p, vs[jj][part * DP + e], acc[e]);
      }
      m = mnew;
    }
  }
  if (i < seq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < DP; ++e) o[((size_t)h * seq + i) * D + part * DP + e] = acc[e] * inv;
    if (lse && part == 0) lse[(size_t)h * seq + i] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, int BLK>
static hipError_t launch_t(const Shape &s, const AttnArgs &a, hipStream_t st) {
  const float scale2 = a.sm_scale * kLog2e;
  hipLaunchKernelGGL((attn_f32_kernel<D, BLK>), dim3(s.hq * s.nb), dim3(256), 0, st,
                     (const float *)a.q, (const float *)a.k, (const float *)a.v, a.kv_idx,
                     a.kv_cnt, (float *)a.o, a.lse, s.hq, s.hkv, s.seq, s.nb, scale2);
  return hipGetLastError();
}

hipError_t launch_attn_f32(const Shape &s, const AttnArgs &a, hipStream_t st) {
  if (s.d == 64 && s.block == 64) return launch_t<64, 64>(s, a, st);
  if (s.d == 64 && s.block == 128) return launch_t<64, 128>(s, a, st);
  if (s.d == 128 && s.block == 64) return launch_t<128, 64>(s, a, st);
  return launch_t<128, 128>(s, a, st);
}

}  // namespace bsp
