// Stage 3 for bf16 and fp8 inputs: block-sparse causal attention on MFMA
// (FlashPrefill summary page, Appendix B "Block Sparse Attention": only the
// selected key blocks are visited, causal masking is applied where required -
// here only on the diagonal block - with online softmax updates and a final
// normalisation).  fp8 inputs follow the FP8 inference of the FlashPrefill V2
// abstract (thelatestinai.com page): e4m3 operands, fp32 accumulation.
//
// gfx950 design
//   * One workgroup per (q head, query block I): B/32 wavefronts, each owning
//     32 queries, whose Q fragments stay in registers for the whole row.
//   * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16,
//     or v_mfma_scale_f32_32x32x64_f8f6f4 with unit scales for e4m3): in the
//     32x32 result every lane holds one query and 16 keys, so the softmax row
//     max and row sum are in-lane plus one exchange with the lane 32 away.
//   * The output is accumulated transposed, O^T += V^T P^T (bf16 MFMA), so
//     each lane's accumulators belong to its own query and the online-softmax
//     rescale is a per-lane scalar.  P^T is the B operand straight from the
//     score registers; the key order within a 16-key step is permuted the same
//     way on both operands.
//   * K and V sub-tiles of 64 keys are staged through LDS.  K rows carry an
//     XOR swizzle of their read units (conflict-free 16/32-byte reads).  V is
//     stored row-major as bf16 (fp8 codes are widened exactly) and read with
//     ds_read_b64_tr_b16, whose 4x16 transpose hands each lane one d column
//     of four consecutive keys - the V^T operand without a transposed copy.
//   * Softmax in fp32 with exp2 (log2 e and, for fp8, the q/k scales folded
//     into one factor); the v scale is applied at the final normalisation.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace bsp {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int DT, int D, int BLK>
struct AttnCfg {
  static constexpr int ES = DT == kFP8 ? 1 : 2;  // bytes per Q/K element
  static constexpr int RB = D * ES;              // bytes per K row
  static constexpr int KSTEP = DT == kFP8 ? 64 : 16;
  static constexpr int LB = KSTEP / 2 * ES;      // bytes per lane per S^T step (16 or 32)
  static constexpr int DK = D / KSTEP;           // S^T k-steps
  static constexpr int UNITS = RB / LB;          // read units per K row
  static constexpr int KRPW = RB >= 256 ? 1 : 256 / RB;  // K rows per 256-byte window
  static constexpr int VCH = D / 8;              // 16-byte chunks per bf16 V row
  static constexpr int VRPW = D >= 128 ? 1 : 128 / D;
  static constexpr int NW = BLK / 32;
  static constexpr int NT = NW * 64;
  static constexpr int KT = 64;                  // keys per LDS sub-tile
  static constexpr int NSUB = BLK / KT;
  static constexpr int KTS = KT / 32;
  static constexpr int DTL = D / 32;
};

template <int DT, int D, int BLK>
__device__ __forceinline__ int k_unit(int r, int u) {
  using C = AttnCfg<DT, D, BLK>;
  return u ^ ((r / C::KRPW) % C::UNITS);
}

template <int D>
__device__ __forceinline__ int v_chunk(int r, int c) {
  constexpr int VCH = D / 8, VRPW = D >= 128 ? 1 : 128 / D;
  return c ^ (((r / VRPW) % (VCH / 2)) * 2);
}

__device__ __forceinline__ uint32_t e4m3_pair_to_bf16(uint32_t two) {
  // two e4m3 codes (low byte first) -> two bf16 (exact: 4 significant bits)
  return (__float_as_uint(e4m3_to_f32(two & 0xFFu)) >> 16) |
         (__float_as_uint(e4m3_to_f32((two >> 8) & 0xFFu)) & 0xFFFF0000u);
}

template <int DT, int D, int BLK>
__global__ __launch_bounds__(BLK * 2) void attn_mfma_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ k, const uint8_t *__restrict__ v,
    const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ kv_cnt,
    uint16_t *__restrict__ o, float *__restrict__ lse, const float *__restrict__ q_scale,
    const float *__restrict__ k_scale, const float *__restrict__ v_scale, int hq, int hkv,
    int seq, int nb, float sm_scale_log2) {
  using C = AttnCfg<DT, D, BLK>;
  constexpr int ES = C::ES, RB = C::RB, LB = C::LB, DK = C::DK, KT = C::KT, NT = C::NT;
  constexpr int KTS = C::KTS, DTL = C::DTL;
  __shared__ __attribute__((aligned(16))) uint8_t Ks[KT * RB];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[KT * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const int bid = blockIdx.x;
  const int I = nb - 1 - bid / hq;
  const int h = bid % hq;
  const int g = h / (hq / hkv);
  const int qi = I * BLK + w * 32 + l32;
  const size_t row = (size_t)h * nb + I;
  float scale2 = sm_scale_log2;
  if constexpr (DT == kFP8) scale2 *= q_scale[h] * k_scale[g];

  // Q fragments: B operand of S^T = K Q^T, query qi, LB bytes per step.
  typedef typename std::conditional<DT == kFP8, i32x8, bf16x8>::type frag_t;
  frag_t qf[DK];
#pragma unroll
  for (int kk = 0; kk < DK; ++kk) {
    const uint8_t *src = q + ((size_t)h * seq + qi) * RB + kk * 2 * LB + half * LB;
    uint4 a = make_uint4(0, 0, 0, 0), b = a;
    if (qi < seq) {
      a = *(const uint4 *)src;
      if constexpr (LB == 32) b = *(const uint4 *)(src + 16);
    }
    if constexpr (LB == 32) {
      const uint4 ab[2] = {a, b};
      __builtin_memcpy(&qf[kk], ab, 32);
    } else {
      __builtin_memcpy(&qf[kk], &a, 16);
    }
  }

  f32x16 oacc[DTL];
#pragma unroll
  for (int db = 0; db < DTL; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const int n = kv_idx ? min(kv_cnt[row], nb) : I + 1;
  for (int t = 0; t < n; ++t) {
    const int J = kv_idx ? kv_idx[row * nb + t] : t;
    if (J < 0 || J > I) continue;
    const bool diag = J == I;
    for (int sub = 0; sub < C::NSUB; ++sub) {
      const int j0 = J * BLK + sub * KT;
      __syncthreads();
      // ---- stage K (swizzled read units) and V (bf16, swizzled chunks)
      for (int e = tid; e < KT * RB / 16; e += NT) {
        const int r = e / (RB / 16), c = e % (RB / 16);
        uint4 kv4 = make_uint4(0, 0, 0, 0), vv4 = kv4;
        if (j0 + r < seq) {
          const size_t goff = ((size_t)g * seq + j0 + r) * RB + c * 16;
          kv4 = *(const uint4 *)(k + goff);
          vv4 = *(const uint4 *)(v + goff);
        }
        constexpr int CPU = LB / 16;  // 16-byte chunks per read unit
        const int pu = k_unit<DT, D, BLK>(r, c / CPU);
        *(uint4 *)&Ks[r * RB + pu * LB + (c % CPU) * 16] = kv4;
        if constexpr (DT == kFP8) {
          const uint4 lo = make_uint4(e4m3_pair_to_bf16(vv4.x), e4m3_pair_to_bf16(vv4.x >> 16),
                                      e4m3_pair_to_bf16(vv4.y), e4m3_pair_to_bf16(vv4.y >> 16));
          const uint4 hi = make_uint4(e4m3_pair_to_bf16(vv4.z), e4m3_pair_to_bf16(vv4.z >> 16),
                                      e4m3_pair_to_bf16(vv4.w), e4m3_pair_to_bf16(vv4.w >> 16));
          *(uint4 *)&Vs[r * D + v_chunk<D>(r, 2 * c) * 8] = lo;
          *(uint4 *)&Vs[r * D + v_chunk<D>(r, 2 * c + 1) * 8] = hi;
        } else {
          *(uint4 *)&Vs[r * D + v_chunk<D>(r, c) * 8] = vv4;
        }
      }
      __syncthreads();

      // ---- S^T tiles: rows = keys of the sub-tile, columns = the wave's queries
      f32x16 s[KTS];
#pragma unroll
      for (int kt = 0; kt < KTS; ++kt) {
        s[kt] = f32x16{};
        const int r = kt * 32 + l32;
#pragma unroll
        for (int kk = 0; kk < DK; ++kk) {
          const uint8_t *src = &Ks[r * RB + k_unit<DT, D, BLK>(r, kk * 2 + half) * LB];
          if constexpr (DT == kFP8) {
            i32x8 a;
            __builtin_memcpy(&a, src, 32);
            s[kt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[kk], s[kt], 0, 0, 0, 127,
                                                                    0, 127);
          } else {
            bf16x8 a;
            __builtin_memcpy(&a, src, 16);
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[kt], 0, 0, 0);
          }
        }
      }
      // ---- online softmax, log2 domain.  Element r of tile kt is key
      //      j0 + kt*32 + (r/4)*8 + half*4 + r%4 for query qi.
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kt][r] * scale2;
          if (diag) {
            const int key = j0 + kt * 32 + (r / 4) * 8 + half * 4 + (r % 4);
            if (key > qi) x = -INFINITY;
          }
          s[kt][r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(m, mx);
      const float msub = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2f(m - msub);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DTL; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m = mnew;
      bf16x8 pb[KTS][2];
#pragma unroll
      for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int s8 = 0; s8 < 8; ++s8) {
            const float p = exp2f(s[kt][st * 8 + s8] - msub);
            l += p;
            pb[kt][st][s8] = (__bf16)p;
          }
      // ---- O^T += V^T P^T.  Step (kt, st) covers keys kt*32 + st*16 + [0,16);
      //      operand slot s of lane half `half` is key
      //      kt*32 + st*16 + (s/4)*8 + half*4 + s%4 on both operands.
      const int grp = lane >> 4, gi = lane & 15;
      const int rr = gi >> 2, ss = gi & 3;
#pragma unroll
      for (int db = 0; db < DTL; ++db) {
        const int dcol = db * 32 + (grp & 1) * 16 + ss * 4;
#pragma unroll
        for (int kt = 0; kt < KTS; ++kt)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int r0 = kt * 32 + st * 16 + (grp >> 1) * 4 + rr;
            const int r1 = r0 + 8;
            const uint16_t *p0 = &Vs[r0 * D + v_chunk<D>(r0, dcol >> 3) * 8 + (dcol & 7)];
            const uint16_t *p1 = &Vs[r1 * D + v_chunk<D>(r1, dcol >> 3) * 8 + (dcol & 7)];
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p1);
            const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kt][st], oacc[db], 0, 0, 0);
          }
      }
    }
  }

  const float lt = l + __shfl_xor(l, 32, 64);
  if (qi < seq) {
    float inv = lt > 0.f ? 1.f / lt : 0.f;
    if constexpr (DT == kFP8) inv *= v_scale[g];
    uint16_t *orow = o + ((size_t)h * seq + qi) * D;
#pragma unroll
    for (int db = 0; db < DTL; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = db * 32 + gq * 8 + half * 4;
        uint2 pk;
        pk.x = f32_to_bf16_bits(oacc[db][gq * 4 + 0] * inv) |
               (f32_to_bf16_bits(oacc[db][gq * 4 + 1] * inv) << 16);
        pk.y = f32_to_bf16_bits(oacc[db][gq * 4 + 2] * inv) |
               (f32_to_bf16_bits(oacc[db][gq * 4 + 3] * inv) << 16);
        *(uint2 *)(orow + d0) = pk;
      }
    if (lse && half == 0)
      lse[(size_t)h * seq + qi] = lt > 0.f ? (m + log2f(lt)) * kLn2 : -INFINITY;
  }
  (void)ES;
}

template <int DT, int D, int BLK>
static hipError_t launch_t(const Shape &s, const AttnArgs &a, hipStream_t st) {
  hipLaunchKernelGGL((attn_mfma_kernel<DT, D, BLK>), dim3(s.hq * s.nb), dim3(BLK * 2), 0, st,
                     (const uint8_t *)a.q, (const uint8_t *)a.k, (const uint8_t *)a.v, a.kv_idx,
                     a.kv_cnt, (uint16_t *)a.o, a.lse, a.q_scale, a.k_scale, a.v_scale, s.hq,
                     s.hkv, s.seq, s.nb, a.sm_scale * kLog2e);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_dt(const Shape &s, const AttnArgs &a, hipStream_t st) {
  if (s.d == 64 && s.block == 64) return launch_t<DT, 64, 64>(s, a, st);
  if (s.d == 64 && s.block == 128) return launch_t<DT, 64, 128>(s, a, st);
  if (s.d == 128 && s.block == 64) return launch_t<DT, 128, 64>(s, a, st);
  return launch_t<DT, 128, 128>(s, a, st);
}

hipError_t launch_attn_bf16(const Shape &s, const AttnArgs &a, hipStream_t st) {
  return launch_dt<kBF16>(s, a, st);
}

hipError_t launch_attn_fp8(const Shape &s, const AttnArgs &a, hipStream_t st) {
  return launch_dt<kFP8>(s, a, st);
}

}  // namespace bsp
