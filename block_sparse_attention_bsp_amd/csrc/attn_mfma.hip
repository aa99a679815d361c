// Stage 3 for bf16 and fp8 inputs: block-sparse causal attention on MFMA
// (FlashPrefill summary page, Appendix B "Block Sparse Attention": only the
// selected key blocks are visited, causal masking is applied where required -
// here only on the diagonal block - with online softmax updates and a final
// normalisation).  fp8 inputs follow the FP8 inference of the FlashPrefill V2
// abstract (thelatestinai.com page): e4m3 operands, fp32 accumulation.
//
// gfx950 design
//   * One workgroup per (q head, query block I): B/32 wavefronts, each owning
//     32 queries whose Q fragments stay in registers for the whole row.  Two
//     workgroups share a CU (2 waves per SIMD) so one wave's MFMAs overlap the
//     other's softmax.
//   * Workgroups are numbered heaviest row first and, when the kv heads divide
//     the 8 XCDs evenly, every XCD serves whole GQA groups: the 64 workgroups
//     resident on an XCD walk the same K/V blocks in the same order, so K/V
//     come from that XCD's L2.  When the K/V of all groups would overflow
//     the memory-side cache, the groups go in phases of fewer at a time, so
//     blocks that miss L2 (scattered kept blocks) are served from it.
//   * Scores are computed transposed in 16x16 tiles, S^T = K Q^T
//     (v_mfma_f32_16x16x32_bf16, or one v_mfma_scale_f32_16x16x128_f8f6f4
//     with unit scales per tile for e4m3).  Lane 16g + r owns query r of each
//     of the wave's two 16-query tiles and keys 4g .. 4g+3 of every 16-key
//     tile, so everything on the common path stays in-lane; a query's four
//     lanes meet only to rescale and at the end.
//   * The output is accumulated transposed, O^T += V^T P^T (16x16x32 bf16):
//     every accumulator of a lane belongs to one of its two queries.  P^T is
//     the B operand straight from the score registers (slots 0-3 and 4-7 are
//     the lane's rows of two consecutive key tiles); the V^T operand reads the
//     same keys with two ds_read_b64_tr_b16, whose 4x16 transpose yields it.
//   * K/V sub-tiles of 64 keys are double-buffered in LDS and filled one
//     sub-tile ahead by buffer_load_dwordx4 ... lds (no VGPR staging; one
//     buffer descriptor per kv head, the sub-tile position as the scalar
//     offset, loop-invariant lane offsets), so the load of sub-tile i+1
//     overlaps the MFMAs of sub-tile i; one barrier per sub-tile.  K rows
//     carry an XOR swizzle of their read units; V is stored row-major bf16
//     (fp8 codes are widened exactly on the way in).
//   * Softmax in fp32, exp2 domain with log2(e) and (fp8) the q/k scales in
//     one factor; the exponent is one FMA against a reference max per query
//     that moves only when a lane's partial sum of probabilities passes 2^8
//     (then the query's max over the sub-tile is taken, the output rescaled
//     and P recomputed), so the common path has no max reduction at all.

#include <type_traits>

#include "attn_common.h"

namespace bsp {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// The accumulators are rescaled only when a lane's partial sum of
// probabilities for a sub-tile exceeds this bound, so every probability stays
// at or below 2^8, well inside bf16 and fp32.
constexpr float kRescaleBound = 256.0f;

template <int DT, int D, int BLK>
struct AttnCfg {
  static constexpr int ES = DT == kFP8 ? 1 : 2;  // bytes per Q/K element
  static constexpr int RB = D * ES;              // bytes per K row
  // S^T MFMA: 16x16x32 bf16 (16 bytes per lane per step), or one
  // 16x16x128 f8f6f4 per tile for e4m3 (32 bytes per lane; d = 64 fills
  // half of it and zeroes the rest).
  static constexpr int LB = DT == kFP8 ? (D == 128 ? 32 : 16) : 16;  // bytes read per lane per step
  static constexpr int CPU = LB / 16;            // 16-byte chunks per read unit
  static constexpr int DK = DT == kFP8 ? 1 : D / 32;  // S^T k-steps
  static constexpr int UNITS = RB / LB;          // read units per K row
  static constexpr int KRPW = RB >= 256 ? 1 : 256 / RB;  // K rows per 256-byte window
  static constexpr int NW = BLK / 32;            // wavefronts: 32 queries each
  static constexpr int NT = NW * 64;
  static constexpr int KT = 64;                  // keys per LDS sub-tile
  static constexpr int NSUB = BLK / KT;
  static constexpr int NKT = KT / 16;            // 16-key S^T tiles per sub-tile
  static constexpr int NJ = KT / 32;             // 32-key PV steps per sub-tile
  static constexpr int NDT = D / 16;             // 16-wide d tiles of O^T
  static constexpr int KBYTES = KT * RB;         // K sub-tile bytes
  static constexpr int VBYTES = KT * D * 2;      // V sub-tile bytes (bf16)
  static constexpr int KCH = KBYTES / 16;        // 16-byte chunks per K sub-tile
  static constexpr int VCHK = KT * RB / 16;      // 16-byte global chunks per V sub-tile
};

template <int DT, int D, int BLK>
__device__ __forceinline__ int k_unit(int r, int u) {
  using C = AttnCfg<DT, D, BLK>;
  return u ^ ((r / C::KRPW) % C::UNITS);
}

// e4m3 with d = 128: a read unit is two 16-byte chunks, read by two
// ds_read_b128 of 16 rows each.  Rows 8-15 of every 16 keep the chunks of a
// unit in swapped order, so that each read's 16 lanes land on 16 distinct
// 16-byte bank groups (the unit swizzle alone covers only the even or only
// the odd ones, and rows r and r + 8 collided).
template <int DT, int D, int BLK>
__device__ __forceinline__ int k_half(int r) {
  using C = AttnCfg<DT, D, BLK>;
  return C::CPU == 2 ? (r >> 3) & 1 : 0;
}

// V rows are stored in 16-byte chunks whose index is XORed with a function
// of the row that moves whole 32-byte pairs, so that the rows one
// ds_read_b64_tr_b16 reads together (32 bytes from each of 4 rows per 16
// lanes, 8 rows per 32 lanes) land on distinct banks: 128 B per 16 lanes
// and 256 B per 32 lanes, no bank taken twice (measured with the LDS
// bank-conflict counter).  Depends on the row modulo 8 only, so per-lane
// offsets are loop constants.
template <int D>
__device__ __forceinline__ int v_chunk(int r, int c) {
  if constexpr (D >= 128) return c ^ ((r & 7) << 1);
  return c ^ ((((r ^ (r >> 2)) & 1) << 1) | (((r >> 1) & 1) << 2));
}



// V16: V is stored as bf16 (always for bf16; for e4m3 Q/K when the caller
// passes V already widened), so it reaches LDS by the same direct loads as K.
template <int DT, int D, int BLK, bool V16>
struct Attn {
  static_assert(DT == kFP8 || V16, "bf16 inputs store V as bf16");
  using C = AttnCfg<DT, D, BLK>;
  static constexpr int RB = C::RB, LB = C::LB, DK = C::DK, KT = C::KT;
  static constexpr int NKT = C::NKT, NJ = C::NJ, NDT = C::NDT, NSUB = C::NSUB, NW = C::NW,
                       NT = C::NT;
  static constexpr int KPW = C::KCH / NW;               // K DMA chunks per wave
  static constexpr int VPW = (C::VBYTES / 16) / NW;     // V DMA chunks per wave (bf16)
  static constexpr int VPER = C::VCHK / NT > 0 ? C::VCHK / NT : 1;  // e4m3 V chunks per thread
  typedef typename std::conditional<DT == kFP8, i32x8, bf16x8>::type frag_t;

  const uint8_t *k, *v;
  __amdgpu_buffer_rsrc_t krs, vrs;  // this kv head's K and V
  // lane = 16 * g + r: in every 16x16 tile the lane owns column r (a query)
  // and rows 4g .. 4g + 3 (keys of S^T, dimensions of O^T)
  int seq, I, w, lane, g, r16;
  int qi[2];      // the lane's two queries (query tiles 0 and 1 of the wave)
  size_t kvrow0;  // kv head * seq
  float scale2;
  frag_t qf[2][DK];
  f32x4 oacc[NDT][2];
  float m_used[2], l[2];
  // per-lane byte offsets (loop constants)
  uint32_t kdma[KPW / 64], vdma[V16 ? VPW / 64 : 1];
  int krow[KPW / 64], vrow[V16 ? VPW / 64 : 1];
  int koff[DK], voff[NDT];
  int khalf;  // e4m3, d = 128: byte offset of a unit's first chunk (0 or 16)
  uint4 vreg[V16 ? 1 : VPER];

  __device__ __forceinline__ void setup() {
#pragma unroll
    for (int it = 0; it < KPW / 64; ++it) {
      const int p = w * KPW + it * 64 + lane;
      const int r = p / (RB / 16), pc = p % (RB / 16);
      const int c = k_unit<DT, D, BLK>(r, pc / C::CPU) * C::CPU + ((pc % C::CPU) ^ k_half<DT, D, BLK>(r));
      kdma[it] = r * RB + c * 16;
      krow[it] = r;
    }
    if constexpr (V16) {
#pragma unroll
      for (int it = 0; it < VPW / 64; ++it) {
        const int p = w * VPW + it * 64 + lane;
        const int r = p / (D / 8), pc = p % (D / 8);
        vdma[it] = r * (D * 2) + v_chunk<D>(r, pc) * 16;  // the swizzle is an involution
        vrow[it] = r;
      }
    }
    // K (A operand): key row r16 of a tile, read unit ks * 4 + g (bf16) or g (fp8)
#pragma unroll
    for (int ks = 0; ks < DK; ++ks)
      koff[ks] = r16 * RB + k_unit<DT, D, BLK>(r16, (DT == kFP8 ? 0 : ks * 4) + g) * LB;
    khalf = k_half<DT, D, BLK>(r16) * 16;
    // V^T (A operand) via ds_read_b64_tr_b16: in lane group g, lane r16 supplies
    // row 4g + r16 / 4 (a key) and columns 4 (r16 % 4) .. + 3 of a 16-wide d
    // tile dt.
    const int vr = 4 * g + (r16 >> 2), vq = r16 & 3;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int dcol = dt * 16 + vq * 4;
      voff[dt] = vr * (D * 2) + v_chunk<D>(vr, dcol >> 3) * 16 + (dcol & 7) * 2;
    }
  }

  // Rows [r0, r0 + KT) of a K/V region -> LDS buffers, issued one sub-tile
  // ahead.  kr / vr describe the region (one kv head's sequence, or one cache
  // page), vb is its V base for e4m3 V, lim the number of valid rows in it.
  // K (and bf16 V) go straight to LDS; e4m3 V comes back in registers for
  // widening.
  __device__ __forceinline__ void issue_rows(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                             const uint8_t *vb, int r0, int lim, uint8_t *Kb,
                                             uint16_t *Vb) {
    const uint32_t ksoff = (uint32_t)r0 * RB, vsoff = (uint32_t)r0 * (D * 2);
    if (r0 + KT <= lim) {
#pragma unroll
      for (int it = 0; it < KPW / 64; ++it) lds_dma16(kr, kdma[it], ksoff, Kb + (w * KPW + it * 64) * 16);
      if constexpr (V16) {
#pragma unroll
        for (int it = 0; it < VPW / 64; ++it)
          lds_dma16(vr, vdma[it], vsoff, (uint8_t *)Vb + (w * VPW + it * 64) * 16);
      }
    } else {
      // ragged last block: rows past the end re-read the last valid row
      // (finite data whose keys are masked as causal-future for every query)
#pragma unroll
      for (int it = 0; it < KPW / 64; ++it)
        lds_dma16(kr, kdma[it] - (uint32_t)max(0, r0 + krow[it] - (lim - 1)) * RB, ksoff,
                  Kb + (w * KPW + it * 64) * 16);
      if constexpr (V16) {
#pragma unroll
        for (int it = 0; it < VPW / 64; ++it)
          lds_dma16(vr, vdma[it] - (uint32_t)max(0, r0 + vrow[it] - (lim - 1)) * (D * 2), vsoff,
                    (uint8_t *)Vb + (w * VPW + it * 64) * 16);
      }
    }
    if constexpr (!V16) {
#pragma unroll
      for (int it = 0; it < VPER; ++it) {
        const int e = threadIdx.x + it * NT;
        const int r = e / (RB / 16), c = e % (RB / 16);
        const int jr = min(r0 + r, lim - 1);
        vreg[it] = *(const uint4 *)(vb + (size_t)jr * RB + c * 16);
      }
    }
  }

  // Sub-tile (J, sub) of this kv head's contiguous K/V
  __device__ __forceinline__ void issue(int J, int sub, uint8_t *Kb, uint16_t *Vb) {
    issue_rows(krs, vrs, v + kvrow0 * (V16 ? D * 2 : RB), J * BLK + sub * KT, seq, Kb, Vb);
  }

  // e4m3 V only: widen the prefetched V codes to bf16 into the LDS buffer.
  __device__ __forceinline__ void store_v(uint16_t *Vb) {
    if constexpr (!V16) {
#pragma unroll
      for (int it = 0; it < VPER; ++it) {
        const int e = threadIdx.x + it * NT;
        const int r = e / (RB / 16), c = e % (RB / 16);
        const uint4 vv4 = vreg[it];
        const uint4 lo = make_uint4(e4m3x2_to_bf16x2(vv4.x, false), e4m3x2_to_bf16x2(vv4.x, true),
                                    e4m3x2_to_bf16x2(vv4.y, false), e4m3x2_to_bf16x2(vv4.y, true));
        const uint4 hi = make_uint4(e4m3x2_to_bf16x2(vv4.z, false), e4m3x2_to_bf16x2(vv4.z, true),
                                    e4m3x2_to_bf16x2(vv4.w, false), e4m3x2_to_bf16x2(vv4.w, true));
        *(uint4 *)&Vb[r * D + v_chunk<D>(r, 2 * c) * 8] = lo;
        *(uint4 *)&Vb[r * D + v_chunk<D>(r, 2 * c + 1) * 8] = hi;
      }
    }
  }

  __device__ __forceinline__ void mask_diag(f32x4 (&s)[NKT][2], int j0) {
    // Element e of tile (kt, qt) is key j0 + kt*16 + 4g + e of query qi[qt].
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (j0 + kt * 16 + 4 * g + e > qi[qt]) s[kt][qt][e] = -INFINITY;
  }

  __device__ __forceinline__ void load_k(frag_t (&a)[NKT], const uint8_t *__restrict__ Kb, int ks) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      if constexpr (DT == kFP8 && LB == 16) {
        uint4 lo;
        __builtin_memcpy(&lo, Kb + koff[ks] + kt * 16 * RB, 16);
        const uint4 ab[2] = {lo, make_uint4(0, 0, 0, 0)};
        __builtin_memcpy(&a[kt], ab, 32);
      } else {
        if constexpr (C::CPU == 2) {
          const uint8_t *u = Kb + koff[ks] + kt * 16 * RB;
          uint4 h[2];
          __builtin_memcpy(&h[0], u + khalf, 16);
          __builtin_memcpy(&h[1], u + (16 - khalf), 16);
          __builtin_memcpy(&a[kt], h, 32);
        } else {
          __builtin_memcpy(&a[kt], Kb + koff[ks] + kt * 16 * RB, sizeof(frag_t));
        }
      }
    }
  }

  // V^T fragment of d tile dt for PV step j: keys j*32 + 4g + [0,4) and
  // j*32 + 16 + 4g + [0,4), matching the P^T slots of the lane.
  __device__ __forceinline__ bf16x8 load_v(const uint16_t *__restrict__ Vb, int j, int dt) {
    const uint8_t *p0 = (const uint8_t *)Vb + voff[dt] + j * 32 * (D * 2);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p0);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p0 + 16 * D * 2));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }

  __device__ __forceinline__ f32x4 mma_qk(const frag_t &a, const frag_t &b, f32x4 c) {
    if constexpr (DT == kFP8)
      return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
    else
      return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }

  // One 64-key sub-tile from LDS.  LDS fragments are double-buffered in
  // registers one MFMA group ahead; scheduling barriers keep that order.
  // kfirst: the first K fragments, when the caller has already read them.
  __device__ __forceinline__ void compute(const uint8_t *__restrict__ Kb,
                                          const uint16_t *__restrict__ Vb, int j0, bool diag,
                                          const frag_t *kfirst) {
    // ---- S^T = K Q^T: NKT key tiles x 2 query tiles, 16x16 each
    f32x4 s[NKT][2];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) s[kt][0] = s[kt][1] = f32x4{};
    frag_t ka[2][NKT];
    if (kfirst) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) ka[0][kt] = kfirst[kt];
    } else {
      load_k(ka[0], Kb, 0);
    }
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      if (ks + 1 < DK) load_k(ka[(ks + 1) & 1], Kb, ks + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) s[kt][qt] = mma_qk(ka[ks & 1][kt], qf[qt][ks], s[kt][qt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // From here to the end of the sub-tile (softmax and PV) the wave runs at
    // raised priority: a SIMD's other wave fills the gaps with its S^T MFMAs.
    __builtin_amdgcn_s_setprio(1);
    // V^T fragments: a ring of four, three PV MFMA pairs ahead; the first
    // three load while the softmax runs
    constexpr int NV = NJ * NDT;
    bf16x8 va[4];
#pragma unroll
    for (int n = 0; n < 3 && n < NV; ++n) va[n] = load_v(Vb, n / NDT, n % NDT);
    if (diag) mask_diag(s, j0);
    // ---- P = exp2(s * scale2 - m) against a reference max m per query,
    //      packed to bf16 for the MFMA; the row sums take the fp32 values.
    //      Slot e of P^T step j for query tile qt: key tile 2j + e/4, row e%4.
    bf16x8 pb[NJ][2];
    float ps[2];
    auto exps = [&]() {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float mneg = m_used[qt] == -INFINITY ? 0.f : -m_used[qt];
        float a0, a1;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][e], scale2, mneg));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][e + 1], scale2, mneg));
            a0 = (kt == 0 && e == 0) ? p0 : a0 + p0;
            a1 = (kt == 0 && e == 0) ? p1 : a1 + p1;
            pb[kt / 2][qt][(kt % 2) * 4 + e] = (__bf16)p0;
            pb[kt / 2][qt][(kt % 2) * 4 + e + 1] = (__bf16)p1;
          }
        ps[qt] = a0 + a1;
      }
    };
    exps();
    // ---- The reference max moves only when needed: when a lane's partial
    //      sum for a query exceeds kRescaleBound = 2^8 (which bounds every
    //      term of it), or while a query has no reference yet.  Then the
    //      query's max over the sub-tile is taken across the four lanes that
    //      hold it, the output is rescaled and P recomputed.
    if (__any(!(ps[0] <= kRescaleBound) || !(ps[1] <= kRescaleBound) ||
              m_used[0] == -INFINITY || m_used[1] == -INFINITY)) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
          mx = fmaxf(fmaxf(mx, fmaxf(s[kt][qt][0], s[kt][qt][1])), fmaxf(s[kt][qt][2], s[kt][qt][3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(m_used[qt], mx * scale2);
        const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_used[qt] - mnew);
        l[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) oacc[dt][qt] *= alpha;
        m_used[qt] = mnew;
      }
      exps();
    }
    l[0] += ps[0];
    l[1] += ps[1];
    // ---- O^T += V^T P^T: d tiles x 2 query tiles, 32 keys per step
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int n = j * NDT + dt;
        if (n + 3 < NV) va[(n + 3) & 3] = load_v(Vb, (n + 3) / NDT, (n + 3) % NDT);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
          oacc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[n & 3], pb[j][qt], oacc[dt][qt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    __builtin_amdgcn_s_setprio(0);
  }
};

template <int DT, int D, int BLK, bool VL, bool V16>
__global__ __launch_bounds__(BLK * 2, (BLK == 64 && D == 128) ? 1 : 2) void attn_mfma_kernel(
    const uint8_t *__restrict__ q, const uint8_t *__restrict__ k, const uint8_t *__restrict__ v,
    const int32_t *__restrict__ kv_idx, const int32_t *__restrict__ kv_cnt,
    uint16_t *__restrict__ o, float *__restrict__ lse, const float *__restrict__ q_scale,
    const float *__restrict__ k_scale, const float *__restrict__ v_scale, int hq, int hkv,
    int seq, int nb, float sm_scale_log2, int xcd_map, VarlenArgs vl) {
  using A = Attn<DT, D, BLK, V16>;
  using C = typename A::C;
  constexpr int RB = C::RB, LB = C::LB, DK = C::DK, KT = C::KT, NSUB = C::NSUB;
  __shared__ __attribute__((aligned(16))) uint8_t Ks0[C::KBYTES];
  __shared__ __attribute__((aligned(16))) uint8_t Ks1[C::KBYTES];
  __shared__ __attribute__((aligned(16))) uint16_t Vs0[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs1[KT * D];

  A T;
  const int tid = threadIdx.x;
  T.lane = tid & 63;
  T.w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar LDS bases
  T.g = T.lane >> 4;
  T.r16 = T.lane & 15;
  const int grp = hq / hkv;
  int I, h;
  attn_row_of(blockIdx.x, xcd_map, hq, hkv, nb, I, h);
  const int g = h / grp;
  // token rows of q / o / lse: ntok per head, this sequence from tok0; len
  // tokens in this sequence; the kv list row gb and its stride
  const int ntok = seq;
  const AttnRow R = attn_locate<VL>(I, seq, nb, vl);
  I = R.I;
  const int len = R.len, tok0 = R.tok0, gb = R.gb, stride = R.stride;
  const int32_t *ptab = R.ptab;
  T.I = I;
  T.seq = len;
  T.k = k;
  T.v = v;
  T.kvrow0 = (size_t)g * seq;
  if constexpr (!VL) {
    T.krs = make_rsrc(k + T.kvrow0 * RB, (uint32_t)seq * RB);
    T.vrs = make_rsrc(v + T.kvrow0 * (V16 ? D * 2 : RB), (uint32_t)seq * (V16 ? D * 2 : RB));
  }
  // key block J -> LDS, through the page table for VL
  constexpr int VRB = V16 ? D * 2 : RB;  // bytes per V row in memory
  auto issue_block = [&](int J, int sub, uint8_t *Kb, uint16_t *Vb) {
    if constexpr (VL) {
      const size_t slab = ((size_t)ptab[J] * hkv + g) * BLK;
      T.issue_rows(make_rsrc(k + slab * RB, BLK * RB), make_rsrc(v + slab * VRB, BLK * VRB),
                   v + slab * VRB, sub * KT, min(BLK, len - J * BLK), Kb, Vb);
    } else {
      T.issue(J, sub, Kb, Vb);
    }
  };
  T.qi[0] = I * BLK + T.w * 32 + T.r16;
  T.qi[1] = T.qi[0] + 16;
  const size_t row = (size_t)h * nb + gb;  // kv list row (gb == I unless VL)
  T.scale2 = sm_scale_log2;
  if constexpr (DT == kFP8) T.scale2 *= q_scale[h] * k_scale[g];
  T.setup();

  // Q fragments: B operand of S^T = K Q^T.  Lane (g, r16) holds query
  // qi[qt], dimensions ks*32 + 8g .. + 8 (bf16) or LB bytes at g*LB (fp8).
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qq = T.qi[qt];
#pragma unroll
    for (int ks = 0; ks < DK; ++ks) {
      const uint8_t *src = q + ((size_t)h * ntok + tok0 + min(qq, len - 1)) * RB +
                           (DT == kFP8 ? T.g * LB : (ks * 32 + 8 * T.g) * 2);
      uint4 a = *(const uint4 *)src, b = make_uint4(0, 0, 0, 0);
      if constexpr (LB == 32) b = *(const uint4 *)(src + 16);
      if (qq >= len) a = b = make_uint4(0, 0, 0, 0);
      if constexpr (DT == kFP8) {
        const uint4 ab[2] = {a, b};
        __builtin_memcpy(&T.qf[qt][ks], ab, 32);
      } else {
        __builtin_memcpy(&T.qf[qt][ks], &a, 16);
      }
    }
  }
#pragma unroll
  for (int dt = 0; dt < C::NDT; ++dt) T.oacc[dt][0] = T.oacc[dt][1] = f32x4{};
  T.m_used[0] = T.m_used[1] = -INFINITY;
  T.l[0] = T.l[1] = 0.f;

  const int nblk = kv_idx ? max(0, min(kv_cnt[row], stride)) : I + 1;
  const int ns = nblk * NSUB;
  KvStream kv;
  kv.init(kv_idx ? kv_idx + row * stride : nullptr, nblk, I, T.lane);
  auto block_of = [&](int t) { return kv.block_of(t); };

  // Pipeline: step i waits for sub-tile i (issued one step earlier), passes a
  // barrier, issues sub-tile i+1 into the other buffer and computes i.
  int Jc = ns > 0 ? block_of(0) : -1;
  if (Jc >= 0) {
    issue_block(Jc, 0, Ks0, Vs0);
    if constexpr (!V16) T.store_v(Vs0);
  }
  for (int i = 0; i < ns; i += 2) {
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      const int ii = i + ph;
      if (ii < ns) {
        const int Jn = ii + 1 < ns ? block_of((ii + 1) / NSUB) : -1;
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // fp8: the sub-tile's first K fragments are read before the next
        // sub-tile's loads are issued, which hides their LDS latency behind
        // the issue (2-4% faster for e4m3; no gain for bf16)
        typename A::frag_t kf[C::NKT];
        if (DT == kFP8 && Jc >= 0) T.load_k(kf, ph ? Ks1 : Ks0, 0);
        if (Jn >= 0) issue_block(Jn, (ii + 1) % NSUB, ph ? Ks0 : Ks1, ph ? Vs0 : Vs1);
        if (Jc >= 0)
          T.compute(ph ? Ks1 : Ks0, ph ? Vs1 : Vs0, Jc * BLK + (ii % NSUB) * KT, Jc == I,
                    DT == kFP8 ? kf : nullptr);
        if constexpr (!V16) {
          if (Jn >= 0) T.store_v(ph ? Vs0 : Vs1);
        }
        Jc = Jn;
      }
    }
  }

  // each query's row sum is split over the four lanes 16 apart
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float lt = T.l[qt];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int qq = T.qi[qt];
    if (qq < len) {
      float inv = lt > 0.f ? 1.f / lt : 0.f;
      if constexpr (DT == kFP8) inv *= v_scale[g];
      uint16_t *orow = o + ((size_t)h * ntok + tok0 + qq) * D;
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt) {
        uint2 pk;
        pk.x = f32_to_bf16_bits(T.oacc[dt][qt][0] * inv) |
               (f32_to_bf16_bits(T.oacc[dt][qt][1] * inv) << 16);
        pk.y = f32_to_bf16_bits(T.oacc[dt][qt][2] * inv) |
               (f32_to_bf16_bits(T.oacc[dt][qt][3] * inv) << 16);
        *(uint2 *)(orow + dt * 16 + 4 * T.g) = pk;
      }
      if (lse && T.g == 0)
        lse[(size_t)h * ntok + tok0 + qq] = lt > 0.f ? (T.m_used[qt] + log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

// kv bytes of one group, for the phase decision: K, and V at its stored width
template <int DT, int D, bool V16>
constexpr long kv_row_bytes() {
  return (long)D * ((DT == kFP8 ? 1 : 2) + (V16 ? 2 : (DT == kFP8 ? 1 : 2)));
}

template <int DT, int D, int BLK, bool V16>
static hipError_t launch_t(const Shape &s, const AttnArgs &a, hipStream_t st) {
  const long items = (long)s.hq * s.nb;
  const int xcd = attn_xcd_mode(s, (long)s.seq * kv_row_bytes<DT, D, V16>());
  hipLaunchKernelGGL((attn_mfma_kernel<DT, D, BLK, false, V16>), dim3((unsigned)items),
                     dim3(BLK * 2), 0, st, (const uint8_t *)a.q, (const uint8_t *)a.k,
                     (const uint8_t *)a.v, a.kv_idx, a.kv_cnt, (uint16_t *)a.o, a.lse, a.q_scale,
                     a.k_scale, a.v_scale, s.hq, s.hkv, s.seq, s.nb, a.sm_scale * kLog2e, xcd,
                     VarlenArgs{});
  return hipGetLastError();
}

// Varlen: s.seq = tokens in the packed batch, s.nb = query blocks in it.
template <int DT, int D, int BLK, bool V16>
static hipError_t launch_vl_t(const Shape &s, const AttnArgs &a, const VarlenArgs &v,
                              hipStream_t st) {
  const long items = (long)s.hq * s.nb;
  // a row reads only its own sequence's pages: all groups at once
  const int xcd = attn_xcd_mode(s, 0);
  hipLaunchKernelGGL((attn_mfma_kernel<DT, D, BLK, true, V16>), dim3((unsigned)items),
                     dim3(BLK * 2), 0, st, (const uint8_t *)a.q, (const uint8_t *)a.k,
                     (const uint8_t *)a.v, a.kv_idx, a.kv_cnt, (uint16_t *)a.o, a.lse, a.q_scale,
                     a.k_scale, a.v_scale, s.hq, s.hkv, s.seq, s.nb, a.sm_scale * kLog2e, xcd, v);
  return hipGetLastError();
}

template <int DT, bool V16>
static hipError_t launch_dt(const Shape &s, const AttnArgs &a, hipStream_t st) {
  if (s.d == 64 && s.block == 64) return launch_t<DT, 64, 64, V16>(s, a, st);
  if (s.d == 64 && s.block == 128) return launch_t<DT, 64, 128, V16>(s, a, st);
  if (s.d == 128 && s.block == 64) return launch_t<DT, 128, 64, V16>(s, a, st);
  return launch_t<DT, 128, 128, V16>(s, a, st);
}

template <int DT, bool V16>
static hipError_t launch_vl_dt(const Shape &s, const AttnArgs &a, const VarlenArgs &v,
                               hipStream_t st) {
  if (s.d == 64 && s.block == 64) return launch_vl_t<DT, 64, 64, V16>(s, a, v, st);
  if (s.d == 64 && s.block == 128) return launch_vl_t<DT, 64, 128, V16>(s, a, v, st);
  if (s.d == 128 && s.block == 64) return launch_vl_t<DT, 128, 64, V16>(s, a, v, st);
  return launch_vl_t<DT, 128, 128, V16>(s, a, v, st);
}

hipError_t launch_attn_bf16(const Shape &s, const AttnArgs &a, hipStream_t st) {
  return launch_dt<kBF16, true>(s, a, st);
}

hipError_t launch_attn_fp8(const Shape &s, const AttnArgs &a, hipStream_t st) {
  if (s.dtype == kFP8V16) return launch_dt<kFP8, true>(s, a, st);
  return launch_dt<kFP8, false>(s, a, st);
}

hipError_t launch_attn_varlen(const Shape &s, const AttnArgs &a, const VarlenArgs &v,
                              hipStream_t st) {
  if (s.dtype == kBF16) return launch_vl_dt<kBF16, true>(s, a, v, st);
  if (s.dtype == kFP8V16) return launch_vl_dt<kFP8, true>(s, a, v, st);
  return launch_vl_dt<kFP8, false>(s, a, v, st);
}

}  // namespace bsp
