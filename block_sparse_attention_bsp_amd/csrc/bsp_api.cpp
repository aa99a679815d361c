// C-ABI host layer of libbsp: argument checks on the host, then kernel
// launches on the caller's stream.  No allocation, no synchronisation, no
// global state.  The operations are defined in include/bsp.h.
#include <math.h>

#include "bsp.h"
#include "internal.h"

namespace {

using bsp::Shape;

bsp_status check_desc(const bsp_desc *d, bool need_dtype) {
  if (!d) return BSP_ERR_NULL_POINTER;
  if (d->hq < 1 || d->hq > BSP_MAX_HEADS || d->hkv < 1 || d->hkv > d->hq || d->hq % d->hkv)
    return BSP_ERR_BAD_SHAPE;
  if (d->seq < 0 || d->seq > BSP_MAX_SEQ) return BSP_ERR_BAD_SHAPE;
  if (d->d != 64 && d->d != 128) return BSP_ERR_BAD_SHAPE;
  if (d->block != 64 && d->block != 128) return BSP_ERR_BAD_SHAPE;
  if (d->causal != 1) return BSP_ERR_UNSUPPORTED;
  if (need_dtype) {
    if (d->dtype != BSP_DTYPE_F32 && d->dtype != BSP_DTYPE_BF16 && d->dtype != BSP_DTYPE_FP8_E4M3 &&
        d->dtype != BSP_DTYPE_FP8_E4M3_V_BF16)
      return BSP_ERR_BAD_DTYPE;
  }
  if (!isfinite(d->sm_scale)) return BSP_ERR_BAD_VALUE;
  return BSP_OK;
}

Shape shape_of(const bsp_desc *d) {
  Shape s;
  s.hq = d->hq;
  s.hkv = d->hkv;
  s.seq = d->seq;
  s.d = d->d;
  s.block = d->block;
  s.nb = (d->seq + d->block - 1) / d->block;
  s.dtype = d->dtype;
  return s;
}

float scale_of(const bsp_desc *d) {
  return d->sm_scale > 0.f ? d->sm_scale : 1.0f / sqrtf((float)d->d);
}

bsp_status hip_status(hipError_t e) { return e == hipSuccess ? BSP_OK : BSP_ERR_HIP; }

// Q and K in e4m3 codes with per-head scales (V's storage aside)
bool fp8_qk(const bsp_desc *d) {
  return d->dtype == BSP_DTYPE_FP8_E4M3 || d->dtype == BSP_DTYPE_FP8_E4M3_V_BF16;
}

}  // namespace

extern "C" {

bsp_status bsp_score(const bsp_desc *desc, const void *q, const void *k, float *q_pool,
                     float *k_pool, float *score, void *stream) {
  bsp_status st = check_desc(desc, true);
  if (st != BSP_OK) return st;
  if (desc->seq == 0) return BSP_OK;
  if (!q || !k || !q_pool || !k_pool || !score) return BSP_ERR_NULL_POINTER;
  const bool fp8 = fp8_qk(desc);
  if (fp8 && (!desc->q_scale || !desc->k_scale)) return BSP_ERR_BAD_DTYPE;
  if (!fp8 && (desc->q_scale || desc->k_scale || desc->v_scale)) return BSP_ERR_BAD_DTYPE;
  const Shape s = shape_of(desc);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = bsp::launch_pool(s, q, k, desc->q_scale, desc->k_scale, q_pool, k_pool, hs);
  if (e != hipSuccess) return BSP_ERR_HIP;
  return hip_status(bsp::launch_score(s, scale_of(desc), q_pool, k_pool, nullptr, score, hs));
}

bsp_status bsp_score_mask(const bsp_desc *desc, const void *q, const void *k, float *q_pool,
                          float *k_pool, float *score, uint8_t *mask, int32_t *kv_idx,
                          int32_t *kv_cnt, void *stream) {
  bsp_status st = check_desc(desc, true);
  if (st != BSP_OK) return st;
  if (!(desc->gamma >= 0.f && desc->gamma <= 1.f)) return BSP_ERR_BAD_VALUE;  // also NaN
  if (desc->sink_blocks < 0 || desc->local_blocks < 0) return BSP_ERR_BAD_VALUE;
  if (desc->seq == 0) return BSP_OK;
  if (!q || !k || !q_pool || !k_pool || !score || !kv_idx || !kv_cnt) return BSP_ERR_NULL_POINTER;
  const bool fp8 = fp8_qk(desc);
  if (fp8 && (!desc->q_scale || !desc->k_scale)) return BSP_ERR_BAD_DTYPE;
  if (!fp8 && (desc->q_scale || desc->k_scale || desc->v_scale)) return BSP_ERR_BAD_DTYPE;
  const Shape s = shape_of(desc);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = bsp::launch_pool(s, q, k, desc->q_scale, desc->k_scale, q_pool, k_pool, hs);
  if (e != hipSuccess) return BSP_ERR_HIP;
  const bsp::FuseMask fz{desc->gamma, desc->sink_blocks, desc->local_blocks, mask, kv_idx, kv_cnt};
  return hip_status(bsp::launch_score_mask(s, scale_of(desc), q_pool, k_pool, score, fz, hs));
}

bsp_status bsp_score_arith(const bsp_desc *desc, const void *q, const void *k, float *k_pool,
                           float *score, void *stream) {
  bsp_status st = check_desc(desc, true);
  if (st != BSP_OK) return st;
  if (desc->seq == 0) return BSP_OK;
  if (!q || !k || !k_pool || !score) return BSP_ERR_NULL_POINTER;
  const bool fp8 = fp8_qk(desc);
  if (fp8 && (!desc->q_scale || !desc->k_scale)) return BSP_ERR_BAD_DTYPE;
  if (!fp8 && (desc->q_scale || desc->k_scale || desc->v_scale)) return BSP_ERR_BAD_DTYPE;
  Shape s = shape_of(desc);
  hipStream_t hs = (hipStream_t)stream;
  Shape sk = s;
  sk.hq = 0;  // keys only
  if (bsp::launch_pool(sk, nullptr, k, nullptr, desc->k_scale, nullptr, k_pool, hs) != hipSuccess)
    return BSP_ERR_HIP;
  return hip_status(bsp::launch_score_arith(s, scale_of(desc), q, k_pool, score, desc->q_scale, hs));
}

bsp_status bsp_mask(const bsp_desc *desc, const float *score, const uint8_t *user_mask,
                    uint8_t *mask, int32_t *kv_idx, int32_t *kv_cnt, void *stream) {
  bsp_status st = check_desc(desc, false);
  if (st != BSP_OK) return st;
  if (!(desc->gamma >= 0.f && desc->gamma <= 1.f)) return BSP_ERR_BAD_VALUE;  // also NaN
  if (desc->sink_blocks < 0 || desc->local_blocks < 0) return BSP_ERR_BAD_VALUE;
  if (desc->seq == 0) return BSP_OK;
  if ((!score && !user_mask) || !kv_idx || !kv_cnt) return BSP_ERR_NULL_POINTER;
  const Shape s = shape_of(desc);
  return hip_status(bsp::launch_mask(s, desc->gamma, desc->sink_blocks, desc->local_blocks,
                                     user_mask ? nullptr : score, user_mask, mask, kv_idx, kv_cnt,
                                     (hipStream_t)stream));
}

bsp_status bsp_score_rescue(const bsp_desc *desc, const void *k, const float *q_pool,
                            const float *k_pool, float *k_radius, float *rescue, void *stream) {
  bsp_status st = check_desc(desc, true);
  if (st != BSP_OK) return st;
  if (desc->seq == 0) return BSP_OK;
  if (!k || !q_pool || !k_pool || !k_radius || !rescue) return BSP_ERR_NULL_POINTER;
  const bool fp8 = fp8_qk(desc);
  if (fp8 && !desc->k_scale) return BSP_ERR_BAD_DTYPE;
  if (!fp8 && (desc->q_scale || desc->k_scale || desc->v_scale)) return BSP_ERR_BAD_DTYPE;
  const Shape s = shape_of(desc);
  hipStream_t hs = (hipStream_t)stream;
  if (bsp::launch_radius(s, k, desc->k_scale, k_pool, k_radius, hs) != hipSuccess)
    return BSP_ERR_HIP;
  return hip_status(bsp::launch_score(s, scale_of(desc), q_pool, k_pool, k_radius, rescue, hs));
}

bsp_status bsp_mask_dual(const bsp_desc *desc, const float *score, const float *rescue,
                         float gamma_rescue, uint8_t *mask, int32_t *kv_idx, int32_t *kv_cnt,
                         void *stream) {
  bsp_status st = check_desc(desc, false);
  if (st != BSP_OK) return st;
  if (!(desc->gamma >= 0.f && desc->gamma <= 1.f)) return BSP_ERR_BAD_VALUE;
  if (!(gamma_rescue >= 0.f && gamma_rescue <= 1.f)) return BSP_ERR_BAD_VALUE;
  if (desc->sink_blocks < 0 || desc->local_blocks < 0) return BSP_ERR_BAD_VALUE;
  if (desc->seq == 0) return BSP_OK;
  if (!score || !rescue || !kv_idx || !kv_cnt) return BSP_ERR_NULL_POINTER;
  const Shape s = shape_of(desc);
  return hip_status(bsp::launch_mask(s, desc->gamma, desc->sink_blocks, desc->local_blocks, score,
                                     nullptr, mask, kv_idx, kv_cnt, (hipStream_t)stream, rescue,
                                     gamma_rescue));
}

bsp_status bsp_attn_fwd(const bsp_desc *desc, const void *q, const void *k, const void *v,
                        const int32_t *kv_idx, const int32_t *kv_cnt, void *o, float *lse,
                        void *stream) {
  bsp_status st = check_desc(desc, true);
  if (st != BSP_OK) return st;
  if (desc->seq == 0) return BSP_OK;
  if (!q || !k || !v || !o) return BSP_ERR_NULL_POINTER;
  if ((kv_idx == nullptr) != (kv_cnt == nullptr)) return BSP_ERR_NULL_POINTER;
  const bool fp8 = fp8_qk(desc);
  if (fp8 && (!desc->q_scale || !desc->k_scale || !desc->v_scale)) return BSP_ERR_BAD_DTYPE;
  if (!fp8 && (desc->q_scale || desc->k_scale || desc->v_scale)) return BSP_ERR_BAD_DTYPE;
  const Shape s = shape_of(desc);
  bsp::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.q_scale = desc->q_scale;
  a.k_scale = desc->k_scale;
  a.v_scale = desc->v_scale;
  a.o = o;
  a.lse = lse;
  a.sm_scale = scale_of(desc);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e;
  switch (desc->dtype) {
    case BSP_DTYPE_F32: e = bsp::launch_attn_f32(s, a, hs); break;
    case BSP_DTYPE_BF16: e = bsp::launch_attn_bf16(s, a, hs); break;
    default: e = bsp::launch_attn_fp8(s, a, hs); break;
  }
  return hip_status(e);
}

bsp_status bsp_calibrate_gamma(const bsp_desc *desc, const float *score, float target, float tol,
                               uint8_t *mask, int32_t *kv_idx, int32_t *kv_cnt, int32_t *cnt_host,
                               float *gamma_out, float *density_out, void *stream) {
  bsp_status st = check_desc(desc, false);
  if (st != BSP_OK) return st;
  if (!(target > 0.f && target <= 1.f) || !(tol > 0.f && tol < 1.f)) return BSP_ERR_BAD_VALUE;
  if (desc->sink_blocks < 0 || desc->local_blocks < 0) return BSP_ERR_BAD_VALUE;
  if (!gamma_out || !density_out) return BSP_ERR_NULL_POINTER;
  if (desc->seq == 0) {
    *gamma_out = 1.f;
    *density_out = 1.f;
    return BSP_OK;
  }
  if (!score || !kv_idx || !kv_cnt || !cnt_host) return BSP_ERR_NULL_POINTER;
  const Shape s = shape_of(desc);
  hipStream_t hs = (hipStream_t)stream;
  const size_t rows = (size_t)s.hq * s.nb;
  const double causal = (double)s.hq * s.nb * (s.nb + 1) / 2.0;
  auto density = [&](float g, double *dens) -> bsp_status {
    if (bsp::launch_mask(s, g, desc->sink_blocks, desc->local_blocks, score, nullptr, mask, kv_idx,
                         kv_cnt, hs) != hipSuccess)
      return BSP_ERR_HIP;
    if (hipMemcpyAsync(cnt_host, kv_cnt, rows * sizeof(int32_t), hipMemcpyDeviceToHost, hs) !=
            hipSuccess ||
        hipStreamSynchronize(hs) != hipSuccess)
      return BSP_ERR_HIP;
    double kept = 0.0;
    for (size_t i = 0; i < rows; ++i) kept += cnt_host[i];
    *dens = kept / causal;
    return BSP_OK;
  };
  double d = 0.0;
  if ((st = density(1.f, &d)) != BSP_OK) return st;
  if (d >= target) {
    *gamma_out = 1.f;
    *density_out = (float)d;
    return BSP_OK;
  }
  float lo = 0.f, hi = 1.f;  // density(lo) >= target > density(hi)
  while (hi - lo > tol) {
    const float mid = 0.5f * (lo + hi);
    if ((st = density(mid, &d)) != BSP_OK) return st;
    if (d >= target)
      lo = mid;
    else
      hi = mid;
  }
  if ((st = density(lo, &d)) != BSP_OK) return st;  // leave the buffers at lo
  *gamma_out = lo;
  *density_out = (float)d;
  return BSP_OK;
}

bsp_status bsp_attn_fwd_varlen(const bsp_desc *desc, const bsp_varlen *vl, const void *q,
                               const void *k_cache, const void *v_cache, const int32_t *kv_idx,
                               const int32_t *kv_cnt, void *o, float *lse, void *stream) {
  bsp_status st = check_desc(desc, true);
  if (st != BSP_OK) return st;
  if (!vl) return BSP_ERR_NULL_POINTER;
  if (vl->nseq < 1 || vl->total_blocks < 0 || vl->max_pages < 1 || vl->idx_stride < 1)
    return BSP_ERR_BAD_SHAPE;
  if ((long)desc->hq * vl->total_blocks > 0x7fffffffL) return BSP_ERR_BAD_SHAPE;
  if (desc->dtype == BSP_DTYPE_F32) return BSP_ERR_UNSUPPORTED;
  if (desc->seq == 0 || vl->total_blocks == 0) return BSP_OK;
  if (!vl->cu_seqlens || !vl->cu_blocks || !vl->page_table) return BSP_ERR_NULL_POINTER;
  if (!q || !k_cache || !v_cache || !o) return BSP_ERR_NULL_POINTER;
  if ((kv_idx == nullptr) != (kv_cnt == nullptr)) return BSP_ERR_NULL_POINTER;
  const bool fp8 = fp8_qk(desc);
  if (fp8 && (!desc->q_scale || !desc->k_scale || !desc->v_scale)) return BSP_ERR_BAD_DTYPE;
  if (!fp8 && (desc->q_scale || desc->k_scale || desc->v_scale)) return BSP_ERR_BAD_DTYPE;
  Shape s = shape_of(desc);
  s.nb = vl->total_blocks;
  bsp::AttnArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.kv_idx = kv_idx;
  a.kv_cnt = kv_cnt;
  a.q_scale = desc->q_scale;
  a.k_scale = desc->k_scale;
  a.v_scale = desc->v_scale;
  a.o = o;
  a.lse = lse;
  a.sm_scale = scale_of(desc);
  bsp::VarlenArgs v{vl->cu_seqlens, vl->cu_blocks, vl->page_table, vl->block_order,
                    vl->nseq,       vl->max_pages, vl->idx_stride};
  return hip_status(bsp::launch_attn_varlen(s, a, v, (hipStream_t)stream));
}

// Shared checks of the packed-batch entry points; BSP_OK with *empty set
// when there is nothing to do.
static bsp_status check_varlen(const bsp_desc *desc, const bsp_varlen *vl, bool *empty) {
  if (!vl) return BSP_ERR_NULL_POINTER;
  if (vl->nseq < 1 || vl->total_blocks < 0 || vl->max_pages < 1 || vl->idx_stride < 1)
    return BSP_ERR_BAD_SHAPE;
  if ((long)desc->hq * vl->total_blocks > 0x7fffffffL ||
      (long)desc->hq * vl->total_blocks * vl->idx_stride > 0x7fffffffffffL)
    return BSP_ERR_BAD_SHAPE;
  *empty = desc->seq == 0 || vl->total_blocks == 0;
  if (!*empty && (!vl->cu_seqlens || !vl->cu_blocks)) return BSP_ERR_NULL_POINTER;
  return BSP_OK;
}

bsp_status bsp_score_varlen(const bsp_desc *desc, const bsp_varlen *vl, const void *q,
                            const void *k_cache, float *q_pool, float *k_pool, float *score,
                            void *stream) {
  bsp_status st = check_desc(desc, true);
  if (st != BSP_OK) return st;
  bool empty = false;
  if ((st = check_varlen(desc, vl, &empty)) != BSP_OK) return st;
  if (empty) return BSP_OK;
  if (!vl->page_table || !q || !k_cache || !q_pool || !k_pool || !score)
    return BSP_ERR_NULL_POINTER;
  const bool fp8 = fp8_qk(desc);
  if (fp8 && (!desc->q_scale || !desc->k_scale)) return BSP_ERR_BAD_DTYPE;
  if (!fp8 && (desc->q_scale || desc->k_scale || desc->v_scale)) return BSP_ERR_BAD_DTYPE;
  Shape s = shape_of(desc);
  s.nb = vl->total_blocks;
  const bsp::VarlenArgs v{vl->cu_seqlens, vl->cu_blocks, vl->page_table, vl->block_order,
                          vl->nseq,       vl->max_pages, vl->idx_stride};
  hipStream_t hs = (hipStream_t)stream;
  if (bsp::launch_pool_varlen(s, v, q, k_cache, desc->q_scale, desc->k_scale, q_pool, k_pool,
                              hs) != hipSuccess)
    return BSP_ERR_HIP;
  return hip_status(bsp::launch_score_varlen(s, v, scale_of(desc), q_pool, k_pool, score, hs));
}

bsp_status bsp_mask_varlen(const bsp_desc *desc, const bsp_varlen *vl, const float *score,
                           const uint8_t *user_mask, uint8_t *mask, int32_t *kv_idx,
                           int32_t *kv_cnt, void *stream) {
  bsp_status st = check_desc(desc, false);
  if (st != BSP_OK) return st;
  if (!(desc->gamma >= 0.f && desc->gamma <= 1.f)) return BSP_ERR_BAD_VALUE;  // also NaN
  if (desc->sink_blocks < 0 || desc->local_blocks < 0) return BSP_ERR_BAD_VALUE;
  bool empty = false;
  if ((st = check_varlen(desc, vl, &empty)) != BSP_OK) return st;
  if (empty) return BSP_OK;
  if ((!score && !user_mask) || !kv_idx || !kv_cnt) return BSP_ERR_NULL_POINTER;
  Shape s = shape_of(desc);
  s.nb = vl->total_blocks;
  const bsp::VarlenArgs v{vl->cu_seqlens, vl->cu_blocks, vl->page_table, vl->block_order,
                          vl->nseq,       vl->max_pages, vl->idx_stride};
  return hip_status(bsp::launch_mask_varlen(s, v, desc->gamma, desc->sink_blocks,
                                            desc->local_blocks, score, user_mask, mask, kv_idx,
                                            kv_cnt, (hipStream_t)stream));
}

bsp_status bsp_widen_e4m3(const void *src, void *dst, int64_t n, void *stream) {
  if (n < 0) return BSP_ERR_BAD_SHAPE;
  if (n == 0) return BSP_OK;
  if (!src || !dst) return BSP_ERR_NULL_POINTER;
  if (((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return BSP_ERR_BAD_VALUE;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + 2 * (uintptr_t)n && d0 < s0 + (uintptr_t)n) return BSP_ERR_BAD_VALUE;
  return hip_status(bsp::launch_widen(src, dst, (long)n, (hipStream_t)stream));
}

const char *bsp_status_string(int32_t status) {
  switch (status) {
    case BSP_OK: return "BSP_OK";
    case BSP_ERR_NULL_POINTER: return "BSP_ERR_NULL_POINTER: a required pointer is NULL";
    case BSP_ERR_BAD_SHAPE: return "BSP_ERR_BAD_SHAPE: sizes out of range or inconsistent";
    case BSP_ERR_BAD_DTYPE: return "BSP_ERR_BAD_DTYPE: unknown dtype or fp8 scale mismatch";
    case BSP_ERR_BAD_VALUE: return "BSP_ERR_BAD_VALUE: gamma, sm_scale or window out of range";
    case BSP_ERR_UNSUPPORTED: return "BSP_ERR_UNSUPPORTED: request not served by this build";
    case BSP_ERR_HIP: return "BSP_ERR_HIP: the HIP runtime rejected a launch";
    default: return "unknown bsp_status";
  }
}

int32_t bsp_abi_version(void) { return BSP_ABI_VERSION; }

}  // extern "C"
