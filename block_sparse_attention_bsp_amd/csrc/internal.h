// Launchers shared between the C-ABI host layer (bsp_api.cpp) and the
// kernel translation units.  Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsp {

struct Shape {
  int hq, hkv, seq, d, block, nb, dtype;
};

struct AttnArgs {
  const void *q, *k, *v;
  const int32_t *kv_idx, *kv_cnt;  // both null = dense causal
  const float *q_scale, *k_scale, *v_scale;
  void *o;
  float *lse;
  float sm_scale;
};

hipError_t launch_pool(const Shape &s, const void *q, const void *k, const float *q_scale,
                       const float *k_scale, float *q_pool, float *k_pool, hipStream_t st);
hipError_t launch_score(const Shape &s, float c, const float *q_pool, const float *k_pool,
                        const float *k_radius, float *score, hipStream_t st);
// The threshold of stage 2 fused into the score kernel's second pass
// (passed to the kernel by value): keep = P >= gamma * row max, or J < sink,
// or I - J < local, and J <= I; mask may be null.
struct FuseMask {
  float gamma;
  int sink, local;
  uint8_t *mask;
  int32_t *idx, *cnt;
};
hipError_t launch_score_mask(const Shape &s, float c, const float *q_pool, const float *k_pool,
                             float *score, const FuseMask &fz, hipStream_t st);
hipError_t launch_radius(const Shape &s, const void *k, const float *k_scale, const float *k_pool,
                         float *k_radius, hipStream_t st);
hipError_t launch_score_arith(const Shape &s, float c, const void *q, const float *k_pool,
                              float *score, const float *q_scale, hipStream_t st);
// rescue != nullptr (and no user mask): a block is also kept when its rescue
// score reaches gamma_r times the row's maximum rescue score.
hipError_t launch_mask(const Shape &s, float gamma, int sink_blocks, int local_blocks,
                       const float *score, const uint8_t *user_mask, uint8_t *mask,
                       int32_t *kv_idx, int32_t *kv_cnt, hipStream_t st,
                       const float *rescue = nullptr, float gamma_r = 0.f);
// Packed variable-length batch over a paged K/V cache (passed to kernels by
// value): sequence s owns tokens cu_seqlens[s] .. cu_seqlens[s+1] of q / o /
// lse and query blocks cu_blocks[s] .. cu_blocks[s+1] of the batch; key
// block J of sequence s is cache page page_table[s * max_pages + J], laid out
// [page][hkv][block][d]; kv lists and score / mask rows have stride
// idx_stride; block_order is an optional launch order of the batch's blocks.
struct VarlenArgs {
  const int32_t *cu_seqlens, *cu_blocks, *page_table, *block_order;
  int nseq, max_pages, idx_stride;
};

// Packed variable-length batches (s.seq = the batch's tokens, s.nb = its
// query blocks): stage 1 over Q and the paged K cache, per-sequence block
// scores in rows of stride vl.idx_stride, and the mask with the same rows.
hipError_t launch_pool_varlen(const Shape &s, const VarlenArgs &vl, const void *q,
                              const void *k_cache, const float *q_scale, const float *k_scale,
                              float *q_pool, float *k_pool, hipStream_t st);
hipError_t launch_score_varlen(const Shape &s, const VarlenArgs &vl, float c, const float *q_pool,
                               const float *k_pool, float *score, hipStream_t st);
hipError_t launch_mask_varlen(const Shape &s, const VarlenArgs &vl, float gamma, int sink,
                              int local, const float *score, const uint8_t *user, uint8_t *mask,
                              int32_t *kv_idx, int32_t *kv_cnt, hipStream_t st);

hipError_t launch_attn_f32(const Shape &s, const AttnArgs &a, hipStream_t st);
hipError_t launch_attn_varlen(const Shape &s, const AttnArgs &a, const VarlenArgs &v,
                              hipStream_t st);
hipError_t launch_attn_bf16(const Shape &s, const AttnArgs &a, hipStream_t st);
// e4m3 Q and K; V as e4m3 codes, or bf16 when s.dtype is the mixed code
hipError_t launch_attn_fp8(const Shape &s, const AttnArgs &a, hipStream_t st);
// n e4m3 codes -> n bf16 values, exactly
hipError_t launch_widen(const void *src, void *dst, long n, hipStream_t st);

}  // namespace bsp
