// Ascending compaction of a row's kept key blocks into its kv_idx row, shared
// by the mask kernels and the fused score-and-mask kernel (FlashPrefill
// summary page, Appendix B: after the masks are combined, the active block
// indices are compressed; section 3 "Max-based Dynamic Thresholding": no sort
// and no cumulative sum is needed).
#pragma once

#include "device.h"

namespace bsp {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Orders a wavefront's LDS accesses across its lanes: every LDS store a
// lane issued before it is visible to the loads any lane of the same
// wavefront issues after it (a wavefront-scope release/acquire fence, which
// also keeps the compiler from moving LDS accesses across it).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A row's kept key blocks in ascending order, written to its kv_idx row.
// Kept entry k of the row waits in slot k % 512 of the wavefront's LDS ring;
// whenever 256 entries wait, they leave as one 1 KiB store of 16 bytes per
// lane, aligned (their first k is a multiple of 256) and non-temporal, so the
// list streams to HBM in whole lines without passing through L2 (at 2048
// blocks per row this takes the kernel from 166 to 125 us; ordinary stores,
// scattered 4-byte or whole 16-byte ones, ran at the slower rate).  Entries
// past the last whole run leave at the end.
struct KeptList {
  int32_t *ring;  // 512 entries, private to the wavefront
  int32_t *dst;   // the row of kv_idx
  uint64_t below;  // lanes under this one
  int lane, n, flushed;
  bool vec;  // dst is 16-byte aligned

  __device__ __forceinline__ void init(int32_t *ring_, int32_t *dst_, int lane_, bool vec_) {
    ring = ring_;
    dst = dst_;
    lane = lane_;
    vec = vec_;
    below = (1ull << lane) - 1ull;
    n = flushed = 0;
  }
  // the lane's blocks J .. J + 3, kept where keep[e]
  __device__ __forceinline__ void push(const bool (&keep)[4], int J) {
    int before = 0, total = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint64_t bal = __ballot(keep[e]);
      before += __popcll(bal & below);
      total += __popcll(bal);
    }
    int mine = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (keep[e]) ring[(n + before + mine) & 511] = J + e;
      mine += keep[e] ? 1 : 0;
    }
    n += total;
    if (n - flushed >= 256) {  // at most 511 wait, so one run per step
      // lanes read entries other lanes stored: order the LDS accesses
      wave_lds_sync();
      const int4 v = *(const int4 *)&ring[(flushed & 511) + 4 * lane];
      int32_t *d = dst + flushed + 4 * lane;
      if (vec) {
        __builtin_nontemporal_store(i32x4{v.x, v.y, v.z, v.w}, (i32x4 *)d);
      } else {
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
      }
      flushed += 256;
      wave_lds_sync();  // the next push may overwrite the slots just read
    }
  }
  // the last n - flushed (< 256) entries; returns the row's count
  __device__ __forceinline__ int finish() {
    wave_lds_sync();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = flushed + 4 * lane + e;
      if (i < n) dst[i] = ring[i & 511];
    }
    return n;
  }
};

}  // namespace bsp
