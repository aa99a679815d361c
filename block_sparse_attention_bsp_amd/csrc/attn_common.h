// Pieces shared by the MFMA attention kernels (bf16 and fp8): the order in
// which workgroups take (q head, query block) rows, the packed-batch lookup,
// and the stream of a row's kept key-block list.
#pragma once

#include "device.h"
#include "internal.h"

namespace bsp {

// Workgroup bid -> (query block I, q head h), heaviest rows first.
//   xcd_map == 0: plain order.
//   xcd_map >= hkv: XCD x = bid % 8 (the hardware's round-robin) serves kv
//     group x % hkv, so the workgroups resident on an XCD walk the same K/V
//     blocks together out of its L2.
//   0 < xcd_map < hkv: phases of P = xcd_map groups, so that the K/V of the
//     groups in flight stay within the memory-side cache: in phase p, XCD x
//     serves group p * P + x / S (S = 8 / P XCDs per group) and, of that
//     group, the rows I with (nb - 1 - I) % S == x % S, all its q heads.
__device__ __forceinline__ void attn_row_of(int bid, int xcd_map, int hq, int hkv, int nb, int &I,
                                            int &h) {
  const int grp = hq / hkv;
  if (xcd_map > 0 && xcd_map < hkv) {
    const int P = xcd_map, S = 8 / P;
    const int x = bid & 7, j = bid >> 3;
    const int len = grp * nb / S;
    const int p = j / len, jj = j - p * len;
    I = nb - 1 - (x % S + S * (jj / grp));
    h = (p * P + x / S) * grp + jj % grp;
  } else if (xcd_map) {
    const int x = bid & 7, j = bid >> 3, X = 8 / hkv;
    const int n = x / hkv + X * j;
    I = nb - 1 - n / grp;
    h = (x % hkv) * grp + n % grp;
  } else {
    I = nb - 1 - bid / hq;
    h = bid % hq;
  }
}

// Host: the xcd_map value for a launch of hq * nb workgroups whose kv groups
// each hold kv_bytes_per_group of K and V.  Groups go in phases when all of
// them exceed half of the 256 MiB memory-side cache; the dense order is
// unaffected by it, while scattered kept blocks that miss L2 then come from
// that cache instead of HBM.
static inline int attn_xcd_mode(const Shape &s, long kv_bytes_per_group) {
  const long items = (long)s.hq * s.nb;
  if (!(s.hkv <= 8 && 8 % s.hkv == 0 && items % 8 == 0)) return 0;
  int P = s.hkv;
  while (P > 1 && (long)P * kv_bytes_per_group > (128l << 20)) P >>= 1;
  if (P < s.hkv && s.nb % (8 / P) != 0) P = s.hkv;
  return P;
}

// The row a workgroup serves, after the packed-batch lookup (VL): batch
// block gb (the kv-list row), the sequence's query block I, its first token
// tok0 and length len, the kv-list row stride and the sequence's page table.
struct AttnRow {
  int I, gb, tok0, len, stride;
  const int32_t *ptab;
};

template <bool VL>
__device__ __forceinline__ AttnRow attn_locate(int I, int seq, int nb, const VarlenArgs &vl) {
  AttnRow r{I, I, 0, seq, nb, nullptr};
  if constexpr (VL) {
    // launch order: the caller's permutation (heaviest first), if given
    if (vl.block_order) r.gb = vl.block_order[nb - 1 - I];
    const int lo = varlen_seq_of(vl.cu_blocks, vl.nseq, r.gb);
    r.I = r.gb - vl.cu_blocks[lo];
    r.tok0 = vl.cu_seqlens[lo];
    r.len = vl.cu_seqlens[lo + 1] - r.tok0;
    r.ptab = vl.page_table + (size_t)lo * vl.max_pages;
    r.stride = vl.idx_stride;
  }
  return r;
}

// A row's kept key blocks, streamed through registers 64 entries at a time:
// lane l holds entry 64c + l of chunk c, and chunk c + 1 is loaded on
// entering chunk c.  An entry is picked with readlane, so no step waits on a
// global load of its block index (such waits desynchronise the workgroups
// that otherwise walk the same K/V blocks together out of L2).  Without a
// list the blocks are 0 .. I (dense causal).  Entries outside [0, I] read as
// -1 (skipped).
struct KvStream {
  const int32_t *ilist;
  int nblk, I, lane, lcur, lnxt, chunk;

  __device__ __forceinline__ void init(const int32_t *list, int n, int I_, int lane_) {
    ilist = list;
    nblk = n;
    I = I_;
    lane = lane_;
    lcur = lnxt = chunk = 0;
    if (ilist) {
      lcur = lane < nblk ? ilist[lane] : 0;
      lnxt = 64 + lane < nblk ? ilist[64 + lane] : 0;
    }
  }
  // t grows by at most one per call
  __device__ __forceinline__ int block_of(int t) {
    if (!ilist) return t;
    if ((t >> 6) != chunk) {
      chunk = t >> 6;
      lcur = lnxt;
      const int e = (chunk + 1) * 64 + lane;
      lnxt = e < nblk ? ilist[e] : 0;
    }
    const int J = __builtin_amdgcn_readlane(lcur, t & 63);
    return (J < 0 || J > I) ? -1 : J;
  }
};

}  // namespace bsp
