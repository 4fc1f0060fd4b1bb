// Decode work items shared by the decode kernels: which (sequence, split)
// a workgroup takes, and the XCD-aware order the workgroups take them in.
#pragma once

#include "common.hpp"

namespace mla {

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// Workgroup order on the XCDs.  Consecutive workgroups are dealt to the eight
// XCDs in turn, and each XCD has its own L2; when the grid is a multiple of
// 32, workgroup x takes work index xcd_local(x), which puts every run of four
// consecutive work indices (the splits of one sequence, or neighbouring query
// blocks, which read the same rows) on one XCD while dispatch still follows
// the index order to within 32.  A bijection on [0, n).
__device__ __forceinline__ int64_t xcd_local(int64_t x, int64_t n) {
  if (n % 32 != 0) return x;
  const int64_t k = x % 8, j = x / 8;
  return ((j / 4) * 8 + k) * 4 + j % 4;
}

struct DecodeItem {
  int b, s, n_s, slot;
  bool ok;
};

// Map a work-item index to (sequence, split).  Items [0, n_full) are the
// full splits of split_pages pages in sequence order, then one remainder
// split per sequence whose page count is not a multiple of split_pages; the
// long items go first.  slot = index of (b, s) in sequence-major order.
inline __device__ DecodeItem find_decode_item(const AttnParams& p, int64_t item) {
  const int lane = threadIdx.x & 63;
  const int L = p.split_pages;
  const bool want_full = item < p.n_full;
  const int target = static_cast<int>(want_full ? item : item - p.n_full);
  int base_cnt = 0, base_ns = 0;
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int b = b0 + lane;
    int t = b < p.batch ? p.seq_lens[b] : 0;
    t = t < 0 ? 0 : t;
    const int pages = (t + kPage - 1) / kPage;
    const int nf = pages / L;
    const int rem = (pages % L) != 0 ? 1 : 0;
    const int ns = nf + rem;
    const int cnt = want_full ? nf : rem;
    const int c_incl = wave_incl_scan(cnt);
    const int ns_incl = wave_incl_scan(ns);
    const int lo = base_cnt + c_incl - cnt;
    const bool hit = cnt > 0 && target >= lo && target < lo + cnt;
    const unsigned long long mask = __ballot(hit);
    if (mask) {
      const int src = __ffsll(static_cast<long long>(mask)) - 1;
      DecodeItem it;
      it.b = b0 + src;
      const int lo_s = __shfl(lo, src, 64);
      const int nf_s = __shfl(nf, src, 64);
      it.n_s = __shfl(ns, src, 64);
      it.s = want_full ? target - lo_s : nf_s;
      it.slot = base_ns + __shfl(ns_incl, src, 64) - it.n_s + it.s;
      it.ok = true;
      return it;
    }
    base_cnt += __shfl(c_incl, 63, 64);
    base_ns += __shfl(ns_incl, 63, 64);
  }
  DecodeItem none{0, 0, 0, 0, false};
  return none;
}

}  // namespace mla
