// Expert row ranges -> workgroup tiles for the grouped (MoE) GEMMs.
//
// The rows of the permuted activation matrix are grouped by expert
// (off[e] .. off[e + 1] - 1 belong to expert e; off is non-decreasing, with
// off[0] = 0 and off[E] = P).  Each expert's rows are cut into BM-row tiles,
// and tiles are numbered in expert order; group_tile maps a tile number to its
// expert and row range.  Method reference: the block-wise scheme of "DeepSeek
// R1 INT8 quantisation in SGLang" (Meituan), section 2.3, applied per expert;
// that DeepSeek's feed-forward layers are mixture-of-experts is stated on
// "FP8 vs INT8 quantisation for DeepSeek", section 1.2.
#pragma once

#include "common.h"

namespace w8 {

struct ExpertTile {
  int e, r0, r1;  // e < 0: the tile number is past the last tile
};

// Wave 0 counts the tiles of E / 64 experts per lane, prefix-sums the counts
// across the wave and lets the lane whose range holds tile t walk to it.
// Only experts with more than clo and at most chi rows have tiles (the others
// count zero), so one launch can take the light experts and another the
// heavy ones.  Every thread of the workgroup must call it (it ends with a
// barrier); sel is three ints of LDS that the caller leaves alone until every
// thread has returned.
template <int BM>
__device__ ExpertTile group_tile(const int32_t* __restrict__ off, int E, int P, int t, int* sel, int clo, int chi) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    const int e1 = e0 + per < E ? e0 + per : E;
    int cnt = 0;
    for (int e = e0; e < e1; ++e) {
      int lo = off[e], hi = off[e + 1];
      lo = lo < 0 ? 0 : (lo > P ? P : lo);
      hi = hi < lo ? lo : (hi > P ? P : hi);
      if (hi - lo > clo && hi - lo <= chi) cnt += (hi - lo + BM - 1) / BM;
    }
    int inc = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(inc, d, 64);
      if (lane >= d) inc += v;
    }
    if (lane == 0) sel[0] = -1;  // program order within the wave: before any hit below
    if (t >= inc - cnt && t < inc) {
      int acc = inc - cnt;
      for (int e = e0; e < e1; ++e) {
        int lo = off[e], hi = off[e + 1];
        lo = lo < 0 ? 0 : (lo > P ? P : lo);
        hi = hi < lo ? lo : (hi > P ? P : hi);
        const int c = hi - lo > clo && hi - lo <= chi ? (hi - lo + BM - 1) / BM : 0;
        if (t < acc + c) {
          const int r0 = lo + (t - acc) * BM;
          sel[0] = e;
          sel[1] = r0;
          sel[2] = r0 + BM < hi ? r0 + BM : hi;
          break;
        }
        acc += c;
      }
    }
  }
  __syncthreads();
  ExpertTile g;
  g.e = sel[0];
  g.r0 = sel[1];
  g.r1 = sel[2];
  return g;
}

}  // namespace w8
