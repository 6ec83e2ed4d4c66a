// Device helpers shared by the large-M GEMM kernels (channel-wise tiles in
// gemm_tile.hip, block-wise tiles in gemm_block.hip): output stores and the
// XCD-aware workgroup -> tile order.
#pragma once

#include "launch.h"
#include "pipeline.h"

namespace w8 {
namespace {

// Store 4 consecutive outputs Y[m][n..n+3] (n multiple of 4).
template <int OUT>
__device__ __forceinline__ void store4(void* Y, int64_t idx, int n, int N, bool vec, float a, float b, float c,
                                       float d) {
  if (OUT == OUT_F32) {
    float* y = static_cast<float*>(Y) + idx;
    if (vec && n + 3 < N) {
      *reinterpret_cast<float4*>(y) = make_float4(a, b, c, d);
    } else {
      if (n < N) y[0] = a;
      if (n + 1 < N) y[1] = b;
      if (n + 2 < N) y[2] = c;
      if (n + 3 < N) y[3] = d;
    }
  } else {
    uint16_t* y = static_cast<uint16_t*>(Y) + idx;
    const uint32_t ha = f32_to_bf16_rne(a), hb = f32_to_bf16_rne(b), hc = f32_to_bf16_rne(c),
                   hd = f32_to_bf16_rne(d);
    if (vec && n + 3 < N) {
      *reinterpret_cast<uint2*>(y) = make_uint2(ha | (hb << 16), hc | (hd << 16));
    } else {
      if (n < N) y[0] = (uint16_t)ha;
      if (n + 1 < N) y[1] = (uint16_t)hb;
      if (n + 2 < N) y[2] = (uint16_t)hc;
      if (n + 3 < N) y[3] = (uint16_t)hd;
    }
  }
}

__device__ __forceinline__ void store4i(int32_t* y, int n, int N, bool vec, v4i v) {
  if (vec && n + 3 < N) {
    *reinterpret_cast<v4i*>(y) = v;
  } else {
    if (n < N) y[0] = v[0];
    if (n + 1 < N) y[1] = v[1];
    if (n + 2 < N) y[2] = v[2];
    if (n + 3 < N) y[3] = v[3];
  }
}

// Workgroup -> tile.  The hardware dispatches workgroup b to XCD b % 8, and
// each XCD has its own L2.  Tiles t = x*T/8 .. (x+1)*T/8 - 1 of the sequence
// go to XCD x (a contiguous band), and the sequence walks strips of GM row
// tiles (m fastest inside a strip): an XCD's 32 concurrent workgroups then
// cover about GM row tiles x 32 / GM column tiles and share both operands'
// panels in its L2 (with GM = TM, one column of row tiles at a time, an
// XCD's 32 workgroups span 2 column tiles x 16 row tiles at M = 4096 and
// fetch each K block's panels once per 18 tiles instead of once per 12).
__device__ __forceinline__ void strip_tile(int b, int TM, int TN, int GM, int& tm, int& tn) {
  const int T = TM * TN;
  const int x = b & 7, j = b >> 3;
  const int T8 = T >> 3, rem = T & 7;
  const int t = x * T8 + (x < rem ? x : rem) + j;
  const int strip = t / (GM * TN);
  const int r = t - strip * GM * TN;
  const int gm = TM - strip * GM < GM ? TM - strip * GM : GM;
  tm = strip * GM + r % gm;
  tn = r / gm;
}

}  // namespace
}  // namespace w8
