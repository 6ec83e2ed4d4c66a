// Asymmetric per-tensor UINT8 activations with symmetric per-channel INT8
// weights on gfx950.
//
// Method: page 2, "Meituan open-sources a lossless INT8 DeepSeek R1:
// technical breakthroughs and practice guide", part two, item 1 (dynamic
// range-aware quantisation): a tensor's min and max spread over the 256
// codes of a byte, s = (max - min) / 255, zero point z = -min / s,
// q = clamp(rne((x - min) / s), 0, 255); x^ = s (q - z).  Every step is one
// fp32 IEEE operation; a constant tensor's range is floored at 1e-10, as the
// symmetric quantiser floors its amax.  Weights stay symmetric per output
// channel (page 1, section 2.3, channel-wise scheme), so
//   Y[m][n] = s w_scale[n] (ACC[m][n] - z WS[n]),
//   ACC = sum_k q Wq (exact), WS[n] = sum_k Wq[n][k] (exact),
// evaluated as fp32(fp32(s * w_scale[n]) * fp32(fp32(ACC) - fp32(z * fp32(WS)))).
//
// Codes are stored as q - 128 (int8), which the signed int8 MFMA takes as is:
// ACC = ACC' + 128 WS with ACC' the channel-wise GEMM's exact int32
// accumulation of the stored codes.  Where the channel-wise tile grid runs
// unsplit (large M) the epilogue is the tile kernel's own; otherwise (decode
// kernels, K split) the int32 accumulators go through a workspace to
// k_asym_epilogue.
//
// The quantiser takes two launches: every workgroup of the first reduces its
// share of the tensor to a partial (min, max); every workgroup of the second
// reduces all partials (exact, so each derives the same s and z) and then
// quantises its share.  The quotient goes through a reciprocal estimate with
// a tie check (proof at kAsymTieGuard), exact division deciding near ties.
#include "common.h"
#include "launch.h"

namespace w8 {
namespace {

constexpr int kAsymMaxWgs = 1024;       // partial ranges per tensor
constexpr float kURange = 255.0f;
// Quotient estimate y = fp32(d * fp32(1 / s)) for 0 <= d / s <= 255.00003:
// |y - d / s| <= (d / s)(2^-23 + 2^-48) < 3.05e-5, and the correctly rounded
// fp32(d / s) lies within half an ulp (7.7e-6 below 256) of d / s, so the
// two differ by less than 3.9e-5 < 2^-14.  If y is farther than 2^-14 from
// every half-integer, both round to the same integer; otherwise the exact
// division decides.
constexpr float kAsymTieGuard = 0.49993896484375f;   // 0.5 - 2^-14

// Block-wide min and max for a 256-thread workgroup, every thread gets both.
__device__ __forceinline__ void block_minmax256(float& mn, float& mx, float* red4) {
  const float nmn = block_max256(-mn, red4);
  __syncthreads();
  mx = block_max256(mx, red4);
  mn = -nmn;
}

template <bool FP16>
__global__ __launch_bounds__(256) void k_minmax_partial(const uint4* __restrict__ x, int64_t nchunks,
                                                        float* __restrict__ part) {
  __shared__ float red[4];
  float mn = INFINITY, mx = -INFINITY;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * 256) {
    float v[8];
    unpack8<FP16>(x[c], v);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mn = fminf(mn, v[i]);
      mx = fmaxf(mx, v[i]);
    }
  }
  block_minmax256(mn, mx, red);
  if (threadIdx.x == 0) {
    part[2 * blockIdx.x] = mn;
    part[2 * blockIdx.x + 1] = mx;
  }
}

template <bool FP16>
__global__ __launch_bounds__(256) void k_quant_asym(const uint4* __restrict__ x, int64_t nchunks,
                                                    const float* __restrict__ part, int nparts,
                                                    uint2* __restrict__ q, float* __restrict__ params) {
  __shared__ float red[4];
  float mn = INFINITY, mx = -INFINITY;
  for (int i = threadIdx.x; i < nparts; i += 256) {
    mn = fminf(mn, part[2 * i]);
    mx = fmaxf(mx, part[2 * i + 1]);
  }
  block_minmax256(mn, mx, red);
  const float s = fmaxf(__fsub_rn(mx, mn), kEps) / kURange;   // correctly rounded fp32 divisions
  const float z = -mn / s;
  const float r = 1.0f / s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    params[0] = s;
    params[1] = z;
  }
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * 256) {
    float v[8];
    unpack8<FP16>(x[c], v);
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float d = __fsub_rn(v[i], mn);
      const float y = __fmul_rn(d, r);
      float t = __builtin_rintf(y);
      if (__builtin_expect(__builtin_fabsf(__fsub_rn(y, t)) > kAsymTieGuard, 0)) t = __builtin_rintf(d / s);
      t = fminf(fmaxf(t, 0.f), kURange);
      b[i] = (uint32_t)((int)t - 128) & 0xffu;
    }
    q[c] = make_uint2(b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24));
  }
}

// WS[n] = sum_k W[n][k]: one wave per row, 16 bytes per lane and step.
__global__ __launch_bounds__(256) void k_weight_row_sums(const uint4* __restrict__ W, int N, int K,
                                                         int32_t* __restrict__ ws) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const int nch = K >> 4;
  const uint4* row = W + (int64_t)n * nch;
  int acc = 0;
  for (int c = lane; c < nch; c += 64) {
    const uint4 u = row[c];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc += (int)(int8_t)(w[i] >> (8 * j));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) ws[n] = acc;
}

// Y from the stored codes' int32 accumulation; 4 consecutive outputs of one
// row per thread.
template <int OUT>
__global__ __launch_bounds__(256) void k_asym_epilogue(const int32_t* __restrict__ acc, int M, int N,
                                                       const float* __restrict__ params,
                                                       const float* __restrict__ sw,
                                                       const int32_t* __restrict__ wsum, void* __restrict__ Y) {
  const int64_t q4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nq = (N + 3) >> 2;
  if (q4 >= (int64_t)M * nq) return;
  const int m = (int)(q4 / nq), n = (int)(q4 - (int64_t)m * nq) * 4;
  const int64_t idx = (int64_t)m * N + n;
  const float s = params[0], z = params[1];
  float o[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (n + r < N) {
      const int32_t ws = wsum[n + r];
      const int32_t a = acc[idx + r] + 128 * ws;
      o[r] = __fmul_rn(__fmul_rn(s, sw[n + r]), __fsub_rn((float)a, __fmul_rn(z, (float)ws)));
    } else {
      o[r] = 0.f;
    }
  }
  if (OUT == OUT_F32) {
    float* y = static_cast<float*>(Y) + idx;
    if ((N & 3) == 0) {
      *reinterpret_cast<float4*>(y) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) y[r] = o[r];
    }
  } else {
    uint16_t* y = static_cast<uint16_t*>(Y) + idx;
    uint32_t h[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(o[r]);
    if ((N & 3) == 0) {
      *reinterpret_cast<uint2*>(y) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) y[r] = (uint16_t)h[r];
    }
  }
}

}  // namespace

hipError_t launch_quant_asym(const void* x, bool fp16, int64_t M, int64_t K, int8_t* q, float* params,
                             hipStream_t st) {
  const int64_t nchunks = M * K / 8;
  int64_t g = (nchunks + 4 * 256 - 1) / (4 * 256);
  const int wgs = (int)(g < kAsymMaxWgs ? g : kAsymMaxWgs);
  // the partial ranges live in the stream's slot-1 scratch, held until both
  // passes are enqueued
  const WsLease lease = stream_workspace(st, 1, (size_t)wgs * 2 * sizeof(float));
  if (lease.status() != kWsOk) return ws_error(lease);
  void* part = lease.ptr();
  const uint4* xp = static_cast<const uint4*>(x);
  float* pp = static_cast<float*>(part);
  if (fp16) {
    hipLaunchKernelGGL((k_minmax_partial<true>), dim3(wgs), dim3(256), 0, st, xp, nchunks, pp);
    hipLaunchKernelGGL((k_quant_asym<true>), dim3(wgs), dim3(256), 0, st, xp, nchunks, pp, wgs,
                       reinterpret_cast<uint2*>(q), params);
  } else {
    hipLaunchKernelGGL((k_minmax_partial<false>), dim3(wgs), dim3(256), 0, st, xp, nchunks, pp);
    hipLaunchKernelGGL((k_quant_asym<false>), dim3(wgs), dim3(256), 0, st, xp, nchunks, pp, wgs,
                       reinterpret_cast<uint2*>(q), params);
  }
  return hipGetLastError();
}

hipError_t launch_weight_row_sums(const int8_t* W, int64_t N, int64_t K, int32_t* ws, hipStream_t st) {
  hipLaunchKernelGGL(k_weight_row_sums, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(W), (int)N, (int)K, ws);
  return hipGetLastError();
}

hipError_t launch_gemm_asym(const int8_t* A, const float* params, const int8_t* W, const float* sw,
                            const int32_t* wsum, void* Y, OutKind out, int64_t M, int64_t N, int64_t K,
                            hipStream_t st) {
  if (channel_tiles_unsplit(M, N, K)) return launch_gemm_channel_asym_tiles(A, params, W, sw, wsum, Y, out, M, N, K, st);
  // int32 accumulators in the stream's slot-1 scratch, held until the
  // epilogue is enqueued (the GEMM may take slot 0 inside it)
  const WsLease lease = stream_workspace(st, 1, (size_t)M * N * 4);
  if (lease.status() != kWsOk) return ws_error(lease);
  void* acc = lease.ptr();
  hipError_t e = launch_gemm_channel(A, nullptr, W, nullptr, acc, OUT_I32, M, N, K, st);
  if (e != hipSuccess) return e;
  const dim3 g((unsigned)((M * ((N + 3) / 4) + 255) / 256));
  const int32_t* ap = static_cast<const int32_t*>(acc);
  if (out == OUT_F32)
    hipLaunchKernelGGL((k_asym_epilogue<OUT_F32>), g, dim3(256), 0, st, ap, (int)M, (int)N, params, sw, wsum, Y);
  else
    hipLaunchKernelGGL((k_asym_epilogue<OUT_BF16>), g, dim3(256), 0, st, ap, (int)M, (int)N, params, sw, wsum, Y);
  return hipGetLastError();
}

}  // namespace w8
