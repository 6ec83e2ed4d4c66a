// Small-M (decode-shaped) GEMMs on gfx950: weight streaming.
//
// With M <= 64 the weights dominate the traffic (N x K bytes against M x K of
// activations), so these kernels are HBM-bound: every weight byte is loaded
// once, straight from global memory into MFMA operand registers (no LDS
// staging), with the next K block's loads in flight while the current one is
// multiplied.  A workgroup owns 16 * FNW output columns; its SK waves split
// the K blocks between them (block kb goes to wave kb % SK) and their partial
// results are summed in LDS in wave order, so results are deterministic.
//
// Method references:
//   W8A8 block-wise / channel-wise: "DeepSeek R1 INT8 quantisation in SGLang"
//   (Meituan), section 2.3 (per-K-block dequant vs one epilogue dequant);
//   W8A16 group-wise: "DeepSeek-R1-0528-Qwen3-8B Int8 W8A16" release note
//   (symmetric group-wise INT8 weights, fp16 activations).
#include "common.h"
#include "launch.h"

namespace w8 {
namespace {

typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v4i ld16(const int8_t* p) { return *reinterpret_cast<const v4i*>(p); }

// --------------------------------------------------------------- W8A8
// MODE 0: block-wise (fp32 accumulate of per-block dequantised partials);
// MODE 1: channel-wise (int32 accumulate over all K, one epilogue dequant).
template <int MODE, int MF, int FNW, int SK, int OUT>
__global__ __launch_bounds__(64 * SK) void k_decode_w8a8(const int8_t* __restrict__ A, const float* __restrict__ sa,
                                                         const int8_t* __restrict__ W, const float* __restrict__ sw,
                                                         void* __restrict__ Y, int M, int N, int K) {
  __shared__ v4i red[SK][FNW][MF][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int n0 = blockIdx.x * 16 * FNW;
  const int KB = K >> 7;

  const int8_t* wrow[FNW];
  int nb[FNW];
#pragma unroll
  for (int f = 0; f < FNW; ++f) {
    int n = n0 + f * 16 + (lane & 15);
    n = n < N ? n : N - 1;
    wrow[f] = W + (int64_t)n * K + q * 16;
    int b = (n0 + f * 16) >> 7;
    nb[f] = b;
  }
  const int8_t* arow[MF];
  bool aval[MF];
#pragma unroll
  for (int j = 0; j < MF; ++j) {
    int m = j * 16 + (lane & 15);
    aval[j] = m < M;
    arow[j] = A + (int64_t)(m < M ? m : M - 1) * K + q * 16;
  }

  v4f facc[FNW][MF];
  v4i iacc[FNW][MF];
#pragma unroll
  for (int f = 0; f < FNW; ++f)
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      facc[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};
      iacc[f][j] = (v4i){0, 0, 0, 0};
    }

  v4i wv[FNW][2], av[MF][2];
  int kb = wave;
  if (kb < KB) {
#pragma unroll
    for (int f = 0; f < FNW; ++f) {
      wv[f][0] = ld16(wrow[f] + kb * 128);
      wv[f][1] = ld16(wrow[f] + kb * 128 + 64);
    }
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      av[j][0] = ld16(arow[j] + kb * 128);
      av[j][1] = ld16(arow[j] + kb * 128 + 64);
    }
  }
  for (; kb < KB; kb += SK) {
    v4i cw[FNW][2], ca[MF][2];
#pragma unroll
    for (int f = 0; f < FNW; ++f) {
      cw[f][0] = wv[f][0];
      cw[f][1] = wv[f][1];
    }
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      ca[j][0] = aval[j] ? av[j][0] : (v4i){0, 0, 0, 0};
      ca[j][1] = aval[j] ? av[j][1] : (v4i){0, 0, 0, 0};
    }
    const int kn = kb + SK;
    if (kn < KB) {
#pragma unroll
      for (int f = 0; f < FNW; ++f) {
        wv[f][0] = ld16(wrow[f] + kn * 128);
        wv[f][1] = ld16(wrow[f] + kn * 128 + 64);
      }
#pragma unroll
      for (int j = 0; j < MF; ++j) {
        av[j][0] = ld16(arow[j] + kn * 128);
        av[j][1] = ld16(arow[j] + kn * 128 + 64);
      }
    }
    if (MODE == 0) {
      float s[FNW][MF];
#pragma unroll
      for (int f = 0; f < FNW; ++f) {
        const int bb = nb[f] < ((N + 127) >> 7) ? nb[f] : ((N + 127) >> 7) - 1;
        const float swv = sw[(int64_t)bb * KB + kb];
#pragma unroll
        for (int j = 0; j < MF; ++j) {
          int m = j * 16 + (lane & 15);
          m = m < M ? m : M - 1;
          s[f][j] = __fmul_rn(sa[(int64_t)m * KB + kb], swv);
        }
      }
#pragma unroll
      for (int f = 0; f < FNW; ++f)
#pragma unroll
        for (int j = 0; j < MF; ++j) {
          v4i p = __builtin_amdgcn_mfma_i32_16x16x64_i8(cw[f][0], ca[j][0], (v4i){0, 0, 0, 0}, 0, 0, 0);
          p = __builtin_amdgcn_mfma_i32_16x16x64_i8(cw[f][1], ca[j][1], p, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) facc[f][j][r] = __builtin_fmaf(s[f][j], (float)p[r], facc[f][j][r]);
        }
    } else {
#pragma unroll
      for (int f = 0; f < FNW; ++f)
#pragma unroll
        for (int j = 0; j < MF; ++j) {
          iacc[f][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(cw[f][0], ca[j][0], iacc[f][j], 0, 0, 0);
          iacc[f][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(cw[f][1], ca[j][1], iacc[f][j], 0, 0, 0);
        }
    }
  }

  // cross-wave reduction in wave order
#pragma unroll
  for (int f = 0; f < FNW; ++f)
#pragma unroll
    for (int j = 0; j < MF; ++j)
      red[wave][f][j][lane] = MODE == 0 ? __builtin_bit_cast(v4i, facc[f][j]) : iacc[f][j];
  __syncthreads();
  if (wave != 0) return;
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int f = 0; f < FNW; ++f) {
    const int n = n0 + f * 16 + 4 * q;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      const int m = j * 16 + (lane & 15);
      if (m >= M) continue;
      float o[4];
      if (MODE == 0) {
        v4f t = __builtin_bit_cast(v4f, red[0][f][j][lane]);
#pragma unroll
        for (int w = 1; w < SK; ++w) t += __builtin_bit_cast(v4f, red[w][f][j][lane]);
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = t[r];
      } else {
        v4i t = red[0][f][j][lane];
#pragma unroll
        for (int w = 1; w < SK; ++w) t += red[w][f][j][lane];
        if (OUT == OUT_I32) {
          int32_t* y = static_cast<int32_t*>(Y) + (int64_t)m * N + n;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) y[r] = t[r];
          continue;
        }
        const float s_m = sa[m];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = n + r < N ? __fmul_rn((float)t[r], __fmul_rn(s_m, sw[n + r])) : 0.f;
      }
      const int64_t idx = (int64_t)m * N + n;
      if (OUT == OUT_F32) {
        float* y = static_cast<float*>(Y) + idx;
        if (vec && n + 3 < N) {
          *reinterpret_cast<float4*>(y) = make_float4(o[0], o[1], o[2], o[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) y[r] = o[r];
        }
      } else if (OUT == OUT_BF16) {
        uint16_t* y = static_cast<uint16_t*>(Y) + idx;
        uint32_t h[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) h[r] = f32_to_bf16_rne(o[r]);
        if (vec && n + 3 < N) {
          *reinterpret_cast<uint2*>(y) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < N) y[r] = (uint16_t)h[r];
        }
      }
    }
  }
}

// --------------------------------------------------------------- W8A16
// int8 weight byte q -> fp16 q exactly: the biased byte u = q + 128 under the
// high byte 0x64 is the fp16 value 1024 + u; subtracting 1152 leaves q.
__device__ __forceinline__ v8h i8x8_to_f16(uint32_t lo, uint32_t hi) {
  const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
  uint32_t w[4];
  w[0] = __builtin_amdgcn_perm(0x64646464u, a, 0x04010400u);
  w[1] = __builtin_amdgcn_perm(0x64646464u, a, 0x04030402u);
  w[2] = __builtin_amdgcn_perm(0x64646464u, b, 0x04010400u);
  w[3] = __builtin_amdgcn_perm(0x64646464u, b, 0x04030402u);
  v8h r;
  const v2h bias = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v2h h = __builtin_bit_cast(v2h, w[i]) - bias;
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

template <int MF, int FNW, int SK>
__global__ __launch_bounds__(64 * SK) void k_decode_w8a16(const uint16_t* __restrict__ x, const int8_t* __restrict__ W,
                                                          const float* __restrict__ ws, uint16_t* __restrict__ Y, int M,
                                                          int N, int K) {
  __shared__ v4f red[SK][FNW][MF][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int n0 = blockIdx.x * 16 * FNW;
  const int KB = K >> 7;

  const int8_t* wrow[FNW];
  const float* srow[FNW][4];
#pragma unroll
  for (int f = 0; f < FNW; ++f) {
    int n = n0 + f * 16 + (lane & 15);
    n = n < N ? n : N - 1;
    wrow[f] = W + (int64_t)n * K + q * 16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int no = n0 + f * 16 + 4 * q + r;
      no = no < N ? no : N - 1;
      srow[f][r] = ws + (int64_t)no * KB;
    }
  }
  const uint16_t* xrow[MF];
  bool xval[MF];
#pragma unroll
  for (int j = 0; j < MF; ++j) {
    int m = j * 16 + (lane & 15);
    xval[j] = m < M;
    xrow[j] = x + (int64_t)(m < M ? m : M - 1) * K + q * 16;
  }

  v4f facc[FNW][MF];
#pragma unroll
  for (int f = 0; f < FNW; ++f)
#pragma unroll
    for (int j = 0; j < MF; ++j) facc[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  for (int g = wave; g < KB; g += SK) {
    // weights: two 16-byte loads per fragment (k = 64 h + 16 q + [0, 16))
    v4i wv[FNW][2];
#pragma unroll
    for (int f = 0; f < FNW; ++f) {
      wv[f][0] = ld16(wrow[f] + g * 128);
      wv[f][1] = ld16(wrow[f] + g * 128 + 64);
    }
    // activations: 8 halves per MFMA at k = 64 (t/2) + 16 q + 8 (t%2) + [0, 8)
    v8h xv[MF][4];
#pragma unroll
    for (int j = 0; j < MF; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        v8h v = *reinterpret_cast<const v8h*>(xrow[j] + g * 128 + (t >> 1) * 64 + (t & 1) * 8);
        xv[j][t] = xval[j] ? v : (v8h){0, 0, 0, 0, 0, 0, 0, 0};
      }
    float s[FNW][4];
#pragma unroll
    for (int f = 0; f < FNW; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[f][r] = srow[f][r][g];
#pragma unroll
    for (int f = 0; f < FNW; ++f) {
      v8h wh[4];
      wh[0] = i8x8_to_f16(wv[f][0][0], wv[f][0][1]);
      wh[1] = i8x8_to_f16(wv[f][0][2], wv[f][0][3]);
      wh[2] = i8x8_to_f16(wv[f][1][0], wv[f][1][1]);
      wh[3] = i8x8_to_f16(wv[f][1][2], wv[f][1][3]);
#pragma unroll
      for (int j = 0; j < MF; ++j) {
        v4f p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) p = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh[t], xv[j][t], p, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) facc[f][j][r] = __builtin_fmaf(s[f][r], p[r], facc[f][j][r]);
      }
    }
  }

#pragma unroll
  for (int f = 0; f < FNW; ++f)
#pragma unroll
    for (int j = 0; j < MF; ++j) red[wave][f][j][lane] = facc[f][j];
  __syncthreads();
  if (wave != 0) return;
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int f = 0; f < FNW; ++f) {
    const int n = n0 + f * 16 + 4 * q;
    if (n >= N) continue;
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      const int m = j * 16 + (lane & 15);
      if (m >= M) continue;
      v4f t = red[0][f][j][lane];
#pragma unroll
      for (int w = 1; w < SK; ++w) t += red[w][f][j][lane];
      uint16_t h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = __builtin_bit_cast(uint16_t, (_Float16)t[r]);
      uint16_t* y = Y + (int64_t)m * N + n;
      if (vec && n + 3 < N) {
        *reinterpret_cast<uint2*>(y) = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) y[r] = h[r];
      }
    }
  }
}

template <int MODE, int OUT>
hipError_t decode_dispatch(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y, int64_t M,
                           int64_t N, int64_t K, hipStream_t st) {
  constexpr int SK = 4;
  const int m = (int)M, n = (int)N, k = (int)K;
  if (M <= 16) {
    dim3 g((unsigned)((N + 15) / 16));
    hipLaunchKernelGGL((k_decode_w8a8<MODE, 1, 1, SK, OUT>), g, dim3(64 * SK), 0, st, A, sa, W, sw, Y, m, n, k);
  } else if (M <= 32) {
    dim3 g((unsigned)((N + 31) / 32));
    hipLaunchKernelGGL((k_decode_w8a8<MODE, 2, 2, SK, OUT>), g, dim3(64 * SK), 0, st, A, sa, W, sw, Y, m, n, k);
  } else {
    dim3 g((unsigned)((N + 63) / 64));
    hipLaunchKernelGGL((k_decode_w8a8<MODE, 4, 4, SK, OUT>), g, dim3(64 * SK), 0, st, A, sa, W, sw, Y, m, n, k);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_block_decode(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                                    OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  return out == OUT_BF16 ? decode_dispatch<0, OUT_BF16>(A, sa, W, sw, Y, M, N, K, st)
                         : decode_dispatch<0, OUT_F32>(A, sa, W, sw, Y, M, N, K, st);
}

hipError_t launch_gemm_channel_decode(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                                      OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  switch (out) {
    case OUT_BF16: return decode_dispatch<1, OUT_BF16>(A, sa, W, sw, Y, M, N, K, st);
    case OUT_F32: return decode_dispatch<1, OUT_F32>(A, sa, W, sw, Y, M, N, K, st);
    default: return decode_dispatch<1, OUT_I32>(A, sa, W, sw, Y, M, N, K, st);
  }
}

hipError_t launch_gemm_w8a16(const uint16_t* x, const int8_t* W, const float* s, uint16_t* Y, int64_t M, int64_t N,
                             int64_t K, hipStream_t st) {
  constexpr int SK = 4;
  const int m = (int)M, n = (int)N, k = (int)K;
  // Larger M runs as repeated 64-row slices.
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
    const int mm = (int)(M - m0 < 64 ? M - m0 : 64);
    const uint16_t* xs = x + m0 * K;
    uint16_t* ys = Y + m0 * N;
    if (mm <= 16) {
      hipLaunchKernelGGL((k_decode_w8a16<1, 1, SK>), dim3((unsigned)((N + 15) / 16)), dim3(64 * SK), 0, st, xs, W, s,
                         ys, mm, n, k);
    } else if (mm <= 32) {
      hipLaunchKernelGGL((k_decode_w8a16<2, 2, SK>), dim3((unsigned)((N + 31) / 32)), dim3(64 * SK), 0, st, xs, W, s,
                         ys, mm, n, k);
    } else {
      hipLaunchKernelGGL((k_decode_w8a16<4, 4, SK>), dim3((unsigned)((N + 63) / 64)), dim3(64 * SK), 0, st, xs, W, s,
                         ys, mm, n, k);
    }
    (void)m;
  }
  return hipGetLastError();
}

}  // namespace w8
