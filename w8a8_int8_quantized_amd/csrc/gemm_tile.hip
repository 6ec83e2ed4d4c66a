// Large-M INT8 GEMMs on gfx950 int8 MFMA (v_mfma_i32_16x16x64_i8).
//
// Method: "DeepSeek R1 INT8 quantisation in SGLang" (Meituan), section 2.3
// and its Figure 3.
//   channel-wise: Y = (A . W^T) * a_scale[m] * w_scale[n], one dequant in the
//                 epilogue after an all-integer K loop;
//   block-wise:   the int32 partial of every 128-wide K block is dequantised
//                 with a_scale[m][kb] * w_scale[n/128][kb] and accumulated in
//                 fp32 inside the K loop.
//
// Tiling (all operands K-contiguous, one 128-byte K block per pipeline stage):
//   * global -> registers -> LDS, two LDS stages (the load of block kb+1 is in
//     flight while block kb is multiplied), one barrier per K block;
//   * LDS rows are 128 bytes; 16-byte chunk c of row r sits at chunk c ^ (r & 7)
//     so the 8 lanes that read one ds_read_b128 phase hit 8 distinct bank groups;
//   * MFMA operand A is a 16-row slice of W and operand B a 16-row slice of the
//     activations, so each lane's 4 accumulators are 4 consecutive output
//     columns n of one output row m: contiguous 8/16-byte stores, one
//     activation scale per lane and fragment, and (block-wise) one weight
//     scale per wave since a wave's 128 columns lie in one 128-wide N block;
//   * workgroup ids are remapped so that each XCD (ids congruent mod 8) works
//     on a contiguous band of tiles, grouped 8 tiles tall in M, which keeps the
//     A and W panels it streams in its own L2.
#include "common.h"
#include "launch.h"

namespace w8 {
namespace {

constexpr int kBlockK = 128;

__device__ __forceinline__ int lane_off(int lane, int ks) {
  return (lane & 15) * 128 + ((((ks << 2) | (lane >> 4)) ^ (lane & 7)) << 4);
}

// Global -> registers: ROWS x 128 bytes of the K block kb, NT threads, 16 bytes
// per load.  Thread t loads column chunk t & 7 of rows (t >> 3) + (NT/8) i.
// Rows at or past rows_valid are clamped to the last valid row: they only feed
// output rows/columns that are never stored.
template <int ROWS, int NT>
__device__ __forceinline__ void g2r(const int8_t* __restrict__ tile, int K, int rows_valid, int kb, uint4* reg) {
  constexpr int PER = ROWS * 8 / NT;
  const char* b = reinterpret_cast<const char*>(tile) + kb * kBlockK + (threadIdx.x & 7) * 16;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int r = r0 + (NT / 8) * i;
    r = r < rows_valid ? r : rows_valid - 1;
    reg[i] = *reinterpret_cast<const uint4*>(b + r * K);
  }
}

template <int ROWS, int NT>
__device__ __forceinline__ void r2s(char* lds, const uint4* reg) {
  constexpr int PER = ROWS * 8 / NT;
  const int c = threadIdx.x & 7;
  const int r0 = threadIdx.x >> 3;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int r = r0 + (NT / 8) * i;
    *reinterpret_cast<uint4*>(lds + r * 128 + ((c ^ (r & 7)) << 4)) = reg[i];
  }
}

__device__ __forceinline__ v4i frag(const char* lds, int row_base, int loff) {
  return *reinterpret_cast<const v4i*>(lds + row_base * 128 + loff);
}

__device__ __forceinline__ v4i mfma(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

struct Tile {
  int tm, tn;
};

// XCD-aware tile order: the hardware places workgroup b on XCD b % 8; tiles
// [x*T/8, (x+1)*T/8) go to XCD x, and inside that band tiles run 8 tall in M.
__device__ __forceinline__ Tile map_tile(int b, int TM, int TN) {
  const int T = TM * TN;
  const int x = b & 7, j = b >> 3;
  const int T8 = T >> 3, rem = T & 7;
  const int t = x * T8 + (x < rem ? x : rem) + j;
  constexpr int GM = 8;
  const int per = GM * TN;
  const int g = t / per;
  const int first = g * GM;
  const int gm = TM - first < GM ? TM - first : GM;
  const int r = t - g * per;
  Tile tl;
  tl.tm = first + r % gm;
  tl.tn = r / gm;
  return tl;
}

// Store 4 consecutive outputs Y[m][n..n+3] (n multiple of 4).
template <int OUT>
__device__ __forceinline__ void store4(void* Y, int64_t idx, int n, int N, bool vec, float a, float b, float c, float d) {
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
    uint32_t ha = f32_to_bf16_rne(a), hb = f32_to_bf16_rne(b), hc = f32_to_bf16_rne(c), hd = f32_to_bf16_rne(d);
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

// ------------------------------------------------------------ channel-wise
// 256 x 256 output tile, 4 waves in a 2 (n) x 2 (m) grid, 128 x 128 per wave
// (8 x 8 MFMA fragments, 256 int32 accumulators per lane).
constexpr int kChBM = 256, kChBN = 256;

template <int OUT>
__global__ __launch_bounds__(256, 1) void k_gemm_channel(const int8_t* __restrict__ A, const float* __restrict__ sa,
                                                         const int8_t* __restrict__ W, const float* __restrict__ sw,
                                                         void* __restrict__ Y, int M, int N, int K, int TM, int TN) {
  __shared__ __attribute__((aligned(16))) char smem[2][(kChBM + kChBN) * 128];
  const Tile tl = map_tile(blockIdx.x, TM, TN);
  const int m0 = tl.tm * kChBM, n0 = tl.tn * kChBN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int8_t* Ab = A + (int64_t)m0 * K;
  const int8_t* Wb = W + (int64_t)n0 * K;
  const int mval = M - m0 < kChBM ? M - m0 : kChBM;
  const int nval = N - n0 < kChBN ? N - n0 : kChBN;
  const int KB = K >> 7;

  v4i acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

  uint4 ra[8], rw[8];
  g2r<kChBM, 256>(Ab, K, mval, 0, ra);
  g2r<kChBN, 256>(Wb, K, nval, 0, rw);
  r2s<kChBM, 256>(smem[0], ra);
  r2s<kChBN, 256>(smem[0] + kChBM * 128, rw);
  __syncthreads();
  const int lo0 = lane_off(lane, 0), lo1 = lane_off(lane, 1);

  for (int kb = 0; kb < KB; ++kb) {
    const char* cur = smem[kb & 1];
    const bool more = kb + 1 < KB;
    if (more) {
      g2r<kChBM, 256>(Ab, K, mval, kb + 1, ra);
      g2r<kChBN, 256>(Wb, K, nval, kb + 1, rw);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int lo = ks ? lo1 : lo0;
      v4i wf[8], af[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) wf[i] = frag(cur + kChBM * 128, wn * 128 + i * 16, lo);
#pragma unroll
      for (int j = 0; j < 8; ++j) af[j] = frag(cur, wm * 128 + j * 16, lo);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma(wf[i], af[j], acc[i][j]);
    }
    if (more) {
      char* nxt = smem[(kb + 1) & 1];
      r2s<kChBM, 256>(nxt, ra);
      r2s<kChBN, 256>(nxt + kChBM * 128, rw);
    }
    __syncthreads();
  }

  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = m0 + wm * 128 + j * 16 + (lane & 15);
    if (m >= M) continue;
    const float s_m = OUT == OUT_I32 ? 0.f : sa[m];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + wn * 128 + i * 16 + 4 * (lane >> 4);
      if (n >= N) continue;
      const int64_t idx = (int64_t)m * N + n;
      if (OUT == OUT_I32) {
        store4i(static_cast<int32_t*>(Y) + idx, n, N, vec, acc[i][j]);
      } else {
        float s4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) s4[r] = n + r < N ? __fmul_rn(s_m, sw[n + r]) : 0.f;
        store4<OUT>(Y, idx, n, N, vec, __fmul_rn((float)acc[i][j][0], s4[0]), __fmul_rn((float)acc[i][j][1], s4[1]),
                    __fmul_rn((float)acc[i][j][2], s4[2]), __fmul_rn((float)acc[i][j][3], s4[3]));
      }
    }
  }
}

// -------------------------------------------------------------- block-wise
// 128 (m) x 256 (n) output tile, 4 waves in a 2 (n) x 2 (m) grid, 64 (m) x
// 128 (n) per wave.  Per K block each fragment pair is two chained MFMAs from
// zero (the exact int32 partial P), then acc += (a_scale * w_scale) * P on the
// VALU, interleaved with the next fragment's MFMAs.
constexpr int kBkBM = 128, kBkBN = 256;
enum { MODE_DEQUANT = 0, MODE_PARTIALS = 1, MODE_GROUPED = 2 };

// For the grouped GEMM: find which (expert, 128-row slice) this workgroup's
// linear m-tile index falls in.  Each expert e owns rows [off[e], off[e+1]) of
// the expert-sorted activations and ceil(count / 128) m-tiles.
struct GroupTile {
  int e, r0, r1;   // expert and row range of this tile; e < 0: no tile
};

__device__ GroupTile grouped_lookup(const int32_t* __restrict__ off, int E, int P, int tmg) {
  __shared__ int scan[256];
  __shared__ int sel[3];
  const int t = threadIdx.x;
  const int ept = (E + 255) >> 8;
  const int e0 = t * ept;
  const int e1 = e0 + ept < E ? e0 + ept : E;
  int cnt = 0;
  for (int e = e0; e < e1; ++e) {
    int lo = off[e], hi = off[e + 1];
    lo = lo < 0 ? 0 : (lo > P ? P : lo);
    hi = hi < lo ? lo : (hi > P ? P : hi);
    cnt += (hi - lo + kBkBM - 1) / kBkBM;
  }
  if (t == 0) sel[0] = -1;
  scan[t] = cnt;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    int v = t >= d ? scan[t - d] : 0;
    __syncthreads();
    scan[t] += v;
    __syncthreads();
  }
  const int excl = scan[t] - cnt;
  if (tmg >= excl && tmg < excl + cnt) {
    int acc = excl;
    for (int e = e0; e < e1; ++e) {
      int lo = off[e], hi = off[e + 1];
      lo = lo < 0 ? 0 : (lo > P ? P : lo);
      hi = hi < lo ? lo : (hi > P ? P : hi);
      int c = (hi - lo + kBkBM - 1) / kBkBM;
      if (tmg < acc + c) {
        int r0 = lo + (tmg - acc) * kBkBM;
        sel[0] = e;
        sel[1] = r0;
        sel[2] = r0 + kBkBM < hi ? r0 + kBkBM : hi;
        break;
      }
      acc += c;
    }
  }
  __syncthreads();
  GroupTile g;
  g.e = sel[0];
  g.r0 = sel[1];
  g.r1 = sel[2];
  return g;
}

template <int MODE, int OUT>
__global__ __launch_bounds__(256, 1) void k_gemm_block(const int8_t* __restrict__ A, const float* __restrict__ sa,
                                                       const int8_t* __restrict__ W, const float* __restrict__ sw,
                                                       const int32_t* __restrict__ offsets, void* __restrict__ Y,
                                                       int M, int N, int K, int TM, int TN, int E) {
  __shared__ __attribute__((aligned(16))) char smem[2][(kBkBM + kBkBN) * 128];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  const int KB = K >> 7;
  const int NB = (N + 127) >> 7;

  int m0, mrows, n0;
  const int8_t* Wx = W;
  const float* swx = sw;
  if (MODE == MODE_GROUPED) {
    const int tmg = blockIdx.x / TN;
    n0 = (blockIdx.x - tmg * TN) * kBkBN;
    GroupTile g = grouped_lookup(offsets, E, M, tmg);
    if (g.e < 0) return;
    m0 = g.r0;
    mrows = g.r1 - g.r0;
    Wx = W + (int64_t)g.e * N * K;
    swx = sw + (int64_t)g.e * NB * KB;
  } else {
    const Tile tl = map_tile(blockIdx.x, TM, TN);
    m0 = tl.tm * kBkBM;
    n0 = tl.tn * kBkBN;
    mrows = M - m0 < kBkBM ? M - m0 : kBkBM;
  }
  const int nval = N - n0 < kBkBN ? N - n0 : kBkBN;
  const int8_t* Ab = A + (int64_t)m0 * K;
  const int8_t* Wb = Wx + (int64_t)n0 * K;

  // this wave's 128 columns lie in one 128-wide N block
  int nbw = (n0 + wn * 128) >> 7;
  nbw = nbw < NB ? nbw : NB - 1;
  const float* sw_row = swx + (int64_t)nbw * KB;
  // the activation rows of this lane's 4 m-fragments (clamped for loads)
  int mrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int r = wm * 64 + j * 16 + (lane & 15);
    mrow[j] = m0 + (r < mrows ? r : mrows - 1);
  }

  v4f facc[8][4];
  if (MODE != MODE_PARTIALS) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) facc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};
  }

  uint4 ra[4], rw[8];
  g2r<kBkBM, 256>(Ab, K, mrows, 0, ra);
  g2r<kBkBN, 256>(Wb, K, nval, 0, rw);
  r2s<kBkBM, 256>(smem[0], ra);
  r2s<kBkBN, 256>(smem[0] + kBkBM * 128, rw);
  __syncthreads();
  const int lo0 = lane_off(lane, 0), lo1 = lane_off(lane, 1);
  const bool vec = (N & 3) == 0;

  for (int kb = 0; kb < KB; ++kb) {
    const char* cur = smem[kb & 1];
    const bool more = kb + 1 < KB;
    if (more) {
      g2r<kBkBM, 256>(Ab, K, mrows, kb + 1, ra);
      g2r<kBkBN, 256>(Wb, K, nval, kb + 1, rw);
    }
    float s[4];
    if (MODE != MODE_PARTIALS) {
      const float swv = sw_row[kb];
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] = __fmul_rn(sa[(int64_t)mrow[j] * KB + kb], swv);
    }
    v4i wf0[8], wf1[8], af0[4], af1[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      wf0[i] = frag(cur + kBkBM * 128, wn * 128 + i * 16, lo0);
      wf1[i] = frag(cur + kBkBM * 128, wn * 128 + i * 16, lo1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      af0[j] = frag(cur, wm * 64 + j * 16, lo0);
      af1[j] = frag(cur, wm * 64 + j * 16, lo1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v4i p = mfma(wf0[i], af0[j], (v4i){0, 0, 0, 0});
        p = mfma(wf1[i], af1[j], p);
        if (MODE == MODE_PARTIALS) {
          const int m = m0 + wm * 64 + j * 16 + (lane & 15);
          const int n = n0 + wn * 128 + i * 16 + 4 * (lane >> 4);
          if (m < M && n < N) store4i(static_cast<int32_t*>(Y) + ((int64_t)kb * M + m) * N + n, n, N, vec, p);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) facc[i][j][r] = __builtin_fmaf(s[j], (float)p[r], facc[i][j][r]);
        }
      }
    }
    if (more) {
      char* nxt = smem[(kb + 1) & 1];
      r2s<kBkBM, 256>(nxt, ra);
      r2s<kBkBN, 256>(nxt + kBkBM * 128, rw);
    }
    __syncthreads();
  }

  if (MODE == MODE_PARTIALS) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ml = wm * 64 + j * 16 + (lane & 15);
    if (ml >= mrows) continue;
    const int m = m0 + ml;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int n = n0 + wn * 128 + i * 16 + 4 * (lane >> 4);
      if (n >= N) continue;
      store4<OUT>(Y, (int64_t)m * N + n, n, N, vec, facc[i][j][0], facc[i][j][1], facc[i][j][2], facc[i][j][3]);
    }
  }
}

}  // namespace

hipError_t launch_gemm_channel(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                               OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M <= 64) return launch_gemm_channel_decode(A, sa, W, sw, Y, out, M, N, K, st);
  const int TM = (int)((M + kChBM - 1) / kChBM), TN = (int)((N + kChBN - 1) / kChBN);
  dim3 grid((unsigned)(TM * TN)), block(256);
  switch (out) {
    case OUT_BF16:
      hipLaunchKernelGGL((k_gemm_channel<OUT_BF16>), grid, block, 0, st, A, sa, W, sw, Y, (int)M, (int)N, (int)K, TM, TN);
      break;
    case OUT_F32:
      hipLaunchKernelGGL((k_gemm_channel<OUT_F32>), grid, block, 0, st, A, sa, W, sw, Y, (int)M, (int)N, (int)K, TM, TN);
      break;
    default:
      hipLaunchKernelGGL((k_gemm_channel<OUT_I32>), grid, block, 0, st, A, sa, W, sw, Y, (int)M, (int)N, (int)K, TM, TN);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_block(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                             OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (M <= 64) return launch_gemm_block_decode(A, sa, W, sw, Y, out, M, N, K, st);
  const int TM = (int)((M + kBkBM - 1) / kBkBM), TN = (int)((N + kBkBN - 1) / kBkBN);
  dim3 grid((unsigned)(TM * TN)), block(256);
  if (out == OUT_BF16)
    hipLaunchKernelGGL((k_gemm_block<MODE_DEQUANT, OUT_BF16>), grid, block, 0, st, A, sa, W, sw, nullptr, Y, (int)M,
                       (int)N, (int)K, TM, TN, 0);
  else
    hipLaunchKernelGGL((k_gemm_block<MODE_DEQUANT, OUT_F32>), grid, block, 0, st, A, sa, W, sw, nullptr, Y, (int)M,
                       (int)N, (int)K, TM, TN, 0);
  return hipGetLastError();
}

hipError_t launch_gemm_block_partials(const int8_t* A, const int8_t* W, int32_t* P, int64_t M, int64_t N, int64_t K,
                                      hipStream_t st) {
  const int TM = (int)((M + kBkBM - 1) / kBkBM), TN = (int)((N + kBkBN - 1) / kBkBN);
  hipLaunchKernelGGL((k_gemm_block<MODE_PARTIALS, OUT_I32>), dim3((unsigned)(TM * TN)), dim3(256), 0, st, A, nullptr,
                     W, nullptr, nullptr, P, (int)M, (int)N, (int)K, TM, TN, 0);
  return hipGetLastError();
}

hipError_t launch_gemm_block_grouped(const int8_t* A, const float* sa, const int8_t* W, const float* sw,
                                     const int32_t* offsets, void* Y, OutKind out, int64_t E, int64_t P, int64_t N,
                                     int64_t K, hipStream_t st) {
  // upper bound on the number of 128-row m-tiles over all experts
  const int64_t TMmax = (P + kBkBM - 1) / kBkBM + E;
  const int TN = (int)((N + kBkBN - 1) / kBkBN);
  dim3 grid((unsigned)(TMmax * TN)), block(256);
  if (out == OUT_BF16)
    hipLaunchKernelGGL((k_gemm_block<MODE_GROUPED, OUT_BF16>), grid, block, 0, st, A, sa, W, sw, offsets, Y, (int)P,
                       (int)N, (int)K, (int)TMmax, TN, (int)E);
  else
    hipLaunchKernelGGL((k_gemm_block<MODE_GROUPED, OUT_F32>), grid, block, 0, st, A, sa, W, sw, offsets, Y, (int)P,
                       (int)N, (int)K, (int)TMmax, TN, (int)E);
  return hipGetLastError();
}

}  // namespace w8
