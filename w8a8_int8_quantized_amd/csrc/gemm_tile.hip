// Large-M channel-wise INT8 GEMM on gfx950 int8 MFMA, and the split-K
// workspace shared with the block-wise tiles (gemm_block.hip).
//
// Method: "DeepSeek R1 INT8 quantisation in SGLang" (Meituan), section 2.3
// and its Figure 3, channel-wise scheme: Y = (A . W^T) * a_scale[m] *
// w_scale[n]: an all-integer K loop, one dequantisation in the epilogue.
//
// Data path (see pipeline.h): K blocks of 128 bytes per row stream
// global -> LDS through direct-to-LDS buffer loads into a two-slot ring; the
// load of block kb+1 is in flight while block kb is multiplied.  MFMA operand
// A is a slice of W and operand B a slice of the activations, so each lane's
// accumulators are consecutive output columns n of one output row m:
// contiguous stores and one activation scale per lane and fragment.
#include <mutex>
#include <vector>

#include "tile_common.h"

namespace w8 {
namespace {

// ------------------------------------------------------------ channel-wise
// 256 (m) x BN (n) output tile per workgroup, BN = 32 FN (FN = 8, 7 or 6);
// 4 waves in a 2 (n) x 2 (m) grid, each wave 16 FN x 128 (FN x 8 fragments
// of v_mfma_i32_16x16x64_i8, up to 256 int32 accumulators per lane in
// AGPRs).  An LDS slot holds one K block: A 256 x 128 B then W BN x 128 B.
// The loop runs over 64-wide K steps; the fragments of step t+1 are read
// from LDS while step t's MFMAs run, and every second step (a K block
// boundary) waits for the next block's DMA, synchronises, and starts the DMA
// of the block after it.  Narrower tiles let the launcher fill the last
// round of workgroups (e.g. N = 7168 at M = 4096: 448 tiles of width 256
// leave a quarter of the second round idle, 512 tiles of width 224 do not).
constexpr int kChBM = 256;

// AS: the epilogue of the asymmetric per-tensor activations (codes stored as
// q - 128, prm = {s, z}, wsum = per-row weight sums) in place of the
// channel-wise one: Y = fp32(fp32(s * sw[n]) * fp32(fp32(ACC + 128 WS[n]) -
// fp32(z * fp32(WS[n])))).
template <int OUT, int FN, bool AS = false>
__global__ __launch_bounds__(256, 1) void k_gemm_channel(const int8_t* __restrict__ A, const float* __restrict__ sa,
                                                         const int8_t* __restrict__ W, const float* __restrict__ sw,
                                                         void* __restrict__ Y, int M, int N, int K, int TM,
                                                         const float* __restrict__ prm = nullptr,
                                                         const int32_t* __restrict__ wsum = nullptr) {
  constexpr int kChBN = 32 * FN;
  constexpr int kChStage = (kChBM + kChBN) * 128;
  // two stages, or the bf16 epilogue's 256 rows of 512 bytes
  constexpr int kSmem = 2 * kChStage > kChBM * 512 ? 2 * kChStage : kChBM * 512;
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave & 1, wm = wave >> 1;
  int tm, tn;
  xcd_tile(blockIdx.x, TM, (int)gridDim.x / TM, tm, tn);
  const int m0 = tm * kChBM, n0 = tn * kChBN;
  const int mval = M - m0 < kChBM ? M - m0 : kChBM;
  const int nval = N - n0 < kChBN ? N - n0 : kChBN;
  // split-K: slice blockIdx.y of gridDim.y covers K blocks kbs .. kbe - 1 and
  // writes its raw int32 tile to slice blockIdx.y of Y (M x N each)
  const int KBt = K >> 7;
  const int kbs = (int)((int64_t)blockIdx.y * KBt / gridDim.y);
  const int kbe = (int)((int64_t)(blockIdx.y + 1) * KBt / gridDim.y);
  Y = static_cast<void*>(static_cast<int32_t*>(Y) + (int64_t)blockIdx.y * M * N);
  // the slice's first K block is the descriptors' origin; rows past the tile
  // still fall outside their range
  const v4i ra = make_rsrc(A + (int64_t)m0 * K + kbs * 128, (uint32_t)(mval * K - kbs * 128));
  const v4i rw = make_rsrc(W + (int64_t)n0 * K + kbs * 128, (uint32_t)(nval * K - kbs * 128));
  const int voff = wave * 64 * K + dma_lane_off(lane, K);        // wave fills A rows 64*wave .. +63
  const int voffw = wave * 8 * FN * K + dma_lane_off(lane, K);   // and W rows 8*FN*wave .. +8*FN-1
  const uint32_t lds0 = lds_addr(smem);
  const int NK = kbe - kbs;
  const int K8 = 8 * K;
  const int lo0 = frag_off(lane & 15, lane >> 4);           // 16x16x64 operand: row l%16, chunk l/16
  const int lo1 = frag_off(lane & 15, 4 + (lane >> 4));

  v4i acc[FN][8];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

#define CH_DMA(T)                                                                                  \
  {                                                                                               \
    const uint32_t base = lds0 + ((T) & 1) * kChStage;                                            \
    _Pragma("unroll") for (int b = 0; b < 8; ++b)                                                 \
      dma16(ra, voff, b * K8 + (T) * 128, base + wave * 8192 + b * 1024);                         \
    _Pragma("unroll") for (int b = 0; b < FN; ++b)                                                \
      dma16(rw, voffw, b * K8 + (T) * 128, base + kChBM * 128 + wave * FN * 1024 + b * 1024);     \
  }
#define CH_RD(KS, WF, AF)                                                                          \
  {                                                                                               \
    const char* buf = smem + (((KS) >> 1) & 1) * kChStage;                                        \
    const int lo = ((KS) & 1) ? lo1 : lo0;                                                        \
    _Pragma("unroll") for (int j = 0; j < 8; ++j) AF[j] = *(const v4i*)(buf + (wm * 128 + j * 16) * 128 + lo); \
    _Pragma("unroll") for (int i = 0; i < FN; ++i)                                                \
      WF[i] = *(const v4i*)(buf + kChBM * 128 + (wn * 16 * FN + i * 16) * 128 + lo);              \
  }

  CH_DMA(0)
  waitcnt<0, 15>();
  barrier();
  if (1 < NK) CH_DMA(1)
  v4i wc[FN], ac[8];
  CH_RD(0, wc, ac)
  for (int t = 0; t < 2 * NK; ++t) {
    if (t & 1) {
      // step t+1 opens K block (t+1)/2, whose DMA was started two steps ago
      waitcnt<0, 0>();
      barrier();
      if (((t + 1) >> 1) + 1 < NK) CH_DMA(((t + 1) >> 1) + 1)
    }
    v4i wn_[FN], an_[8];
    CH_RD(t + 1, wn_, an_)
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wc[i], ac[j], acc[i][j], 0, 0, 0);
    // one LDS read for the next step after every 4 MFMAs (the last reads of
    // a narrower tile trail the MFMAs)
#pragma unroll
    for (int g = 0; g < FN + 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ac[j] = an_[j];
#pragma unroll
    for (int i = 0; i < FN; ++i) wc[i] = wn_[i];
  }
#undef CH_DMA
#undef CH_RD
  // every load, and the loop's last (unused) look-ahead read, has landed
  waitcnt<0, 0>();

  const bool vec = (N & 3) == 0;
  if (OUT == OUT_I32) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = m0 + wm * 128 + j * 16 + (lane & 15);
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = n0 + wn * 16 * FN + i * 16 + 4 * (lane >> 4);
        if (n < N) store4i(static_cast<int32_t*>(Y) + (int64_t)m * N + n, n, N, vec, acc[i][j]);
      }
    }
    return;
  }
  // this lane's 8 activation scales and 8 x 4 weight scales, all loads in
  // flight at once (asymmetric: per column fp32(s * sw), fp32(z * WS) and
  // 128 WS instead)
  float sam[8], swn[FN][4], zw[FN][4];
  int wsx[FN][4];
  if (!AS) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = m0 + wm * 128 + j * 16 + (lane & 15);
      sam[j] = m < M ? sa[m] : 0.f;
    }
  }
  const float as_s = AS ? prm[0] : 0.f, as_z = AS ? prm[1] : 0.f;
#pragma unroll
  for (int i = 0; i < FN; ++i) {
    const int n = n0 + wn * 16 * FN + i * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      swn[i][r] = n + r < N ? sw[n + r] : 0.f;
      if (AS) {
        const int ws = n + r < N ? wsum[n + r] : 0;
        swn[i][r] = __fmul_rn(as_s, swn[i][r]);
        zw[i][r] = __fmul_rn(as_z, (float)ws);
        wsx[i][r] = 128 * ws;
      }
    }
  }
  // output value of accumulator r of fragment (i, j)
  auto outv = [&](int i, int j, int r) -> float {
    if (AS) return __fmul_rn(swn[i][r], __fsub_rn((float)(acc[i][j][r] + wsx[i][r]), zw[i][r]));
    return __fmul_rn((float)acc[i][j][r], __fmul_rn(sam[j], swn[i][r]));
  };
  if (OUT == OUT_F32) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = m0 + wm * 128 + j * 16 + (lane & 15);
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = n0 + wn * 16 * FN + i * 16 + 4 * (lane >> 4);
        if (n >= N) continue;
        float o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = outv(i, j, r);
        store4<OUT_F32>(Y, (int64_t)m * N + n, n, N, vec, o[0], o[1], o[2], o[3]);
      }
    }
    return;
  }
  // bf16: the tile goes through LDS (free now: the barrier below also means
  // every wave is past its last stage read) so that it leaves in whole rows.
  // Tile row r holds BN bf16 in a 512-byte pitch; its 16-byte chunk c is
  // stored at c ^ (r & 15) (< 32), so the 16 rows a write instruction
  // touches, and the chunks a row read touches, fall in distinct bank groups.
  barrier();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = wm * 128 + j * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      uint32_t h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) h[q] = f32_to_bf16_rne(outv(i, j, q));
      const int chunk = wn * 2 * FN + 2 * i + (lane >> 5);
      *reinterpret_cast<uint2*>(smem + r * 512 + ((chunk ^ (r & 15)) << 4) + 8 * ((lane >> 4) & 1)) =
          make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    }
  }
  waitcnt<63, 0>();
  barrier();
  // wave w stores tile rows 64 w .. 64 w + 63, two rows per instruction;
  // lane: row half lane >> 5, columns 8 (lane & 31) .. + 7 (chunks past the
  // tile's BN columns are skipped)
  const int cl = lane & 31;
  const int n = n0 + 8 * cl;
  const bool vec8 = (N & 7) == 0 && n + 7 < N;
  const bool inside = cl < 4 * FN;
#pragma unroll 4
  for (int it = 0; it < 32; ++it) {
    const int r = wave * 64 + 2 * it + (lane >> 5);
    const int m = m0 + r;
    const v4i v = *reinterpret_cast<const v4i*>(smem + r * 512 + ((cl ^ (r & 15)) << 4));
    if (m >= M || n >= N || !inside) continue;
    uint16_t* y = static_cast<uint16_t*>(Y) + (int64_t)m * N + n;
    if (vec8) {
      *reinterpret_cast<v4i*>(y) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (n + e < N) y[e] = (uint16_t)(((uint32_t)v[e >> 1]) >> (16 * (e & 1)));
    }
  }
}

// ---------------------------------------------------------------- split-K
// Sum of the S slices' partial tiles, in slice order, then the output.
// Channel-wise: int32 slices (the sum is exact) and the channel epilogue
// fp32(fp32(acc) * fp32(sa[m] * sw[n])); block-wise: fp32 slices.  Each
// thread covers 4 consecutive outputs of one row.
template <int OUT>
__global__ __launch_bounds__(256) void k_splitk_sum_i32(const int32_t* __restrict__ ws, int S, int M, int N,
                                                        const float* __restrict__ sa, const float* __restrict__ sw,
                                                        void* __restrict__ Y) {
  const int64_t q4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nq = (N + 3) >> 2;
  if (q4 >= (int64_t)M * nq) return;
  const int m = (int)(q4 / nq), n = (int)(q4 - (int64_t)m * nq) * 4;
  const int64_t idx = (int64_t)m * N + n;
  const int64_t MN = (int64_t)M * N;
  v4i a = {0, 0, 0, 0};
  for (int sl = 0; sl < S; ++sl)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) a[r] += ws[sl * MN + idx + r];
  const bool vec = (N & 3) == 0;
  if (OUT == OUT_I32) {
    store4i(static_cast<int32_t*>(Y) + idx, n, N, vec, a);
  } else {
    float o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = n + r < N ? __fmul_rn((float)a[r], __fmul_rn(sa[m], sw[n + r])) : 0.f;
    store4<OUT>(Y, idx, n, N, vec, o[0], o[1], o[2], o[3]);
  }
}



// Tile width of the unsplit channel GEMM: FN 16-column fragments per wave
// (BN = 32 FN) in {8, 7, 6}, the smallest modelled time, where a tile costs
// per K block ~2960 FN / 8 cycles of MFMA issue and fragment reads plus
// ~16.5 cycles per 1 KB load instruction (32 for A, 4 FN for W), and the
// grid runs in rounds of 256 workgroups.  Ties keep the wider tile.
int pick_channel_width(int TM, int64_t N) {
  int best = 8;
  double best_t = 1e30;
  for (int fn = 8; fn >= 6; --fn) {
    const int64_t tiles = (int64_t)TM * ((N + 32 * fn - 1) / (32 * fn));
    const double t = (double)((tiles + 255) / 256) * (2960.0 * fn / 8.0 + 16.5 * (32 + 4 * fn));
    if (t < best_t * 0.98) {
      best_t = t;
      best = fn;
    }
  }
  return best;
}

template <int FN>
hipError_t channel_launch(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y, OutKind out,
                          int64_t M, int64_t N, int64_t K, int TM, hipStream_t st) {
  const int TN = (int)((N + 32 * FN - 1) / (32 * FN));
  const dim3 grid((unsigned)(TM * TN)), block(256);
  switch (out) {
    case OUT_BF16:
      hipLaunchKernelGGL((k_gemm_channel<OUT_BF16, FN>), grid, block, 0, st, A, sa, W, sw, Y, (int)M, (int)N, (int)K,
                         TM);
      break;
    case OUT_F32:
      hipLaunchKernelGGL((k_gemm_channel<OUT_F32, FN>), grid, block, 0, st, A, sa, W, sw, Y, (int)M, (int)N, (int)K,
                         TM);
      break;
    default:
      hipLaunchKernelGGL((k_gemm_channel<OUT_I32, FN>), grid, block, 0, st, A, sa, W, sw, Y, (int)M, (int)N, (int)K,
                         TM);
      break;
  }
  return hipGetLastError();
}

template <int FN>
hipError_t channel_asym_launch(const int8_t* A, const float* prm, const int8_t* W, const float* sw,
                               const int32_t* wsum, void* Y, OutKind out, int64_t M, int64_t N, int64_t K, int TM,
                               hipStream_t st) {
  const int TN = (int)((N + 32 * FN - 1) / (32 * FN));
  const dim3 grid((unsigned)(TM * TN)), block(256);
  if (out == OUT_F32)
    hipLaunchKernelGGL((k_gemm_channel<OUT_F32, FN, true>), grid, block, 0, st, A, nullptr, W, sw, Y, (int)M,
                       (int)N, (int)K, TM, prm, wsum);
  else
    hipLaunchKernelGGL((k_gemm_channel<OUT_BF16, FN, true>), grid, block, 0, st, A, nullptr, W, sw, Y, (int)M,
                       (int)N, (int)K, TM, prm, wsum);
  return hipGetLastError();
}

}  // namespace

// Per-(device, stream, slot) workspaces, grown on demand and kept until the
// process ends: slot 0 holds split-K partial tiles, slot 1 the asymmetric
// GEMM's int32 accumulators and its quantiser's partial ranges (a GEMM there
// may split K into slot 0 at the same time).  Calls on one stream are
// ordered, so they may share a slot; different streams get different buffers.
struct Workspace {
  int dev;
  hipStream_t st;
  int slot;
  void* p;
  size_t bytes;
};
namespace {
std::mutex g_ws_mu;
std::vector<Workspace> g_ws;
}  // namespace

// Number of K slices for a tile grid that leaves CUs idle: the smallest
// modelled time over S = 1..16, where a slice of KB / S blocks costs one
// round of workgroups per 256, t_kb microseconds per tile and K block, and
// splitting adds the slices' partial tiles through HBM (written and read,
// 8 bytes per output per slice at ~5 TB/s) plus a reduction launch.
int pick_k_slices(int64_t tiles, int64_t KB, int64_t M, int64_t N, double t_kb_us) {
  int best = 1;
  double best_t = 1e30;
  for (int S = 1; S <= 16 && S <= KB; ++S) {
    const int64_t rounds = (tiles * S + 255) / 256;
    double t = (double)rounds * ((double)KB / S) * t_kb_us;
    if (S > 1) t += (double)S * M * N * 8.0 / 5.0e6 + 3.0;
    if (t < best_t * 0.97) {
      best_t = t;
      best = S;
    }
  }
  return best;
}

hipError_t split_workspace(hipStream_t st, size_t bytes, void** out) { return stream_workspace(st, 0, bytes, out); }

hipError_t stream_workspace(hipStream_t st, int slot, size_t bytes, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (Workspace& w : g_ws) {
    if (w.dev == dev && w.st == st && w.slot == slot) {
      if (w.bytes < bytes) {
        // the stream's earlier kernels may still read the old buffer
        e = hipStreamSynchronize(st);
        if (e != hipSuccess) return e;
        e = hipFree(w.p);
        if (e != hipSuccess) return e;
        w.p = nullptr;
        w.bytes = 0;
        e = hipMalloc(&w.p, bytes);
        if (e != hipSuccess) return e;
        w.bytes = bytes;
      }
      *out = w.p;
      return hipSuccess;
    }
  }
  void* p = nullptr;
  e = hipMalloc(&p, bytes);
  if (e != hipSuccess) return e;
  g_ws.push_back({dev, st, slot, p, bytes});
  *out = p;
  return hipSuccess;
}

bool channel_tiles_unsplit(int64_t M, int64_t N, int64_t K) {
  if (decode_path_takes(M, N, true)) return false;
  const int TM = (int)((M + kChBM - 1) / kChBM), TN = (int)((N + 255) / 256);
  return pick_k_slices((int64_t)TM * TN, K >> 7, M, N, 2.2) == 1;
}

hipError_t launch_gemm_channel_asym_tiles(const int8_t* A, const float* prm, const int8_t* W, const float* sw,
                                          const int32_t* wsum, void* Y, OutKind out, int64_t M, int64_t N,
                                          int64_t K, hipStream_t st) {
  const int TM = (int)((M + kChBM - 1) / kChBM);
  switch (pick_channel_width(TM, N)) {
    case 7: return channel_asym_launch<7>(A, prm, W, sw, wsum, Y, out, M, N, K, TM, st);
    case 6: return channel_asym_launch<6>(A, prm, W, sw, wsum, Y, out, M, N, K, TM, st);
    default: return channel_asym_launch<8>(A, prm, W, sw, wsum, Y, out, M, N, K, TM, st);
  }
}

hipError_t launch_gemm_channel(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                               OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (decode_path_takes(M, N, true)) return launch_gemm_channel_decode(A, sa, W, sw, Y, out, M, N, K, st);
  const int TM = (int)((M + kChBM - 1) / kChBM), TN = (int)((N + 255) / 256);
  // ~2.2 us per 256 x 256 tile and K block at the measured large-M rate
  const int S = pick_k_slices((int64_t)TM * TN, K >> 7, M, N, 2.2);
  if (S > 1) {
    void* ws = nullptr;
    hipError_t e = split_workspace(st, (size_t)S * M * N * 4, &ws);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemm_channel<OUT_I32, 8>), dim3((unsigned)(TM * TN), (unsigned)S), dim3(256), 0, st, A, sa,
                       W, sw, ws, (int)M, (int)N, (int)K, TM);
    const dim3 rg((unsigned)((M * ((N + 3) / 4) + 255) / 256));
    const int32_t* wsi = static_cast<const int32_t*>(ws);
    switch (out) {
      case OUT_BF16:
        hipLaunchKernelGGL((k_splitk_sum_i32<OUT_BF16>), rg, dim3(256), 0, st, wsi, S, (int)M, (int)N, sa, sw, Y);
        break;
      case OUT_F32:
        hipLaunchKernelGGL((k_splitk_sum_i32<OUT_F32>), rg, dim3(256), 0, st, wsi, S, (int)M, (int)N, sa, sw, Y);
        break;
      default:
        hipLaunchKernelGGL((k_splitk_sum_i32<OUT_I32>), rg, dim3(256), 0, st, wsi, S, (int)M, (int)N, sa, sw, Y);
        break;
    }
    return hipGetLastError();
  }
  const int FN = pick_channel_width(TM, N);
  switch (FN) {
    case 7: return channel_launch<7>(A, sa, W, sw, Y, out, M, N, K, TM, st);
    case 6: return channel_launch<6>(A, sa, W, sw, Y, out, M, N, K, TM, st);
    default: return channel_launch<8>(A, sa, W, sw, Y, out, M, N, K, TM, st);
  }
}

}  // namespace w8
