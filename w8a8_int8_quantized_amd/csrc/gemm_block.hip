// Large-M block-wise INT8 GEMM on gfx950 int8 MFMA (dense and grouped/MoE).
//
// Method: "DeepSeek R1 INT8 quantisation in SGLang" (Meituan), section 2.3
// and its Figure 3, block-wise scheme: the int32 partial P of every 128-deep
// K block is dequantised with a_scale[m][kb] * w_scale[n / 128][kb] and
// accumulated in fp32 inside the K loop:
//   acc[m][n] += (a_scale[m][kb] * w_scale[n / 128][kb]) * P_kb[m][n].
//
// Tile: 256 (n) x BM (m), BM = 64 NWM, 2 NWM waves in a 2 (n) x NWM (m) grid,
// each wave 128 (n) x 64 (m) as 4 x 2 fragments ("chains") of
// v_mfma_i32_32x32x32_i8; a chain is four MFMAs over one K block (its exact
// int32 P), then 16 cvt + 16 fma per lane dequantise it into the wave's fp32
// accumulators, which stay in VGPRs.  Operands stream global -> LDS through
// direct-to-LDS loads into a two-slot ring (pipeline.h), one K block per slot.
//
// Software pipeline: the MFMAs of chain t run interleaved with the
// dequantisation of chain t - 1 (one MFMA, then eight VALU ops, pinned with
// sched_group_barrier), and the W fragments of the next chain pair are read
// from LDS two chains ahead; the last chain of a K block is dequantised while
// the next block's first MFMAs run.  The MFMA results must land in VGPRs for
// the VALU: this file is compiled with the backend's VGPR-form MFMA option
// (AGPR results would cost one v_accvgpr_read per output).  At NWM = 4 two
// waves share each SIMD and the 256 x 256 tile moves 1 KB of operands per
// 2^20 MACs; NWM = 2 (128-row tiles) serves small M and MoE experts with few
// rows.
#include <type_traits>

#include "grouped.h"
#include "tile_common.h"

namespace w8 {
namespace {

enum { MODE_DEQUANT = 0, MODE_PARTIALS = 1, MODE_GROUPED = 2 };
constexpr int kTileCUs = 256;   // compute units the tile grids are sized against

// MODE_DEQUANT: dense; gridDim.y > 1 splits K into slices, slice y writing
// its fp32 partial tile to slice y of Y (M x N floats each; OUT_F32 then).
// MODE_GROUPED: the rows of A / Y are expert-sorted (offsets), W and w_scale
// hold E experts; tile b / TN is the expert tile number.
// MODE_PARTIALS: Y gets every K block's raw int32 partial, Y[kb][m][n].
template <int MODE, int OUT, int NWM>
__global__ __launch_bounds__(128 * NWM, 1) void k_gemm_block(const int8_t* __restrict__ A, const float* __restrict__ sa,
                                                             const int8_t* __restrict__ W, const float* __restrict__ sw,
                                                             const int32_t* __restrict__ offsets, void* __restrict__ Y,
                                                             int M, int N, int K, int TM, int TN, int E) {
  constexpr int BM = 64 * NWM, BN = 256, NWV = 2 * NWM;
  constexpr int STG = (BM + BN) * 128;
  constexpr int AI = BM / (8 * NWV);   // DMA instructions per wave per K block for A (= 4)
  constexpr int WI = BN / (8 * NWV);   // ... and for W
  constexpr bool DQ = MODE != MODE_PARTIALS;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STG];
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
    n0 = (blockIdx.x - tmg * TN) * BN;
    const ExpertTile g = group_tile<BM>(offsets, E, M, tmg);
    if (g.e < 0) return;
    m0 = g.r0;
    mrows = g.r1 - g.r0;
    Wx = W + (int64_t)g.e * N * K;
    swx = sw + (int64_t)g.e * NB * KB;
  } else {
    int tm, tn;
    xcd_tile(blockIdx.x, TM, TN, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
    mrows = M - m0 < BM ? M - m0 : BM;
  }
  const int nval = N - n0 < BN ? N - n0 : BN;
  const int kbs = (int)((int64_t)blockIdx.y * KB / gridDim.y);
  const int kbe = (int)((int64_t)(blockIdx.y + 1) * KB / gridDim.y);
  if (MODE == MODE_DEQUANT) Y = static_cast<void*>(static_cast<float*>(Y) + (int64_t)blockIdx.y * M * N);
  // the slice's first K block is the descriptors' origin; rows past the tile
  // fall outside their range and read zero
  const v4i ra = make_rsrc(A + (int64_t)m0 * K + kbs * 128, (uint32_t)(mrows * K - kbs * 128));
  const v4i rw = make_rsrc(Wx + (int64_t)n0 * K + kbs * 128, (uint32_t)(nval * K - kbs * 128));
  const int voffA = wave * AI * 8 * K + dma_lane_off(lane, K);
  const int voffW = wave * WI * 8 * K + dma_lane_off(lane, K);
  const uint32_t lds0 = lds_addr(smem);
  const int K8 = 8 * K;
  int lo[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) lo[ks] = frag_off(lane & 31, 2 * ks + (lane >> 5));   // 32x32x32 operand

  // this wave's 128 columns lie in one 128-wide N block: one weight scale per
  // K block; rows past the tile read the last row's scales (never stored)
  int nbw = (n0 + wn * 128) >> 7;
  nbw = nbw < NB ? nbw : NB - 1;
  const float* sw_row = swx + (int64_t)nbw * KB + kbs;
  const float* sa_t = sa + (int64_t)m0 * KB + kbs;   // uniform base, 32-bit lane offsets
  int sao[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wm * 64 + j * 32 + (lane & 31);
    sao[j] = (r < mrows ? r : mrows - 1) * KB;
  }

  v4f facc[4][2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) facc[i][j][g] = (v4f){0.f, 0.f, 0.f, 0.f};

  const bool vec = (N & 3) == 0;
  // chain (i, j) of K block kbp (slice-relative), partial p: dequantise it
  // with scale s, or store it raw
  auto drain = [&](const v16i& p, auto ic, auto jc, float s, int kbp) {
    constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
    if (DQ) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) facc[i][j][g][r] = __builtin_fmaf(s, (float)p[4 * g + r], facc[i][j][g][r]);
    } else {
      const int ml = wm * 64 + j * 32 + (lane & 31);
      if (ml < mrows) {
        const int m = m0 + ml;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * 128 + i * 32 + g * 8 + 4 * (lane >> 5);
          if (n < N)
            store4i(static_cast<int32_t*>(Y) + ((int64_t)(kbs + kbp) * M + m) * N + n, n, N, vec,
                    (v4i){p[4 * g], p[4 * g + 1], p[4 * g + 2], p[4 * g + 3]});
        }
      }
    }
  };

  // 8-row groups of A past the tile's rows are not loaded (their LDS rows
  // feed only outputs that are never stored), and a wave whose 64 rows all
  // lie past them skips its MFMAs (MoE expert tiles are often part-empty)
  const bool wact = wm * 64 < mrows;
#define BK_DMA(T)                                                                                  \
  {                                                                                               \
    const uint32_t base = lds0 + ((T) & 1) * STG;                                                 \
    _Pragma("unroll") for (int b = 0; b < AI; ++b)                                                \
      if ((wave * AI + b) * 8 < mrows) dma16(ra, voffA, b * K8 + (T) * 128, base + (wave * AI + b) * 1024); \
    _Pragma("unroll") for (int b = 0; b < WI; ++b)                                                \
      dma16(rw, voffW, b * K8 + (T) * 128, base + BM * 128 + (wave * WI + b) * 1024);             \
  }

  const int NK = kbe - kbs;   // K blocks of this slice, numbered from its first
  // scales of the next block to compute (loaded one block ahead), and the
  // pending chain: chain 7 (i = 3, j = 1) of the previous block
  float la0 = 0.f, la1 = 0.f, lw = 0.f;
  if (DQ && NK > 0) {
    la0 = sa_t[sao[0]];
    la1 = sa_t[sao[1]];
    lw = sw_row[0];
  }
  float sp = 0.f;
  v16i pp = {};
  if (NK > 0) BK_DMA(0)
  for (int kb = 0; kb < NK; ++kb) {
    waitcnt<0, 0>();   // block kb and its scales landed; own reads of kb-1 done
    barrier();         // everyone's block kb landed; everyone is past kb-1
    if (kb + 1 < NK) BK_DMA(kb + 1)
    const float sc0 = __fmul_rn(la0, lw), sc1 = __fmul_rn(la1, lw);
    if (DQ) {
      const int kn = kb + 1 < NK ? kb + 1 : kb;
      la0 = sa_t[sao[0] + kn];
      la1 = sa_t[sao[1] + kn];
      lw = sw_row[kn];
    }
    if (!wact) continue;
    const char* buf = smem + (kb & 1) * STG;
    v4i af[2][4], wc[4], wnx[4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) af[j][ks] = *(const v4i*)(buf + (wm * 64 + j * 32) * 128 + lo[ks]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) wc[ks] = *(const v4i*)(buf + BM * 128 + (wn * 128) * 128 + lo[ks]);
    // chain t = 2 i + j
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = t >> 1, j = t & 1;
      if (j == 0 && i < 3) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          wnx[ks] = *(const v4i*)(buf + BM * 128 + (wn * 128 + (i + 1) * 32) * 128 + lo[ks]);
      }
      v16i c = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) c = __builtin_amdgcn_mfma_i32_32x32x32_i8(wc[ks], af[j][ks], c, 0, 0, 0);
      if (t == 0) {
        if (kb > 0) drain(pp, std::integral_constant<int, 3>{}, std::integral_constant<int, 1>{}, sp, kb - 1);
      } else if (t & 1) {   // previous chain: (i, 0)
        if (i == 0) drain(pp, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, sc0, kb);
        if (i == 1) drain(pp, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{}, sc0, kb);
        if (i == 2) drain(pp, std::integral_constant<int, 2>{}, std::integral_constant<int, 0>{}, sc0, kb);
        if (i == 3) drain(pp, std::integral_constant<int, 3>{}, std::integral_constant<int, 0>{}, sc0, kb);
      } else {              // previous chain: (i - 1, 1)
        if (i == 1) drain(pp, std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{}, sc1, kb);
        if (i == 2) drain(pp, std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{}, sc1, kb);
        if (i == 3) drain(pp, std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{}, sc1, kb);
      }
      // one MFMA, then eight VALU ops, four times; the next pair's W reads
      // ride along
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        if (j == 0 && i < 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      pp = c;
      if (j == 1 && i < 3) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) wc[ks] = wnx[ks];
      }
    }
    sp = sc1;
  }
#undef BK_DMA
  if (NK > 0 && wact) drain(pp, std::integral_constant<int, 3>{}, std::integral_constant<int, 1>{}, sp, NK - 1);
  waitcnt<0, 0>();
  if (!DQ) return;

  if (OUT == OUT_BF16) {
    // the bf16 tile goes through LDS (row r of 256 bf16, 16-byte chunk c at
    // c ^ (r & 15)) so that it leaves in whole rows; the barrier also means
    // every wave is past its last stage read
    barrier();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = wm * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint32_t h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) h[q] = f32_to_bf16_rne(facc[i][j][g][q]);
          const int chunk = wn * 16 + i * 4 + g;
          *reinterpret_cast<uint2*>(smem + r * 512 + ((chunk ^ (r & 15)) << 4) + 8 * (lane >> 5)) =
              make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        }
    }
    waitcnt<63, 0>();
    barrier();
    // wave w stores tile rows 32 w .. 32 w + 31, two rows per instruction
    const int cl = lane & 31;
    const int n = n0 + 8 * cl;
    const bool vec8 = (N & 7) == 0 && n + 7 < N;
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int r = wave * 32 + 2 * it + (lane >> 5);
      const v4i v = *reinterpret_cast<const v4i*>(smem + r * 512 + ((cl ^ (r & 15)) << 4));
      if (r >= mrows || n >= N) continue;
      uint16_t* y = static_cast<uint16_t*>(Y) + (int64_t)(m0 + r) * N + n;
      if (vec8) {
        *reinterpret_cast<v4i*>(y) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < N) y[e] = (uint16_t)(((uint32_t)v[e >> 1]) >> (16 * (e & 1)));
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ml = wm * 64 + j * 32 + (lane & 31);
    if (ml >= mrows) continue;
    const int m = m0 + ml;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * 128 + i * 32 + g * 8 + 4 * (lane >> 5);
        if (n >= N) continue;
        store4<OUT>(Y, (int64_t)m * N + n, n, N, vec, facc[i][j][g][0], facc[i][j][g][1], facc[i][j][g][2],
                    facc[i][j][g][3]);
      }
  }
}

template <int MODE, int OUT, int NWM>
void launch_block_kernel(dim3 grid, hipStream_t st, const int8_t* A, const float* sa, const int8_t* W,
                         const float* sw, const int32_t* off, void* Y, int M, int N, int K, int TM, int TN, int E) {
  hipLaunchKernelGGL((k_gemm_block<MODE, OUT, NWM>), grid, dim3(128 * NWM), 0, st, A, sa, W, sw, off, Y, M, N, K, TM,
                     TN, E);
}

// Sum of the S fp32 slices' partial tiles, in slice order, then the output.
// Each thread covers 4 consecutive outputs of one row.
template <int OUT>
__global__ __launch_bounds__(256) void k_splitk_sum_f32(const float* __restrict__ ws, int S, int M, int N,
                                                        void* __restrict__ Y) {
  const int64_t q4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nq = (N + 3) >> 2;
  if (q4 >= (int64_t)M * nq) return;
  const int m = (int)(q4 / nq), n = (int)(q4 - (int64_t)m * nq) * 4;
  const int64_t idx = (int64_t)m * N + n;
  const int64_t MN = (int64_t)M * N;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sl = 0; sl < S; ++sl)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) o[r] = __fadd_rn(o[r], ws[sl * MN + idx + r]);
  store4<OUT>(Y, idx, n, N, (N & 3) == 0, o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_gemm_block(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                             OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (decode_path_takes(M, N, false)) return launch_gemm_block_decode(A, sa, W, sw, Y, out, M, N, K, st);
  const int TN = (int)((N + 255) / 256);
  // 128-row tiles for few rows, and where 256-row tiles would leave CUs idle
  // (twice the tiles before any K split, one wave per SIMD: DeepSeek's q_a
  // and kv_a projections at 4096 tokens run 11-14 % faster than on split
  // 256-row tiles)
  const int BM = (M <= 128 || ((M + 255) / 256) * TN < kTileCUs) ? 128 : 256;
  const int TM = (int)((M + BM - 1) / BM);
  // ~2.6 us per 256 x 256 tile and K block (1.7 for 128 x 256) at the
  // measured large-M rate
  const int S = pick_k_slices((int64_t)TM * TN, K >> 7, M, N, BM == 256 ? 2.6 : 1.7);
  void* dst = Y;
  if (S > 1) {
    hipError_t e = split_workspace(st, (size_t)S * M * N * 4, &dst);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((unsigned)(TM * TN), (unsigned)S);
  const bool f32 = S > 1 || out == OUT_F32;
  if (BM == 128) {
    if (f32)
      launch_block_kernel<MODE_DEQUANT, OUT_F32, 2>(grid, st, A, sa, W, sw, nullptr, dst, (int)M, (int)N, (int)K, TM,
                                                    TN, 0);
    else
      launch_block_kernel<MODE_DEQUANT, OUT_BF16, 2>(grid, st, A, sa, W, sw, nullptr, dst, (int)M, (int)N, (int)K, TM,
                                                     TN, 0);
  } else {
    if (f32)
      launch_block_kernel<MODE_DEQUANT, OUT_F32, 4>(grid, st, A, sa, W, sw, nullptr, dst, (int)M, (int)N, (int)K, TM,
                                                    TN, 0);
    else
      launch_block_kernel<MODE_DEQUANT, OUT_BF16, 4>(grid, st, A, sa, W, sw, nullptr, dst, (int)M, (int)N, (int)K, TM,
                                                     TN, 0);
  }
  if (S > 1) {
    const dim3 rg((unsigned)((M * ((N + 3) / 4) + 255) / 256));
    const float* wsf = static_cast<const float*>(dst);
    if (out == OUT_BF16)
      hipLaunchKernelGGL((k_splitk_sum_f32<OUT_BF16>), rg, dim3(256), 0, st, wsf, S, (int)M, (int)N, Y);
    else
      hipLaunchKernelGGL((k_splitk_sum_f32<OUT_F32>), rg, dim3(256), 0, st, wsf, S, (int)M, (int)N, Y);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_block_partials(const int8_t* A, const int8_t* W, int32_t* P, int64_t M, int64_t N, int64_t K,
                                      hipStream_t st) {
  const int TM = (int)((M + 255) / 256), TN = (int)((N + 255) / 256);
  launch_block_kernel<MODE_PARTIALS, OUT_I32, 4>(dim3((unsigned)(TM * TN)), st, A, nullptr, W, nullptr, nullptr, P,
                                                 (int)M, (int)N, (int)K, TM, TN, 0);
  return hipGetLastError();
}

hipError_t launch_gemm_block_grouped(const int8_t* A, const float* sa, const int8_t* W, const float* sw,
                                     const int32_t* offsets, void* Y, OutKind out, int64_t E, int64_t P, int64_t N,
                                     int64_t K, hipStream_t st) {
  // Every expert tile streams its expert's weight panel once, so even at a
  // few rows per expert this runs at the weight stream's pace; waves whose
  // rows are all past the expert's rows skip their MFMAs.  256-row tiles from
  // 96 rows per expert on average (fewer second tiles re-reading a panel),
  // 128-row tiles below.
  const int TN = (int)((N + 255) / 256);
  const bool big = P >= 96 * E;
  const int BM = big ? 256 : 128;
  // upper bound on the number of m-tiles over all experts
  const int64_t TMmax = (P + BM - 1) / BM + E;
  const dim3 grid((unsigned)(TMmax * TN));
  if (big) {
    if (out == OUT_BF16)
      launch_block_kernel<MODE_GROUPED, OUT_BF16, 4>(grid, st, A, sa, W, sw, offsets, Y, (int)P, (int)N, (int)K,
                                                     (int)TMmax, TN, (int)E);
    else
      launch_block_kernel<MODE_GROUPED, OUT_F32, 4>(grid, st, A, sa, W, sw, offsets, Y, (int)P, (int)N, (int)K,
                                                    (int)TMmax, TN, (int)E);
  } else {
    if (out == OUT_BF16)
      launch_block_kernel<MODE_GROUPED, OUT_BF16, 2>(grid, st, A, sa, W, sw, offsets, Y, (int)P, (int)N, (int)K,
                                                     (int)TMmax, TN, (int)E);
    else
      launch_block_kernel<MODE_GROUPED, OUT_F32, 2>(grid, st, A, sa, W, sw, offsets, Y, (int)P, (int)N, (int)K,
                                                    (int)TMmax, TN, (int)E);
  }
  return hipGetLastError();
}

}  // namespace w8
