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

#include "tile_common.h"

namespace w8 {
namespace {

// ------------------------------------------------------------ channel-wise
// 256 (m) x BN (n) output tile per workgroup, BN = 32 FN (FN = 8, 7 or 6);
// 8 waves, two per SIMD, in a 2 (n) x 4 (m) grid, each wave 16 FN (n) x 64
// (m): FN x 4 fragments of v_mfma_i32_16x16x64_i8, FN x 16 int32
// accumulators per lane.  With two waves per SIMD one issues MFMAs while the
// other waits on LDS or issues loads, and the LDS serves about twice the read
// bandwidth it gives one wave per SIMD.
//
// K runs in 128-deep blocks through two LDS stages (A 256 x 128 B, then W
// BN x 128 B).  A block is two 64-deep K steps, and the loop body is
// unrolled over them so that the fragment registers alternate between two
// sets without copies.  Step A of block kb multiplies (kb, first half) and
// reads (kb, second half); then every wave waits for its loads of block kb+1
// and for its own reads, and all meet at a barrier; step B multiplies (kb,
// second half), reads (kb+1, first half) and loads block kb+2 into the stage
// block kb has just left.  A wave's eight loads of a block (1 KB each: eight
// rows of 128 B) go two at a time before the first four of its FN groups of
// four MFMAs in step B, so no burst of loads stalls a wave's MFMAs.  The last
// block is peeled (a branch inside the loop body breaks the in-place
// accumulator allocation), and loads of blocks past the end are pushed
// outside the descriptors' ranges: they move no data.
//
// A load that finds nothing in range still writes zeros to LDS (measured on
// gfx950), so a wave without an eighth W row block (BN < 256) sends that
// load to a junk kilobyte past the two stages, never onto the other stage.
//
// Tile order: workgroup b runs on XCD b % 8, and XCD x owns a contiguous band
// of the tile sequence; the sequence walks strips of GM row tiles (m fastest
// within a strip), so the 32 CUs of an XCD work on about GM row tiles x 32/GM
// column tiles at a time and share both operands' panels in their L2.
constexpr int kChBM = 256;
constexpr unsigned kChOob = 0x20000000u;   // added to a load's offset: past every range

// AS: the epilogue of the asymmetric per-tensor activations (codes stored as
// q - 128, prm = {s, z}, wsum = per-row weight sums) in place of the
// channel-wise one: Y = fp32(fp32(s * sw[n]) * fp32(fp32(ACC + 128 WS[n]) -
// fp32(z * fp32(WS[n])))).
// SKINNY (int32 output, M <= 128, FN = 4): a 128 (m) x 256 (n) tile on the
// eight waves as 4 (n) x 2 (m), each wave 64 x 64 (4 x 4 fragments), so every
// SIMD keeps two MFMA waves on rows that exist (a 256-row tile would leave
// half its row bands empty, one MFMA wave per SIMD waiting on its LDS reads).
// A stage is 48 KB (A 128 rows, W 256 rows), so three fit: a barrier waits
// for the older of two blocks in flight, six loads per wave per block.
template <int OUT, int FN, bool AS = false, bool SKINNY = false>
__global__ __launch_bounds__(512, 1) void k_gemm_channel(const int8_t* __restrict__ A, const float* __restrict__ sa,
                                                         const int8_t* __restrict__ W, const float* __restrict__ sw,
                                                         void* __restrict__ Y, int M, int N, int K, int TM, int GM,
                                                         const float* __restrict__ prm = nullptr,
                                                         const int32_t* __restrict__ wsum = nullptr) {
  static_assert(!SKINNY || (FN == 4 && OUT == OUT_I32 && !AS), "SKINNY: int32 128 x 256 tiles");
  constexpr int NWN = SKINNY ? 4 : 2;            // waves along n
  constexpr int BM = SKINNY ? 128 : kChBM;       // tile rows
  constexpr int BN = NWN * 16 * FN;
  constexpr int NST = SKINNY ? 3 : 2;            // stages in the ring
  constexpr int LPB = SKINNY ? 6 : 8;            // loads per wave per block
  constexpr int kStage = (BM + BN) * 128;
  constexpr int kJunk = NST * kStage;
  // the stages and the junk kilobyte, or the bf16 epilogue's 256 rows of 512 B
  constexpr int kSmem = kJunk + 1024 > kChBM * 512 || SKINNY ? kJunk + 1024 : kChBM * 512;
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % NWN, wm = wave / NWN;
  int tm, tn;
  strip_tile(blockIdx.x, TM, (int)gridDim.x / TM, GM, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int mval = M - m0 < BM ? M - m0 : BM;
  const int nval = N - n0 < BN ? N - n0 : BN;
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
  const int NK = kbe - kbs;
  const int voff = dma_lane_off(lane, K);
  const uint32_t lds0 = lds_addr(smem);
  const int K8 = 8 * K;
  const int lo0 = frag_off(lane & 15, lane >> 4);            // 16x16x64 operand: row l % 16, chunk l / 16
  const int lo1 = frag_off(lane & 15, 4 + (lane >> 4));
  // load d (0..7) of a block: A row block wave + 8 d (d < 4), W row block
  // wave + 8 (d - 4); the eighth exists when wave + 24 < 4 FN
  const bool w8th = wave + 24 < 4 * FN;
  const int soff0 = wave * K8;
  const uint32_t dlds0 = lds0 + wave * 1024;
  const uint32_t ljunk = lds0 + kJunk;

  v4i acc[FN][4];
#pragma unroll
  for (int i = 0; i < FN; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

#define CH_LOAD(T, D, SO)                                                                          \
  if constexpr (SKINNY) {                                                                         \
    const uint32_t base = dlds0 + ((T) % 3) * kStage;                                             \
    if ((D) < 2)                                                                                  \
      dma16(ra, voff, soff0 + 8 * (D) * K8 + (T) * 128 + (SO), base + 8 * (D) * 1024);            \
    else                                                                                          \
      dma16(rw, voff, soff0 + 8 * ((D) - 2) * K8 + (T) * 128 + (SO), base + BM * 128 + 8 * ((D) - 2) * 1024); \
  } else {                                                                                        \
    const uint32_t base = dlds0 + ((T) & 1) * kStage;                                             \
    if ((D) < 4) {                                                                                \
      dma16(ra, voff, soff0 + 8 * (D) * K8 + (T) * 128 + (SO), base + 8 * (D) * 1024);            \
    } else if ((D) < 7) {                                                                         \
      dma16(rw, voff, soff0 + 8 * ((D) - 4) * K8 + (T) * 128 + (SO), base + kChBM * 128 + 8 * ((D) - 4) * 1024); \
    } else {                                                                                      \
      dma16(rw, voff, soff0 + 24 * K8 + (T) * 128 + (SO) + (w8th ? 0u : kChOob),                  \
            w8th ? base + kChBM * 128 + 24 * 1024 : ljunk);                                       \
    }                                                                                             \
  }
#define CH_READ(BLK, LO, WF, AF, R)                                                                \
  if constexpr (SKINNY) {                                                                         \
    const char* buf = smem + ((BLK) % 3) * kStage;                                                \
    if ((R) < 4) AF[(R)] = *(const v4i*)(buf + (wm * 64 + (R) * 16) * 128 + (LO));                \
    else WF[(R) - 4] = *(const v4i*)(buf + BM * 128 + (wn * 16 * FN + ((R) - 4) * 16) * 128 + (LO)); \
  } else {                                                                                        \
    const char* buf = smem + ((BLK) & 1) * kStage;                                                \
    if ((R) < 4) AF[(R)] = *(const v4i*)(buf + (wm * 64 + (R) * 16) * 128 + (LO));                \
    else WF[(R) - 4] = *(const v4i*)(buf + kChBM * 128 + (wn * 16 * FN + ((R) - 4) * 16) * 128 + (LO)); \
  }
  // one K step: FN groups of four MFMAs (one W fragment against the four
  // activation fragments); before group g, two of the 4 + FN reads of the
  // next fragments (RD) and two of the eight loads of block LT (LD)
#define CH_STEP(WC, AC, RD, RBLK, RLO, WN_, AN_, LD, LT, LSO)                                       \
  _Pragma("unroll") for (int g = 0; g < FN; ++g) {                                                \
    if ((RD) && 2 * g < 4 + FN) {                                                                 \
      CH_READ(RBLK, RLO, WN_, AN_, 2 * g)                                                         \
      if (2 * g + 1 < 4 + FN) CH_READ(RBLK, RLO, WN_, AN_, 2 * g + 1)                             \
    }                                                                                             \
    if ((LD) && 2 * g < LPB) {                                                                    \
      CH_LOAD(LT, 2 * g, LSO)                                                                     \
      CH_LOAD(LT, 2 * g + 1, LSO)                                                                 \
    }                                                                                             \
    _Pragma("unroll") for (int j = 0; j < 4; ++j)                                                 \
      acc[g][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(WC[g], AC[j], acc[g][j], 0, 0, 0);        \
    __builtin_amdgcn_sched_barrier(0);                                                            \
  }

  // prologue: block 0 loaded and visible, block 1 (SKINNY: blocks 1 and 2)
  // in flight
#pragma unroll
  for (int d = 0; d < LPB; ++d) CH_LOAD(0, d, 0u)
  if constexpr (SKINNY) {
    const unsigned so1 = 1 < NK ? 0u : kChOob, so2 = 2 < NK ? 0u : kChOob;
#pragma unroll
    for (int d = 0; d < LPB; ++d) CH_LOAD(1, d, so1)
#pragma unroll
    for (int d = 0; d < LPB; ++d) CH_LOAD(2, d, so2)
    wait_barrier<2 * LPB, 15>();
  } else {
    wait_barrier<0, 15>();
    const unsigned so1 = 1 < NK ? 0u : kChOob;
#pragma unroll
    for (int d = 0; d < 8; ++d) CH_LOAD(1, d, so1)
  }
  v4i w0[FN], a0[4], w1[FN], a1[4];
#pragma unroll
  for (int r = 0; r < 4 + FN; ++r) CH_READ(0, lo0, w0, a0, r)
  // the block loaded in step B: the one two (SKINNY: three) ahead, into the
  // stage block kb has just left
  constexpr int kAhead = SKINNY ? 3 : 2;
  for (int kb = 0; kb + 1 < NK; ++kb) {
    CH_STEP(w0, a0, true, kb, lo1, w1, a1, false, 0, 0u)
    // block kb + 1 has landed everywhere (SKINNY: block kb + 2 may still be
    // in flight); every wave is past its reads of kb
    wait_barrier<SKINNY ? LPB : 0, 0>();
    const unsigned so = kb + kAhead < NK ? 0u : kChOob;
    CH_STEP(w1, a1, true, kb + 1, lo0, w0, a0, true, kb + kAhead, so)
  }
  CH_STEP(w0, a0, true, NK - 1, lo1, w1, a1, false, 0, 0u)
  // the epilogue's scales: for the bf16 channel-wise output they load under
  // the last K step (the first fragment set is free by then, and all of the
  // tile's stage loads were issued earlier, so the compiler's wait for these
  // loads covers them too); the other epilogues hold more values per lane
  // and load them after it
  const bool vec = (N & 3) == 0;
  constexpr bool kEarly = OUT == OUT_BF16 && !AS;
  float sam[4], swn[FN][4], zw[FN][4];
  int wsx[FN][4];
  auto load_scales = [&]() {
    if (!AS) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + wm * 64 + j * 16 + (lane & 15);
        sam[j] = m < M ? sa[m] : 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < FN; ++i) {
      const int n = n0 + wn * 16 * FN + i * 16 + 4 * (lane >> 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        swn[i][r] = n + r < N ? sw[n + r] : 0.f;
        if (AS) wsx[i][r] = n + r < N ? wsum[n + r] : 0;
      }
    }
  };
  if (kEarly) load_scales();
  CH_STEP(w1, a1, false, 0, 0, w0, a0, false, 0, 0u)
#undef CH_LOAD
#undef CH_READ
#undef CH_STEP
  // every stage load (the past-the-end ones included) has landed
  waitcnt<0, 0>();
  if (!kEarly && OUT != OUT_I32) load_scales();

  if (OUT == OUT_I32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 64 + j * 16 + (lane & 15);
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = n0 + wn * 16 * FN + i * 16 + 4 * (lane >> 4);
        if (n < N) store4i(static_cast<int32_t*>(Y) + (int64_t)m * N + n, n, N, vec, acc[i][j]);
      }
    }
    return;
  }
  if (AS) {
    const float as_s = prm[0], as_z = prm[1];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        swn[i][r] = __fmul_rn(as_s, swn[i][r]);
        zw[i][r] = __fmul_rn(as_z, (float)wsx[i][r]);
        wsx[i][r] = 128 * wsx[i][r];
      }
  }
  // output value of accumulator r of fragment (i, j)
  auto outv = [&](int i, int j, int r) -> float {
    if (AS) return __fmul_rn(swn[i][r], __fsub_rn((float)(acc[i][j][r] + wsx[i][r]), zw[i][r]));
    return __fmul_rn((float)acc[i][j][r], __fmul_rn(sam[j], swn[i][r]));
  };
  if (OUT == OUT_F32) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wm * 64 + j * 16 + (lane & 15);
      if (m >= M) continue;
#pragma unroll
      for (int i = 0; i < FN; ++i) {
        const int n = n0 + wn * 16 * FN + i * 16 + 4 * (lane >> 4);
        if (n >= N) continue;
        store4<OUT_F32>(Y, (int64_t)m * N + n, n, N, vec, outv(i, j, 0), outv(i, j, 1), outv(i, j, 2),
                        outv(i, j, 3));
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
  for (int j = 0; j < 4; ++j) {
    const int r = wm * 64 + j * 16 + (lane & 15);
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
  // wave w stores tile rows 32 w .. 32 w + 31, two rows per instruction;
  // lane: row half lane >> 5, columns 8 (lane & 31) .. + 7 (chunks past the
  // tile's BN columns are skipped).  The output is written once and not read
  // back by this kernel: non-temporal stores.
  const int cl = lane & 31;
  const int n = n0 + 8 * cl;
  const bool vec8 = (N & 7) == 0 && n + 7 < N;
  const bool inside = cl < 4 * FN;
#pragma unroll 4
  for (int it = 0; it < 16; ++it) {
    const int r = wave * 32 + 2 * it + (lane >> 5);
    const int m = m0 + r;
    const v4i v = *reinterpret_cast<const v4i*>(smem + r * 512 + ((cl ^ (r & 15)) << 4));
    if (m >= M || n >= N || !inside) continue;
    uint16_t* y = static_cast<uint16_t*>(Y) + (int64_t)m * N + n;
    if (vec8) {
      __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(y));
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
  const bool vec = (N & 3) == 0;
  v4i a = {0, 0, 0, 0};
  if (vec) {
    // 16-byte loads, four slices in flight
#pragma unroll 4
    for (int sl = 0; sl < S; ++sl) a += *reinterpret_cast<const v4i*>(ws + sl * MN + idx);
  } else {
    for (int sl = 0; sl < S; ++sl)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) a[r] += ws[sl * MN + idx + r];
  }
  if (OUT == OUT_I32) {
    store4i(static_cast<int32_t*>(Y) + idx, n, N, vec, a);
  } else {
    float o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = n + r < N ? __fmul_rn((float)a[r], __fmul_rn(sa[m], sw[n + r])) : 0.f;
    store4<OUT>(Y, idx, n, N, vec, o[0], o[1], o[2], o[3]);
  }
}



// Height in row tiles of the strips the channel tile kernel walks (the whole
// column of row tiles when there are fewer than 8).
int channel_strip(int TM) { return TM < 8 ? TM : 8; }

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
  const dim3 grid((unsigned)(TM * TN)), block(512);
  const int GM = channel_strip(TM);
  switch (out) {
    case OUT_BF16:
      hipLaunchKernelGGL((k_gemm_channel<OUT_BF16, FN>), grid, block, 0, st, A, sa, W, sw, Y, (int)M, (int)N, (int)K,
                         TM, GM);
      break;
    case OUT_F32:
      hipLaunchKernelGGL((k_gemm_channel<OUT_F32, FN>), grid, block, 0, st, A, sa, W, sw, Y, (int)M, (int)N, (int)K,
                         TM, GM);
      break;
    default:
      hipLaunchKernelGGL((k_gemm_channel<OUT_I32, FN>), grid, block, 0, st, A, sa, W, sw, Y, (int)M, (int)N, (int)K,
                         TM, GM);
      break;
  }
  return hipGetLastError();
}

template <int FN>
hipError_t channel_asym_launch(const int8_t* A, const float* prm, const int8_t* W, const float* sw,
                               const int32_t* wsum, void* Y, OutKind out, int64_t M, int64_t N, int64_t K, int TM,
                               hipStream_t st) {
  const int TN = (int)((N + 32 * FN - 1) / (32 * FN));
  const dim3 grid((unsigned)(TM * TN)), block(512);
  const int GM = channel_strip(TM);
  if (out == OUT_F32)
    hipLaunchKernelGGL((k_gemm_channel<OUT_F32, FN, true>), grid, block, 0, st, A, nullptr, W, sw, Y, (int)M,
                       (int)N, (int)K, TM, GM, prm, wsum);
  else
    hipLaunchKernelGGL((k_gemm_channel<OUT_BF16, FN, true>), grid, block, 0, st, A, nullptr, W, sw, Y, (int)M,
                       (int)N, (int)K, TM, GM, prm, wsum);
  return hipGetLastError();
}

}  // namespace

// The library's scratch buffers (workspace.h): device memory from hipMalloc,
// never freed while the process runs (the cache itself is never destroyed,
// so no HIP call runs during process teardown).
bool HipScratch::alloc(void** p, size_t bytes) { return hipMalloc(p, bytes) == hipSuccess; }
void HipScratch::release(void*) {}

namespace {
WorkspaceCache<HipScratch>& scratch_cache() {
  static WorkspaceCache<HipScratch>* c = new WorkspaceCache<HipScratch>();
  return *c;
}

bool stream_capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs == hipStreamCaptureStatusActive;
}
}  // namespace

// Number of K slices for a tile grid that leaves CUs idle: the smallest
// modelled time over S = 1..16, where a slice of KB / S blocks costs one
// round of workgroups per 256, t_kb microseconds per tile and K block, and
// splitting adds the slices' partial tiles through HBM (written and read,
// 8 bytes per output per slice at ~5 TB/s) plus a reduction launch.
int pick_k_slices(int64_t tiles, int64_t KB, int64_t M, int64_t N, double t_kb_us, double* t_us) {
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
  if (t_us) *t_us = best_t;
  return best;
}

WsLease stream_workspace(hipStream_t st, int slot, size_t bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) (void)hipGetLastError();
  return scratch_cache().acquire(dev, reinterpret_cast<const void*>(st), slot, bytes, stream_capturing(st));
}

hipError_t ws_error(const WsLease& lease) {
  switch (lease.status()) {
    case kWsOk: return hipSuccess;
    case kWsCapturing: return hipErrorStreamCaptureUnsupported;
    default: return hipErrorOutOfMemory;
  }
}

namespace {
int channel_slices(int64_t M, int64_t N, int64_t K);
}  // namespace

bool channel_tiles_unsplit(int64_t M, int64_t N, int64_t K) {
  if (decode_path_takes(M, N, true)) return false;
  return channel_slices(M, N, K) == 1;
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

namespace {

// K slices of the channel tile grid for (M, N, K); 1 runs it unsplit.
// ~1.6 us per 256 x 256 tile and K block at the measured large-M rate.
int channel_slices(int64_t M, int64_t N, int64_t K) {
  const int TM = (int)((M + kChBM - 1) / kChBM), TN = (int)((N + 255) / 256);
  return pick_k_slices((int64_t)TM * TN, K >> 7, M, N, 1.6);
}

// The split-K path: S slices of 256 x 256 tiles write int32 partial tiles to
// ws (S x M x N x 4 bytes), then one pass sums them in slice order and
// applies the epilogue.
hipError_t channel_split(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y, OutKind out,
                         int64_t M, int64_t N, int64_t K, int S, void* ws, hipStream_t st) {
  const int TM = (int)((M + kChBM - 1) / kChBM), TN = (int)((N + 255) / 256);
  const dim3 grid((unsigned)(TM * TN), (unsigned)S);
  if (M <= 128)
    hipLaunchKernelGGL((k_gemm_channel<OUT_I32, 4, false, true>), grid, dim3(512), 0, st, A, sa, W, sw, ws, (int)M,
                       (int)N, (int)K, TM, channel_strip(TM));
  else
    hipLaunchKernelGGL((k_gemm_channel<OUT_I32, 8>), grid, dim3(512), 0, st, A, sa, W, sw, ws, (int)M, (int)N, (int)K,
                       TM, channel_strip(TM));
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

hipError_t channel_tiles(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y, OutKind out,
                         int64_t M, int64_t N, int64_t K, hipStream_t st) {
  const int TM = (int)((M + kChBM - 1) / kChBM);
  switch (pick_channel_width(TM, N)) {
    case 7: return channel_launch<7>(A, sa, W, sw, Y, out, M, N, K, TM, st);
    case 6: return channel_launch<6>(A, sa, W, sw, Y, out, M, N, K, TM, st);
    default: return channel_launch<8>(A, sa, W, sw, Y, out, M, N, K, TM, st);
  }
}

}  // namespace

hipError_t launch_gemm_channel(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                               OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (decode_path_takes(M, N, true)) return launch_gemm_channel_decode(A, sa, W, sw, Y, out, M, N, K, st);
  const int S = channel_slices(M, N, K);
  if (S == 1) return channel_tiles(A, sa, W, sw, Y, out, M, N, K, st);
  // the stream's scratch, held until both kernels are enqueued
  const WsLease lease = stream_workspace(st, 0, (size_t)S * M * N * 4);
  if (lease.status() != kWsOk) return ws_error(lease);
  return channel_split(A, sa, W, sw, Y, out, M, N, K, S, lease.ptr(), st);
}

// ------------------------------------------------- allocation-free variant
// The scratch of gemm_w8a8_channel_noalloc: a file-scope device array, one
// copy per GPU the library runs on, kept until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: the array's
// device address on the current GPU comes from hipGetSymbolAddress, once per
// device, and only that address is passed to kernels.
constexpr size_t kFixedScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kFixedScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_fixed_mu;
void* g_fixed_ptr[kMaxDevices] = {};

// The array's address on the current device (looked up on the device's
// first call, with that device current).
hipError_t fixed_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_fixed_mu);
  if (!g_fixed_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_fixed_ptr[dev] = p;
  }
  *out = g_fixed_ptr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_gemm_channel_noalloc(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                                       OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st, bool* too_big) {
  *too_big = false;
  if (decode_path_takes(M, N, true)) return launch_gemm_channel_decode(A, sa, W, sw, Y, out, M, N, K, st);
  const int S = channel_slices(M, N, K);
  if (S == 1) return channel_tiles(A, sa, W, sw, Y, out, M, N, K, st);
  if ((size_t)S * M * N * 4 > kFixedScratchBytes) {
    *too_big = true;
    return hipErrorInvalidValue;
  }
  void* ws = nullptr;
  const hipError_t e = fixed_scratch(&ws);
  if (e != hipSuccess) return e;
  return channel_split(A, sa, W, sw, Y, out, M, N, K, S, ws, st);
}

}  // namespace w8
