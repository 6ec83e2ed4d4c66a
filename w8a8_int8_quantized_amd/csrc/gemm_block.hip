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
// v_mfma_i32_32x32x32_i8 (128-row tiles also come as 256 x 128 on eight
// waves of 64 x 64, and as 192 x 128 on eight waves of 96 x 64, four on the
// even and four on the odd K blocks); a chain is four MFMAs over one K block
// (its exact int32 P), then 16 cvt + 16 fma per lane dequantise it into the
// wave's fp32 accumulators, which stay in VGPRs.  Operands stream global ->
// LDS through direct-to-LDS loads into a two-slot ring (pipeline.h; four
// slots with K parity), one K block per slot; the activation scales are
// staged in LDS 16 K blocks at a time, or with K parity loaded four K blocks
// per lane.
//
// Software pipeline: the MFMAs of chain t run interleaved with the
// dequantisation of chain t - 1 (one MFMA, then eight VALU ops, pinned with
// sched_group_barrier), and the W fragments of the next chain pair are read
// from LDS two chains ahead; the last chain of a K block is dequantised while
// the next block's first MFMAs run.  Without K parity the block's barrier
// sits before its last chain row, so the next block's first fragments are
// read, and the block after it loaded, while that row's MFMAs run.  The MFMA results must land in VGPRs for
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
// NWN: waves along n.  2: each wave 128 (n) x 64 (m), 4 x 2 chains; 4 (with
// NWM = 2): a 128 x 256 tile on eight waves, each 64 (n) x 64 (m), 2 x 2
// chains, so that 128-row tiles keep two MFMA waves per SIMD (bf16 / fp32
// output: a wave's 64 columns are half a quantisation group).
// BN: tile width, 256 or 192 (with NWM = NWN = 2: a 128 x 192 tile of four
// sub-tiles of 96 (n) x 64 (m), 3 x 2 chains; a wave's columns may straddle
// two 128-column weight-scale blocks, so each 32-column chain takes its own
// weight scale).
// KP (with BN = 192): the four waves' sub-tiles are computed twice over, by
// waves 0..3 on the even K blocks of the slice and by waves 4..7 on the odd
// ones, each into its own fp32 accumulators, summed (even + odd) at the end;
// two MFMA waves per SIMD, and four 40 KB stages (two blocks in use, two in
// flight) fill the 160 KB of LDS.
template <int MODE, int OUT, int NWM, int NWN = 2, int BN = 256, bool KP = false>
__global__ __launch_bounds__(64 * NWM * NWN * (KP ? 2 : 1), 1) void k_gemm_block(
    const int8_t* __restrict__ A, const float* __restrict__ sa, const int8_t* __restrict__ W,
    const float* __restrict__ sw, const int32_t* __restrict__ offsets, void* __restrict__ Y, int M, int N, int K,
    int TM, int TN, int E, float* __restrict__ qs = nullptr, int clo = 0, int chi = 0x7fffffff) {
  static_assert(NWN == 2 || (NWN == 4 && OUT != OUT_Q8), "a Q8 group is one wave's 128 columns");
  static_assert(BN == 256 || (BN == 192 && NWM == 2 && NWN == 2 && MODE == MODE_DEQUANT && OUT != OUT_Q8),
                "192-wide tiles: dense, 128 rows, four waves, bf16 / fp32 output");
  static_assert(!KP || BN == 192, "K-block parity: 192-wide tiles (four 40 KB stages)");
  constexpr int BM = 64 * NWM, NWV = NWN * NWM * (KP ? 2 : 1);   // NWV: waves of the workgroup
  constexpr int KS = KP ? 2 : 1;      // K-block stride of a wave
  constexpr int NSTG = 2 * KS;        // LDS stages
  constexpr int CI = BN / (32 * NWN);   // 32-column chains per wave along n
  constexpr int WC = 32 * CI;           // columns per wave
  // weight scales per wave and K block: one where the wave's columns lie in
  // one 128-wide N block, else one per chain
  constexpr int NSW = (128 % WC) == 0 ? 1 : CI;
  constexpr int STG = (BM + BN) * 128;
  constexpr int AI = BM / (8 * NWV);   // DMA instructions per wave per K block for A
  constexpr int WI = BN / (8 * NWV);   // ... and for W
  constexpr bool DQ = MODE != MODE_PARTIALS;
  // activation scales staged in LDS (not with KP, whose stages fill it):
  // 16 K blocks of every tile row (64 bytes a row) per chunk, two chunks
  constexpr bool SCL = DQ && !KP;
  constexpr int SCB = SCL ? BM * 64 : 0;   // bytes of one scale chunk
  constexpr int SCI = SCL ? BM / (16 * NWV) : 0;   // DMA instructions per wave per chunk
  static_assert(!SCL || SCI * 16 * NWV == BM, "scale chunk rows split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) char smem[NSTG * STG + 2 * SCB];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wsub = KP ? (wave & 3) : wave;   // the wave's sub-tile
  const int par = KP ? (wave >> 2) : 0;      // its first K block (KP: its parity)
  const int wn = wsub % NWN, wm = wsub / NWN;
  const int KB = K >> 7;
  const int NB = (N + 127) >> 7;

  int m0, mrows, n0;
  const int8_t* Wx = W;
  const float* swx = sw;
  if (MODE == MODE_GROUPED) {
    // workgroup b runs on XCD b % 8; the TN column tiles of one expert row
    // tile go to one XCD one after another (row tile 8 (j / TN) + b % 8,
    // column tile j % TN, j = b / 8), so the tile's activation rows are
    // fetched into one L2 rather than into all eight, and the XCDs take
    // alternate row tiles (the empty ones past the last included)
    const int j = blockIdx.x >> 3;
    const int jt = j / TN;
    const int tmg = 8 * jt + (blockIdx.x & 7);
    n0 = (j - jt * TN) * BN;
    // the tile lookup's three ints live in stage 1, which the first loads
    // into it follow a barrier that every thread reaches after reading them
    const ExpertTile g = group_tile<BM>(offsets, E, M, tmg, reinterpret_cast<int*>(smem + STG), clo, chi);
    if (g.e < 0) return;
    m0 = g.r0;
    mrows = g.r1 - g.r0;
    Wx = W + (int64_t)g.e * N * K;
    swx = sw + (int64_t)g.e * NB * KB;
  } else {
    // strips of up to 8 row tiles per XCD band: an XCD's concurrent tiles
    // share both operands' panels in its L2 (tile_common.h)
    int tm, tn;
    strip_tile(blockIdx.x, TM, TN, TM < 8 ? TM : 8, tm, tn);
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

  // the weight-scale row of each 128-wide N block the wave's chains lie in;
  // rows past the tile read the last row's scales (never stored)
  const float* sw_row[NSW];
#pragma unroll
  for (int q = 0; q < NSW; ++q) {
    int nbw = (n0 + wn * WC + 32 * q) >> 7;
    nbw = nbw < NB ? nbw : NB - 1;
    sw_row[q] = swx + (int64_t)nbw * KB + kbs;
  }
  int sao[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = wm * 64 + j * 32 + (lane & 31);
    // staged (SCL): the row's offset in a chunk (16-row groups of 1 KB, each
    // four 256-byte pieces of 16 rows x 16 bytes); KP: the byte offset of its
    // slice's first scale
    sao[j] = SCL ? (r >> 4) * 1024 + (r & 15) * 16 : (r * KB + kbs) * 4;
  }
  // Scale chunk c (slice blocks 16 c .. 16 c + 15) goes to buffer c % 2 by
  // direct-to-LDS loads of 16 bytes (four K blocks of one row) per lane, 16
  // rows per instruction, lane l taking row l % 16 and blocks 4 (l / 16) ..
  // 4 (l / 16) + 3, so that one block's scales of 16 consecutive rows lie
  // 16 bytes apart (reads of 32 rows: two-way bank conflicts, not
  // eight-way); rows past the tile, and bytes past the last row, read zero
  // through the descriptor (the values past a row's last K block are never
  // used).  A per-lane load of one scale per K block would touch a cache
  // line per row.
  const v4i rsa = make_rsrc(SCL ? sa + (int64_t)m0 * KB : sa, SCL ? (uint32_t)(mrows * KB * 4) : 0u);
  const uint32_t scl0 = lds_addr(smem) + NSTG * STG;
#define BK_SCL(C)                                                                                   \
  _Pragma("unroll") for (int s_ = 0; s_ < SCI; ++s_) {                                             \
    const int i_ = wave * SCI + s_;                                                                \
    dma16(rsa, (16 * i_ + (lane & 15)) * KB * 4 + (lane >> 4) * 16, (kbs + 16 * (C)) * 4,          \
          scl0 + ((C) & 1) * SCB + i_ * 1024);                                                     \
  }
  // KP: a lane's row's scales of four consecutive K blocks, loaded at once
  // through a descriptor over the tile's rows (rows past them, and bytes past
  // the last row, read zero), kept for the wave's next two blocks
  const __amdgpu_buffer_rsrc_t rsa4 = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(KP ? sa + (int64_t)m0 * KB : sa), 0, __builtin_amdgcn_readfirstlane(KP ? mrows * KB * 4 : 0),
      0x00020000);
  v4f la4[2] = {};
  int cb = -8;   // la4 holds slice blocks cb .. cb + 3
  // the activation scale of row offset o (sao) and slice block k, staged
  auto la_lds = [&](int o, int k) {
    return *reinterpret_cast<const float*>(smem + NSTG * STG + ((k >> 4) & 1) * SCB + o + ((k >> 2) & 3) * 256 +
                                           (k & 3) * 4);
  };

  v4f facc[CI][2][4];
#pragma unroll
  for (int i = 0; i < CI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) facc[i][j][g] = (v4f){0.f, 0.f, 0.f, 0.f};

  const bool vec = (N & 3) == 0;
  // chain (i, j) of K block kbp (slice-relative), partial p: dequantise it
  // with scale s, or store it raw
  auto drain = [&](const v16i& p, auto ic, auto jc, float s, int kbp) {
    constexpr int i = decltype(ic)::value, j = decltype(jc)::value;
    if constexpr (i >= CI) {
      return;
    } else if (DQ) {
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
          const int n = n0 + wn * WC + i * 32 + g * 8 + 4 * (lane >> 5);
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
    const uint32_t base = lds0 + ((T) & (NSTG - 1)) * STG;                                        \
    _Pragma("unroll") for (int b = 0; b < AI; ++b)                                                \
      if ((wave * AI + b) * 8 < mrows) dma16(ra, voffA, b * K8 + (T) * 128, base + (wave * AI + b) * 1024); \
    _Pragma("unroll") for (int b = 0; b < WI; ++b)                                                \
      dma16(rw, voffW, b * K8 + (T) * 128, base + BM * 128 + (wave * WI + b) * 1024);             \
  }

  // weight-scale index of chain i (i past the last chain: never drained)
#define QI(i) (NSW == 1 || (i) >= NSW ? 0 : (i))
  const int NK = kbe - kbs;   // K blocks of this slice, numbered from its first
  // scales of the wave's next block (loaded one of its blocks ahead), and
  // the pending chain: the last chain (CI - 1, 1) of the wave's previous block
  float la0 = 0.f, la1 = 0.f, lw[NSW];
#pragma unroll
  for (int q = 0; q < NSW; ++q) lw[q] = 0.f;
  auto la_kp = [&](int kn) {
    if (kn - cb >= 4 || kn < cb) {
      cb = kn;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        la4[j] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rsa4, sao[j] + kn * 4, 0, 0));
    }
    la0 = la4[0][kn - cb];
    la1 = la4[1][kn - cb];
  };
  if constexpr (SCL) {
    if (NK > 0) {
      // the first chunk, read below after a wait and a barrier of its own
      BK_SCL(0)
      waitcnt<0, 0>();
      barrier();
      la0 = la_lds(sao[0], 0);
      la1 = la_lds(sao[1], 0);
#pragma unroll
      for (int q = 0; q < NSW; ++q) lw[q] = sw_row[q][0];
    }
  } else if (KP && par < NK) {
    la_kp(par);
#pragma unroll
    for (int q = 0; q < NSW; ++q) lw[q] = sw_row[q][par];
  }
  float sp = 0.f;
  v16i pp = {};
  // One K block's chains from LDS buffer buf, JM 32-row fragments per wave
  // (JM = 1: the wave's second fragment lies wholly past the tile's rows, so
  // its MFMAs and dequantisation are skipped).  Chain t = JM i + j;
  // its MFMAs run interleaved with the dequantisation of chain t - 1 (at
  // t = 0, the wave's previous block's last chain).
  auto block_chains = [&](auto jmc, const char* buf, int kb, int it, const float* sc0, const float* sc1) {
    constexpr int JM = decltype(jmc)::value;
    v4i af[JM][4], wc[4], wnx[4];
#pragma unroll
    for (int j = 0; j < JM; ++j)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) af[j][ks] = *(const v4i*)(buf + (wm * 64 + j * 32) * 128 + lo[ks]);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) wc[ks] = *(const v4i*)(buf + BM * 128 + (wn * WC) * 128 + lo[ks]);
#pragma unroll
    for (int t = 0; t < JM * CI; ++t) {
      const int i = t / JM, j = t % JM;
      const bool rd = j == 0 && i < CI - 1;   // the next chain's W fragments are read now
      if (rd) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          wnx[ks] = *(const v4i*)(buf + BM * 128 + (wn * WC + (i + 1) * 32) * 128 + lo[ks]);
      }
      v16i c = {};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) c = __builtin_amdgcn_mfma_i32_32x32x32_i8(wc[ks], af[j][ks], c, 0, 0, 0);
      if (t == 0) {
        if (it > 0)
          drain(pp, std::integral_constant<int, CI - 1>{}, std::integral_constant<int, JM - 1>{}, sp, kb - KS);
      } else {
        // previous chain (ip, jp), tp = t - 1 = JM ip + jp
        const int tp = t - 1;
#define BK_DRAIN(IP, JP)                                                                                     \
  if (JP < JM && tp == IP * JM + JP)                                                                         \
    drain(pp, std::integral_constant<int, IP>{}, std::integral_constant<int, JP>{}, (JP == 0 ? sc0 : sc1)[QI(IP)], kb);
        BK_DRAIN(0, 0) BK_DRAIN(0, 1) BK_DRAIN(1, 0) BK_DRAIN(1, 1)
        BK_DRAIN(2, 0) BK_DRAIN(2, 1) BK_DRAIN(3, 0)
#undef BK_DRAIN
      }
      // one MFMA, then eight VALU ops, four times; the next chain's W reads
      // ride along
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      pp = c;
      if (j == JM - 1 && i < CI - 1) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) wc[ks] = wnx[ks];
      }
    }
    sp = (JM == 2 ? sc1 : sc0)[QI(CI - 1)];
  };
  // The K loop, JM fragments per wave throughout.  Iteration it: the blocks
  // KS it .. KS it + KS - 1 are in LDS, the wave computes block KS it + par.
  auto kloop = [&](auto jmc) {
    constexpr int JM = decltype(jmc)::value;
    const int NIT = (NK + KS - 1) / KS;
#pragma unroll
    for (int T = 0; T < KS; ++T)
      if (T < NK) BK_DMA(T)
    for (int it = 0; it < NIT; ++it) {
      const int kb = KS * it + par;
      waitcnt<0, 0>();   // this iteration's blocks landed; own reads of the last done
      barrier();         // everyone's landed; everyone is past the last iteration
#pragma unroll
      for (int T = 0; T < KS; ++T)
        if (KS * (it + 1) + T < NK) BK_DMA(KS * (it + 1) + T)
      // the next scale chunk, into the buffer the previous one used (every
      // wave is past its reads of it)
      if constexpr (SCL)
        if ((it & 15) == 0 && it + 16 < NK) BK_SCL((it >> 4) + 1)
      // scale of chain (i, j): sc0[i] for j = 0, sc1[i] for j = 1 (index 0
      // when the wave has one weight scale)
      float sc0[NSW], sc1[NSW];
#pragma unroll
      for (int q = 0; q < NSW; ++q) {
        sc0[q] = __fmul_rn(la0, lw[q]);
        sc1[q] = __fmul_rn(la1, lw[q]);
      }
      if (kb >= NK) continue;   // KP: no odd block in the last iteration
      if (DQ) {
        const int kn = kb + KS < NK ? kb + KS : kb;
        if constexpr (SCL) {
          la0 = la_lds(sao[0], kn);
          la1 = la_lds(sao[1], kn);
        } else {
          la_kp(kn);
        }
#pragma unroll
        for (int q = 0; q < NSW; ++q) lw[q] = sw_row[q][kn];
      }
      if (!wact) continue;
      block_chains(jmc, smem + (kb & (NSTG - 1)) * STG, kb, it, sc0, sc1);
    }
    // the wave's last block: the last of its parity
    if (par < NK && wact)
      drain(pp, std::integral_constant<int, CI - 1>{}, std::integral_constant<int, JM - 1>{}, sp,
            NK - 1 - ((NK - 1 - par) % KS));
  };
  // The K loop without K parity, rotated across K blocks: the barrier of
  // block kb sits before its last chain row (chain TB = JM (CI - 1)), where
  // every wave has issued all its fragment reads of the block, so that the
  // next block's first fragments are read from LDS, and block kb + 2 is
  // loaded into the stage block kb leaves, while the last chains of block kb
  // run; right after a barrier each wave has its next MFMA operands in
  // registers instead of all eight waves reading them from LDS at once.
  // Fragment registers: af[j] (A of fragment j), wc (W of the current chain
  // row), wnx (W of the next chain row, then the next block's first row).
  auto kloop_rot = [&](auto jmc) {
    constexpr int JM = decltype(jmc)::value;
    constexpr int TB = JM * (CI - 1);   // the chain the barrier precedes
    auto stg = [&](int kb) { return smem + (kb & 1) * STG; };
    auto rd_a = [&](v4i(&f)[4], const char* buf, int j) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) f[ks] = *(const v4i*)(buf + (wm * 64 + j * 32) * 128 + lo[ks]);
    };
    auto rd_w = [&](v4i(&f)[4], const char* buf, int i) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) f[ks] = *(const v4i*)(buf + BM * 128 + (wn * WC + i * 32) * 128 + lo[ks]);
    };
    // every wave, active or not, meets one barrier per block (the last
    // block's included) and issues its loads of block kb + 2 (and of the
    // next scale chunk)
    // (branch-free: past the last block the loads' offsets lie outside the
    // descriptors' ranges, so they move no data and write zeros into the
    // stage block kb has left, which nothing reads again; rows past the
    // tile read zeros through the descriptor)
    auto sync_point = [&](int kb) {
      waitcnt<0, 0>();   // block kb + 1 landed; own reads of block kb done
      barrier();         // everyone's landed; everyone is past its reads of block kb
      const int T = kb + 2;
      const uint32_t so = T < NK ? 0u : 0x20000000u;
      const uint32_t base = lds0 + (T & 1) * STG;
#pragma unroll
      for (int b = 0; b < AI; ++b) dma16(ra, voffA, b * K8 + T * 128 + so, base + (wave * AI + b) * 1024);
#pragma unroll
      for (int b = 0; b < WI; ++b) dma16(rw, voffW, b * K8 + T * 128 + so, base + BM * 128 + (wave * WI + b) * 1024);
    };
    if (NK > 0) BK_DMA(0)
    waitcnt<0, 0>();
    barrier();
    if (NK > 1) BK_DMA(1)
    v4i af[JM][4], wc[4], wnx[4];
    if (wact && NK > 0) {
      rd_a(af[0], stg(0), 0);
      rd_w(wc, stg(0), 0);
    }
    for (int kb = 0; kb < NK; ++kb) {
      // scale chunk c + 1 (slice blocks 16 (c + 1) ..) goes into the buffer
      // chunk c - 1 used, once every wave is past the barrier of block 16 c
      // (its last reads of chunk c - 1 were at block 16 c - 2); it is first
      // read at block 16 c + 15
      if constexpr (SCL)
        if (kb >= 1 && ((kb - 1) & 15) == 0 && kb + 15 < NK) BK_SCL(((kb - 1) >> 4) + 1)
      float sc0[NSW], sc1[NSW];
#pragma unroll
      for (int q = 0; q < NSW; ++q) {
        sc0[q] = __fmul_rn(la0, lw[q]);
        sc1[q] = __fmul_rn(la1, lw[q]);
      }
      if (DQ) {
        const int kn = kb + 1 < NK ? kb + 1 : kb;
        if constexpr (SCL) {
          la0 = la_lds(sao[0], kn);
          la1 = la_lds(sao[1], kn);
        }
#pragma unroll
        for (int q = 0; q < NSW; ++q) lw[q] = sw_row[q][kn];
      }
      if (!wact) {
        sync_point(kb);
        continue;
      }
      const char* buf = stg(kb);
#pragma unroll
      for (int t = 0; t < JM * CI; ++t) {
        const int i = t / JM, j = t % JM;
        if (t == TB) {
          sync_point(kb);
          __builtin_amdgcn_sched_barrier(0);
        }
        // LDS reads riding along this chain's MFMAs: the second fragment's A
        // (chain 0), the next chain row's W, and from the barrier on the next
        // block's first W row and first A fragment (in the last block these
        // read the other stage's stale bytes, never used)
        int nrd = 0;
        if constexpr (JM == 2) {
          if (t == 0) {
            rd_a(af[1], buf, 1);
            nrd += 4;
          }
        }
        if (j == 0 && i < CI - 1) {
          rd_w(wnx, buf, i + 1);
          nrd += 4;
        } else if (t == TB) {
          rd_w(wnx, stg(kb + 1), 0);
          nrd += 4;
        }
        if (JM == 2 && t == TB + 1) {
          rd_a(af[0], stg(kb + 1), 0);
          nrd += 4;
        }
        v16i c = {};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) c = __builtin_amdgcn_mfma_i32_32x32x32_i8(wc[ks], af[j][ks], c, 0, 0, 0);
        if (t == 0) {
          if (kb > 0) drain(pp, std::integral_constant<int, CI - 1>{}, std::integral_constant<int, JM - 1>{}, sp, kb - 1);
        } else {
          const int tp = t - 1;
#define BK_DRAIN(IP, JP)                                                                                     \
  if (JP < JM && tp == IP * JM + JP)                                                                         \
    drain(pp, std::integral_constant<int, IP>{}, std::integral_constant<int, JP>{}, (JP == 0 ? sc0 : sc1)[QI(IP)], kb);
          BK_DRAIN(0, 0) BK_DRAIN(0, 1) BK_DRAIN(1, 0) BK_DRAIN(1, 1)
          BK_DRAIN(2, 0) BK_DRAIN(2, 1) BK_DRAIN(3, 0)
#undef BK_DRAIN
        }
        // one MFMA, then eight VALU ops, four times; the reads ride along
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
          if (nrd == 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (nrd == 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        pp = c;
        if (j == JM - 1 && i < CI - 1) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) wc[ks] = wnx[ks];
        }
      }
      sp = (JM == 2 ? sc1 : sc0)[QI(CI - 1)];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) wc[ks] = wnx[ks];
      if (JM == 1) rd_a(af[0], stg(kb + 1), 0);
    }
    if (NK > 0 && wact)
      drain(pp, std::integral_constant<int, CI - 1>{}, std::integral_constant<int, JM - 1>{}, sp, NK - 1);
  };
  // Waves whose second fragment has no rows run a K loop of their own
  // (a branch inside the loop would tie both forms to one register
  // assignment); only the grouped 256-row tiles, where MoE experts of
  // 129-160 rows leave such a wave beside a full one on a SIMD, have it.
  if constexpr (KS == 1) {
    if constexpr (MODE == MODE_GROUPED && NWM == 4) {
      if (wm * 64 + 32 >= mrows)   // (with wact) only the first fragment has rows
        kloop_rot(std::integral_constant<int, 1>{});
      else
        kloop_rot(std::integral_constant<int, 2>{});
    } else {
      kloop_rot(std::integral_constant<int, 2>{});
    }
  } else {
    kloop(std::integral_constant<int, 2>{});
  }
#undef BK_DMA
#undef BK_SCL
#undef QI
  waitcnt<0, 0>();
  if (!DQ) return;
  if constexpr (KP) {
    // odd-block sums through LDS (every wave is past its stage reads after
    // the barrier), added to the even-block sums in fixed order: even + odd
    constexpr int NV = CI * 2 * 4;   // v4f accumulators per lane
    v4f* red = reinterpret_cast<v4f*>(smem) + wsub * NV * 64 + lane;
    barrier();
    if (par == 1) {
#pragma unroll
      for (int i = 0; i < CI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) red[((i * 2 + j) * 4 + g) * 64] = facc[i][j][g];
    }
    wait_barrier<63, 0>();
    if (par == 0) {
#pragma unroll
      for (int i = 0; i < CI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const v4f o = red[((i * 2 + j) * 4 + g) * 64];
#pragma unroll
            for (int r = 0; r < 4; ++r) facc[i][j][g][r] = __fadd_rn(facc[i][j][g][r], o[r]);
          }
    }
  }

  if (OUT == OUT_Q8) {
    // The 128 columns of this wave are one quantisation group of the next
    // layer (1 x 128 along its K = this N), and a row's 128 values sit in two
    // lanes (l and l ^ 32, 64 each): round to bf16, take the group's amax
    // over the pair, quantise as quant_act_group does, and store 4 codes per
    // 4-byte write; lanes 0..31 store the row's scale.  The caller
    // guarantees N % 128 == 0, so a group is never ragged.
    if (!wact || n0 + wn * 128 >= N) return;
    const int G = N >> 7;
    const int grp = (n0 + wn * 128) >> 7;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float a = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            facc[i][j][g][r] = bf16_lo(f32_to_bf16_rne(facc[i][j][g][r]));
            a = fmaxf(a, __builtin_fabsf(facc[i][j][g][r]));
          }
      a = fmaxf(a, __shfl_xor(a, 32));
      const QScale sc = make_scale(a);
      const int ml = wm * 64 + j * 32 + (lane & 31);
      if (ml >= mrows) continue;
      const int64_t m = m0 + ml;
      int8_t* qrow = static_cast<int8_t*>(Y) + m * N + n0 + wn * 128 + 4 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const v4f v = facc[i][j][g];
          *reinterpret_cast<uint32_t*>(qrow + i * 32 + g * 8) =
              pack4(quant_one(v[0], sc), quant_one(v[1], sc), quant_one(v[2], sc), quant_one(v[3], sc));
        }
      if (lane < 32) qs[m * G + grp] = sc.s;
    }
    return;
  }
  if (OUT == OUT_BF16) {
    // the bf16 tile goes through LDS (row r of BN bf16, 16-byte chunk c at
    // c ^ (r & SWZ): 32 chunks a row at BN = 256, 24 = 3 x 8 at 192) so that
    // it leaves in whole rows; the barrier also means every wave is past its
    // last stage read
    constexpr int RB = 2 * BN, SWZ = BN == 256 ? 15 : 7;
    barrier();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (par != 0) break;   // KP: the even waves hold the sums
      const int r = wm * 64 + j * 32 + (lane & 31);
#pragma unroll
      for (int i = 0; i < CI; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint32_t h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) h[q] = f32_to_bf16_rne(facc[i][j][g][q]);
          const int chunk = wn * 4 * CI + i * 4 + g;
          *reinterpret_cast<uint2*>(smem + r * RB + ((chunk ^ (r & SWZ)) << 4) + 8 * (lane >> 5)) =
              make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
        }
    }
    waitcnt<63, 0>();
    barrier();
    // wave w stores tile rows RPW w .. RPW w + RPW - 1, two rows per
    // instruction (a row is LPR lanes of 8 values; at BN = 192 lanes 48..63
    // idle)
    constexpr int RPW = BM / NWV, LPR = BN / 8;
    const int cl = lane % LPR, rl = lane / LPR;
    const int n = n0 + 8 * cl;
    const bool vec8 = (N & 7) == 0 && n + 7 < N;
#pragma unroll 4
    for (int it = 0; it < RPW / 2; ++it) {
      const int r = wave * RPW + 2 * it + (rl < 2 ? rl : 1);
      const v4i v = *reinterpret_cast<const v4i*>(smem + r * RB + ((cl ^ (r & SWZ)) << 4));
      if (rl >= 2 || r >= mrows || n >= N) continue;
      uint16_t* y = static_cast<uint16_t*>(Y) + (int64_t)(m0 + r) * N + n;
      if (vec8) {
        // written once, not read back by this kernel
        __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(y));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < N) y[e] = (uint16_t)(((uint32_t)v[e >> 1]) >> (16 * (e & 1)));
      }
    }
    return;
  }
  if (par != 0) return;   // KP: the even waves hold the sums
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ml = wm * 64 + j * 32 + (lane & 31);
    if (ml >= mrows) continue;
    const int m = m0 + ml;
#pragma unroll
    for (int i = 0; i < CI; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WC + i * 32 + g * 8 + 4 * (lane >> 5);
        if (n >= N) continue;
        store4<OUT>(Y, (int64_t)m * N + n, n, N, vec, facc[i][j][g][0], facc[i][j][g][1], facc[i][j][g][2],
                    facc[i][j][g][3]);
      }
  }
}

template <int MODE, int OUT, int NWM, int NWN = 2, int BN = 256, bool KP = false>
void launch_block_kernel(dim3 grid, hipStream_t st, const int8_t* A, const float* sa, const int8_t* W,
                         const float* sw, const int32_t* off, void* Y, int M, int N, int K, int TM, int TN, int E,
                         float* qs = nullptr, int clo = 0, int chi = 0x7fffffff) {
  hipLaunchKernelGGL((k_gemm_block<MODE, OUT, NWM, NWN, BN, KP>), grid, dim3(64 * NWM * NWN * (KP ? 2 : 1)), 0, st, A,
                     sa, W, sw, off, Y, M, N, K, TM, TN, E, qs, clo, chi);
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
  if ((N & 3) == 0) {
    // 16-byte loads, four slices in flight; the sum stays in slice order
#pragma unroll 4
    for (int sl = 0; sl < S; ++sl) {
      const v4f v = *reinterpret_cast<const v4f*>(ws + sl * MN + idx);
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = __fadd_rn(o[r], v[r]);
    }
  } else {
    for (int sl = 0; sl < S; ++sl)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) o[r] = __fadd_rn(o[r], ws[sl * MN + idx + r]);
  }
  store4<OUT>(Y, idx, n, N, (N & 3) == 0, o[0], o[1], o[2], o[3]);
}

// The same sum in slice order, rounded to bf16 and quantised per 1 x 128
// group along N as quant_act_group does: a group is 32 consecutive threads
// (N % 128 == 0 keeps it inside one row and one half of a wave).
__global__ __launch_bounds__(256) void k_splitk_sum_f32_q8(const float* __restrict__ ws, int S, int M, int N,
                                                           int8_t* __restrict__ q, float* __restrict__ qs) {
  const int64_t q4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nq = N >> 2;
  const bool live = q4 < (int64_t)M * nq;
  const int m = live ? (int)(q4 / nq) : 0, n = live ? (int)(q4 - (int64_t)m * nq) * 4 : 0;
  const int64_t idx = (int64_t)m * N + n;
  const int64_t MN = (int64_t)M * N;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  if (live)
#pragma unroll 4
    for (int sl = 0; sl < S; ++sl) {
      const v4f v = *reinterpret_cast<const v4f*>(ws + sl * MN + idx);
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = __fadd_rn(o[r], v[r]);
    }
  float a = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    o[r] = bf16_lo(f32_to_bf16_rne(o[r]));
    a = fmaxf(a, __builtin_fabsf(o[r]));
  }
  // max over the 32 lanes of this half-wave (the group)
  a = max16(a);
  a = fmaxf(a, __shfl_xor(a, 16));
  const QScale sc = make_scale(a);
  if (!live) return;
  *reinterpret_cast<uint32_t*>(q + idx) =
      pack4(quant_one(o[0], sc), quant_one(o[1], sc), quant_one(o[2], sc), quant_one(o[3], sc));
  if ((threadIdx.x & 31) == 0) qs[(int64_t)m * (N >> 7) + (n >> 7)] = sc.s;
}

// The grouped (MoE) GEMM.  Every expert tile streams its expert's weight
// panel once, so even at a few rows per expert this runs at the weight
// stream's pace; waves whose rows are all past the expert's rows skip their
// MFMAs.  From 96 rows per expert on average, experts with more than 128 rows
// take 256-row tiles (one tile, one pass over the panel, up to 256 rows) and
// the others 128-row tiles, in two launches: a 256-row tile with half its
// row bands idle waits on its loads, a 128-row tile of four waves does not.
// Below 96 rows per expert every expert takes 128-row tiles.  Grids are upper
// bounds on the tile counts (expert row counts live on the device), rounded
// to the XCDs; workgroups past the last tile return at once.
template <int OUT>
hipError_t grouped_launches(const int8_t* A, const float* sa, const int8_t* W, const float* sw, const int32_t* offsets,
                            void* Y, float* qs, int64_t E, int64_t P, int64_t N, int64_t K, hipStream_t st) {
  const int TN = (int)((N + 255) / 256);
  // (four waves: eight waves as 4 x 2 measured 3-4 % slower on the MoE rows)
  constexpr int NWN2 = 2;
  auto round8 = [](int64_t t) { return (t + 7) / 8 * 8; };
  if (P >= 96 * E) {
    const int64_t heavy = P / 129 < E ? P / 129 : E;            // experts with more than 128 rows
    const int64_t TM1 = round8(P / 256 + heavy + 1), TM2 = round8(P < E ? P : E);
    launch_block_kernel<MODE_GROUPED, OUT, 4>(dim3((unsigned)(TM1 * TN)), st, A, sa, W, sw, offsets, Y, (int)P,
                                              (int)N, (int)K, (int)TM1, TN, (int)E, qs, 128, 0x7fffffff);
    launch_block_kernel<MODE_GROUPED, OUT, 2, NWN2>(dim3((unsigned)(TM2 * TN)), st, A, sa, W, sw, offsets, Y, (int)P,
                                              (int)N, (int)K, (int)TM2, TN, (int)E, qs, 0, 128);
  } else {
    const int64_t TM = round8((P + 127) / 128 + E);
    launch_block_kernel<MODE_GROUPED, OUT, 2, NWN2>(dim3((unsigned)(TM * TN)), st, A, sa, W, sw, offsets, Y, (int)P,
                                              (int)N, (int)K, (int)TM, TN, (int)E, qs);
  }
  return hipGetLastError();
}

}  // namespace

namespace {
// Tile shape and K split of the dense tile kernels.  128-row tiles for few
// rows, and where 256-row tiles would leave CUs idle (twice the tiles before
// any K split: DeepSeek's q_a and kv_a projections at 4096 tokens run
// 11-14 % faster than on split 256-row tiles); those are 128 x 256 on eight
// waves as 4 (n) x 2 (m) (two MFMA waves per SIMD: another 4-5 %) or
// 128 x 192 on eight waves by K-block parity, whichever the slice model
// (pick_k_slices) times lower: 192-wide tiles fill the CUs where 256-wide
// ones leave some idle (q_a: 256 tiles instead of 192) and leave no ragged
// tile where N is a multiple of 192 (kv_a, N = 576).
struct BlockPlan {
  int BM, BN, TM, TN, S;
};
BlockPlan plan_block(int64_t M, int64_t N, int64_t K) {
  const int KB = (int)(K >> 7);
  BlockPlan p;
  p.BN = 256;
  p.TN = (int)((N + 255) / 256);
  p.BM = (M <= 128 || ((M + 255) / 256) * p.TN < kTileCUs) ? 128 : 256;
  p.TM = (int)((M + p.BM - 1) / p.BM);
  // microseconds per tile and K block, measured at 4096 rows: 2.6 for
  // 256 x 256 (gate_up), 1.4 for 128 x 256 and 1.17 for the K-parity
  // 128 x 192 tiles (q_a, one round of tiles)
  double t = 0.0;
  p.S = pick_k_slices((int64_t)p.TM * p.TN, KB, M, N, p.BM == 256 ? 2.6 : 1.4, &t);
  if (p.BM == 128) {
    const int TN3 = (int)((N + 191) / 192);
    double t3 = 0.0;
    const int S3 = pick_k_slices((int64_t)p.TM * TN3, KB, M, N, 1.17, &t3);
    if (t3 < t * 0.97) {
      p.BN = 192;
      p.TN = TN3;
      p.S = S3;
    }
  }
  return p;
}
}  // namespace

hipError_t launch_gemm_block(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                             OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (decode_path_takes(M, N, false)) return launch_gemm_block_decode(A, sa, W, sw, Y, out, M, N, K, st);
  const BlockPlan p = plan_block(M, N, K);
  const int BM = p.BM, TM = p.TM, TN = p.TN, S = p.S;
  // a split K takes the stream's scratch, held until the reduction is enqueued
  const WsLease lease = stream_workspace(st, 0, S > 1 ? (size_t)S * M * N * 4 : 0);
  if (lease.status() != kWsOk) return ws_error(lease);
  void* dst = S > 1 ? lease.ptr() : Y;
  const dim3 grid((unsigned)(TM * TN), (unsigned)S);
  const bool f32 = S > 1 || out == OUT_F32;
  if (p.BN == 192) {
    if (f32)
      launch_block_kernel<MODE_DEQUANT, OUT_F32, 2, 2, 192, true>(grid, st, A, sa, W, sw, nullptr, dst, (int)M, (int)N,
                                                                  (int)K, TM, TN, 0);
    else
      launch_block_kernel<MODE_DEQUANT, OUT_BF16, 2, 2, 192, true>(grid, st, A, sa, W, sw, nullptr, dst, (int)M,
                                                                   (int)N, (int)K, TM, TN, 0);
  } else if (BM == 128) {
    if (f32)
      launch_block_kernel<MODE_DEQUANT, OUT_F32, 2, 4>(grid, st, A, sa, W, sw, nullptr, dst, (int)M, (int)N, (int)K,
                                                       TM, TN, 0);
    else
      launch_block_kernel<MODE_DEQUANT, OUT_BF16, 2, 4>(grid, st, A, sa, W, sw, nullptr, dst, (int)M, (int)N, (int)K,
                                                        TM, TN, 0);
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

hipError_t launch_gemm_block_q8(const int8_t* A, const float* sa, const int8_t* W, const float* sw, int8_t* q,
                                float* qs, int64_t M, int64_t N, int64_t K, hipStream_t st) {
  if (decode_path_takes(M, N, false)) {
    // decode-sized M: the weight-streaming kernel that gemm_w8a8_block runs
    // (a wave owns 16 columns, a group spans 8 waves), its bf16 output in the
    // stream's scratch, then the group quantiser; the lease is held until
    // both are enqueued
    const WsLease lease = stream_workspace(st, 0, (size_t)M * N * 2);
    if (lease.status() != kWsOk) return ws_error(lease);
    const hipError_t e = launch_gemm_block_decode(A, sa, W, sw, lease.ptr(), OUT_BF16, M, N, K, st);
    if (e != hipSuccess) return e;
    return launch_quant_group(lease.ptr(), false, M, N, q, qs, st);
  }
  // the tile kernels with launch_gemm_block's tile height and K split on
  // 256-wide tiles (a wave's 128 columns are one group): every output is
  // the same fp32 sum over the same slices, so the same bf16 value.  Where
  // launch_gemm_block takes the K-parity 192-wide tiles (whose sums add the
  // odd blocks' sum to the even blocks'), the same kernel writes fp32 slices
  // and the slice-sum kernel quantises them.
  const BlockPlan p = plan_block(M, N, K);
  if (p.BN == 192) {
    const WsLease lease = stream_workspace(st, 0, (size_t)p.S * M * N * 4);
    if (lease.status() != kWsOk) return ws_error(lease);
    launch_block_kernel<MODE_DEQUANT, OUT_F32, 2, 2, 192, true>(dim3((unsigned)(p.TM * p.TN), (unsigned)p.S), st, A,
                                                                sa, W, sw, nullptr, lease.ptr(), (int)M, (int)N,
                                                                (int)K, p.TM, p.TN, 0);
    const dim3 rg((unsigned)((M * (N / 4) + 255) / 256));
    hipLaunchKernelGGL(k_splitk_sum_f32_q8, rg, dim3(256), 0, st, static_cast<const float*>(lease.ptr()), p.S, (int)M,
                       (int)N, q, qs);
    return hipGetLastError();
  }
  const int TN = (int)((N + 255) / 256);
  const int BM = p.BM, TM = p.TM, S = p.S;
  const dim3 grid((unsigned)(TM * TN), (unsigned)S);
  if (S == 1) {
    if (BM == 128)
      launch_block_kernel<MODE_DEQUANT, OUT_Q8, 2>(grid, st, A, sa, W, sw, nullptr, q, (int)M, (int)N, (int)K, TM, TN,
                                                   0, qs);
    else
      launch_block_kernel<MODE_DEQUANT, OUT_Q8, 4>(grid, st, A, sa, W, sw, nullptr, q, (int)M, (int)N, (int)K, TM, TN,
                                                   0, qs);
    return hipGetLastError();
  }
  // fp32 slices in the stream's scratch, held until the reduction is enqueued
  const WsLease lease = stream_workspace(st, 0, (size_t)S * M * N * 4);
  if (lease.status() != kWsOk) return ws_error(lease);
  if (BM == 128)
    launch_block_kernel<MODE_DEQUANT, OUT_F32, 2, 4>(grid, st, A, sa, W, sw, nullptr, lease.ptr(), (int)M, (int)N, (int)K,
                                                  TM, TN, 0);
  else
    launch_block_kernel<MODE_DEQUANT, OUT_F32, 4>(grid, st, A, sa, W, sw, nullptr, lease.ptr(), (int)M, (int)N, (int)K,
                                                  TM, TN, 0);
  const dim3 rg((unsigned)((M * (N / 4) + 255) / 256));
  hipLaunchKernelGGL(k_splitk_sum_f32_q8, rg, dim3(256), 0, st, static_cast<const float*>(lease.ptr()), S, (int)M,
                     (int)N, q, qs);
  return hipGetLastError();
}

hipError_t launch_gemm_block_grouped_q8(const int8_t* A, const float* sa, const int8_t* W, const float* sw,
                                        const int32_t* offsets, int8_t* q, float* qs, int64_t E, int64_t P,
                                        int64_t N, int64_t K, hipStream_t st) {
  return grouped_launches<OUT_Q8>(A, sa, W, sw, offsets, q, qs, E, P, N, K, st);
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
  return out == OUT_BF16 ? grouped_launches<OUT_BF16>(A, sa, W, sw, offsets, Y, nullptr, E, P, N, K, st)
                         : grouped_launches<OUT_F32>(A, sa, W, sw, offsets, Y, nullptr, E, P, N, K, st);
}

}  // namespace w8
