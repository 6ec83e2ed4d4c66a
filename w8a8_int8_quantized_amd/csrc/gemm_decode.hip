// Small-M (decode-shaped) GEMMs on gfx950: weight streaming.
//
// With M <= 64 the weights dominate the traffic (N x K bytes against M x K of
// activations), so these kernels are HBM-bound: every weight byte is loaded
// once, straight from global memory into MFMA operand registers (no LDS
// staging).  A workgroup owns 16 * FNW output columns; its SK waves split the
// K blocks between them (block kb goes to wave kb % SK), and each wave keeps
// PF blocks of loads in flight in a register ring.  SK is chosen per call so
// that every workgroup of the grid is resident at once (no tail wave of
// workgroups) with as many loads in flight as the register budget allows.
// The per-wave partial results are summed in LDS in wave order, so results
// are deterministic.
//
// Method references:
//   W8A8 block-wise / channel-wise: "DeepSeek R1 INT8 quantisation in SGLang"
//   (Meituan), section 2.3 (per-K-block dequant vs one epilogue dequant);
//   W8A16 group-wise: "DeepSeek-R1-0528-Qwen3-8B Int8 W8A16" release note
//   (symmetric group-wise INT8 weights, fp16 activations).
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "pipeline.h"

namespace w8 {
namespace {

typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));

// SIMDs per GPU the dispatchers size grids against (256 CUs x 4).
constexpr int kSimds = 256 * 4;
constexpr int kCUs = 256;

// Store 4 consecutive outputs of row m (n multiple of 4).
template <int OUT>
__device__ __forceinline__ void store_out4(void* Y, int64_t idx, int n, int N, bool vec, const float* o) {
  if (OUT == OUT_F32) {
    float* y = static_cast<float*>(Y) + idx;
    if (vec && n + 3 < N) {
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
    if (vec && n + 3 < N) {
      *reinterpret_cast<uint2*>(y) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) y[r] = (uint16_t)h[r];
    }
  }
}

// Branch-free loads.  Every operand is read through a raw buffer descriptor
// whose range ends at the last valid byte; a load past it returns zero and
// moves no data.  Rows past M or N fall outside their descriptor by
// construction, and the K blocks past the end of a wave's share get the
// offset kOob added (beyond every range used here: a descriptor spans at most
// 64 rows x 2^20 columns x 2 bytes).  No load sits under a branch, so the
// compiler keeps the whole prefetch ring in flight (a branch around a load
// makes it wait for every outstanding load at the join).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOob = 0x40000000u;

// Base and size are workgroup-uniform; readfirstlane states it, so the
// descriptor stays in scalar registers (a descriptor the compiler cannot
// prove uniform gets a loop around every load).  A size computed as zero or
// less (a wave past the last column in a later K slice) becomes an empty
// range: every load through it reads zero.
__device__ __forceinline__ rsrc_t rsrc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)(bytes > 0 ? bytes : 0));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(lo | (hi << 32)), 0, n, 0x00020000);
}
__device__ __forceinline__ v4i bl16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ v2i bl8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v2i, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ float blf(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// --------------------------------------------------------------- W8A8
// MODE 0: block-wise (fp32 accumulate of per-block dequantised partials);
// MODE 1: channel-wise (int32 accumulate over all K, one epilogue dequant).
// Fragment layout (v_mfma_i32_16x16x64_i8 with W as operand A): lane l holds
// weight row n0 + 16 f + (l & 15) and activation row 16 j + (l & 15), K bytes
// 16 q .. 16 q + 15 (q = l >> 4) of each 64-wide half of the K block; the
// result lane holds columns n0 + 16 f + 4 q + r (r = 0..3) of row 16 j + (l & 15).
// STS (MODE 0): the activation scales of all K blocks ([16 MF][KB] floats,
// rows past M zero, rows KB | 1 floats apart) are staged in dynamic LDS
// before the loop, as in k_decode_shared, instead of one scale load per
// fragment row, block and lane (a cache line per row).
template <int MODE, int MF, int FNW, int SK, int PF, int OUT, bool STS = false>
__global__ __launch_bounds__(64 * SK) void k_decode_w8a8(const int8_t* __restrict__ A, const float* __restrict__ sa,
                                                         const int8_t* __restrict__ W, const float* __restrict__ sw,
                                                         void* __restrict__ Y, int M, int N, int K) {
  static_assert(!STS || MODE == 0, "staged scales: block-wise");
  __shared__ v4i red[SK][64];
  extern __shared__ float dss[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int n0 = blockIdx.x * 16 * FNW;
  const int KB = K >> 7;
  const int rows = N - n0 < 16 * FNW ? N - n0 : 16 * FNW;

  // W rows n0 .. n0 + rows - 1; the workgroup's columns lie in one 128-row
  // weight block (16 * FNW divides 128), so its block scales are one row of sw.
  const rsrc_t rw = rsrc(W + (int64_t)n0 * K, (int64_t)rows * K);
  const rsrc_t ra = rsrc(A, (int64_t)M * K);
  const rsrc_t rsw = rsrc(sw + (int64_t)(n0 >> 7) * KB, (int64_t)KB * 4);
  const rsrc_t rsa = rsrc(sa, (int64_t)M * KB * 4);
  uint32_t woff[FNW], aoff[MF], saoff[MF];
#pragma unroll
  for (int f = 0; f < FNW; ++f) woff[f] = (uint32_t)((f * 16 + (lane & 15)) * K + q * 16);
#pragma unroll
  for (int j = 0; j < MF; ++j) {
    aoff[j] = (uint32_t)((j * 16 + (lane & 15)) * K + q * 16);
    saoff[j] = (uint32_t)((j * 16 + (lane & 15)) * KB * 4);
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

  // register ring: PF K blocks in flight per wave
  v4i wv[PF][FNW][2], av[PF][MF][2];
  float ssa[PF][MF], ssw[PF][FNW];
  auto load = [&](int P, int kb) {
    const uint32_t ko = kb < KB ? (uint32_t)kb * 128u : kOob;
    const uint32_t so = kb < KB ? (uint32_t)kb * 4u : kOob;
#pragma unroll
    for (int f = 0; f < FNW; ++f) {
      wv[P][f][0] = bl16(rw, woff[f] + ko);
      wv[P][f][1] = bl16(rw, woff[f] + ko + 64);
      if (MODE == 0) ssw[P][f] = blf(rsw, so);
    }
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      av[P][j][0] = bl16(ra, aoff[j] + ko);
      av[P][j][1] = bl16(ra, aoff[j] + ko + 64);
      if (MODE == 0 && !STS) ssa[P][j] = blf(rsa, saoff[j] + so);
    }
  };
  constexpr int NT = 64 * SK, SCH = 16;
  const int SST = KB | 1;
  const int stot = 16 * MF * KB;
  float sv[SCH];
  auto scl_load = [&](int e0) {
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const int e = e0 + i * NT + (int)threadIdx.x;
      sv[i] = blf(rsa, e < stot ? (uint32_t)e * 4u : kOob);
    }
  };
  auto scl_store = [&](int e0) {
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const int e = e0 + i * NT + (int)threadIdx.x;
      if (e < stot) {
        const int r = e / KB;
        dss[r * SST + (e - r * KB)] = sv[i];
      }
    }
  };
  if constexpr (STS) scl_load(0);
  // the prologue issues the slots in ring order (the scheduler would reverse
  // them, and the loop would then wait for the whole ring on every pass)
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    load(p, wave + p * SK);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (STS) {
    scl_store(0);
    for (int e0 = SCH * NT; e0 < stot; e0 += SCH * NT) {
      scl_load(e0);
      scl_store(e0);
    }
    __syncthreads();
  }
  // this wave's K blocks: wave, wave + SK, ...; PF of them per iteration, the
  // slots past the end hold zeros
  const int nb = (KB - wave + SK - 1) / SK;
  const int iters = (nb + PF - 1) / PF;
  for (int it = 0; it < iters; ++it) {
    const int kb0 = wave + it * SK * PF;
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      // consume slot p, then refill it with the block SK * PF further on;
      // the other PF - 1 slots stay in flight meanwhile
#pragma unroll
      for (int f = 0; f < FNW; ++f)
#pragma unroll
        for (int j = 0; j < MF; ++j) {
          if (MODE == 0) {
            v4i pp = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[p][f][0], av[p][j][0], (v4i){0, 0, 0, 0}, 0, 0, 0);
            pp = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[p][f][1], av[p][j][1], pp, 0, 0, 0);
            // slot p holds block kb0 + p SK; blocks past the last take a
            // zero scale (past a row's end lie the padding and the next row)
            const int kbp = kb0 + p * SK;
            const float sap = STS ? (kbp < KB ? dss[(16 * j + (lane & 15)) * SST + kbp] : 0.f) : ssa[p][j];
            const float s = __fmul_rn(sap, ssw[p][f]);
#pragma unroll
            for (int r = 0; r < 4; ++r) facc[f][j][r] = __builtin_fmaf(s, (float)pp[r], facc[f][j][r]);
          } else {
            iacc[f][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[p][f][0], av[p][j][0], iacc[f][j], 0, 0, 0);
            iacc[f][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[p][f][1], av[p][j][1], iacc[f][j], 0, 0, 0);
          }
        }
      load(p, kb0 + p * SK + SK * PF);
      // keep slot p's consumers here: hoisted above the refills of earlier
      // slots they would make the wave wait for the whole ring
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // cross-wave reduction, one fragment at a time, summed in wave order
  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int f = 0; f < FNW; ++f)
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      red[wave][lane] = MODE == 0 ? __builtin_bit_cast(v4i, facc[f][j]) : iacc[f][j];
      __syncthreads();
      if (wave == ((f * MF + j) % SK)) {
        const int n = n0 + f * 16 + 4 * q;
        const int m = j * 16 + (lane & 15);
        if (n < N && m < M) {
          float o[4];
          if (MODE == 0) {
            v4f t = __builtin_bit_cast(v4f, red[0][lane]);
#pragma unroll
            for (int w = 1; w < SK; ++w) t += __builtin_bit_cast(v4f, red[w][lane]);
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = t[r];
            store_out4<OUT>(Y, (int64_t)m * N + n, n, N, vec, o);
          } else {
            v4i t = red[0][lane];
#pragma unroll
            for (int w = 1; w < SK; ++w) t += red[w][lane];
            if (OUT == OUT_I32) {
              int32_t* y = static_cast<int32_t*>(Y) + (int64_t)m * N + n;
              if (vec && n + 3 < N) {
                *reinterpret_cast<v4i*>(y) = t;
              } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (n + r < N) y[r] = t[r];
              }
            } else {
              const float s_m = sa[m];
#pragma unroll
              for (int r = 0; r < 4; ++r) o[r] = n + r < N ? __fmul_rn((float)t[r], __fmul_rn(s_m, sw[n + r])) : 0.f;
              store_out4<OUT>(Y, (int64_t)m * N + n, n, N, vec, o);
            }
          }
        }
      }
      __syncthreads();
    }
}

// --------------------------------------------------------------- W8A8, shared activations
// Same contraction and fragment layout as k_decode_w8a8, organised so that
// the activations are loaded once per workgroup rather than once per wave:
// the workgroup's NWV waves own
// 16 adjacent columns each and walk the same K blocks.  The activations move
// in groups of G K blocks: while the waves multiply group g out of one LDS
// buffer, group g + 1 (already in registers) is written to the other and
// group g + 2 is loaded; one barrier per group.  Stage layout: G blocks of
// 16 MF rows x 128 bytes, row r's 16-byte chunk c stored at c ^ (r & 7), so
// fragment reads are conflict-free.  Weights stream straight into registers
// through a PF-deep ring (PF a multiple of G).  No cross-wave reduction: every
// wave covers all of K for its columns.  The dispatcher sizes workgroups so
// that the grid splits evenly over the CUs (the weight stream runs at the pace
// of the most loaded CU).  Block-wise (MODE 0), the activation scales of all
// K blocks ([16 MF][KB] floats, rows past M zero) are staged in dynamic LDS
// once, before the loop, by consecutive dword loads of the row-major array
// (a row's scales in one place, rather than one cache line per row and
// group); rows are stored KB | 1 floats apart, an odd stride, so the 16 rows
// a fragment read touches fall in distinct banks.
template <int MODE, int MF, int NWV, int G, int PF, int OUT>
__global__ __launch_bounds__(64 * NWV) void k_decode_shared(const int8_t* __restrict__ A, const float* __restrict__ sa,
                                                        const int8_t* __restrict__ W, const float* __restrict__ sw,
                                                        void* __restrict__ Y, int M, int N, int K) {
  constexpr int FNW = 1;
  constexpr int ROWS = 16 * MF;                                  // activation rows per block
  constexpr int CHUNKS = ROWS * 8;                               // 16-byte chunks per block
  constexpr int NT = 64 * NWV;                                   // threads
  constexpr int AG = (G * CHUNKS + NT - 1) / NT;                 // chunks per thread per group
  __shared__ v4i as[2][G * CHUNKS];
  extern __shared__ float ssa[];   // MODE 0: ROWS rows of KB | 1 floats
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int KB = K >> 7;
  const int NG = (KB + G - 1) / G;
  const int cg = blockIdx.x;
  const int n0 = cg * 16 * FNW * NWV;
  const int nw = n0 + 16 * FNW * wave;
  int rows = N - nw;
  rows = rows < 0 ? 0 : (rows > 16 * FNW ? 16 * FNW : rows);

  // a wave's 16 FNW columns lie in one 128-row weight block (16 FNW divides
  // 128 and nw is a multiple of 16 FNW), so its block scales are one row of sw
  const int nwc = rows > 0 ? nw : 0;
  const rsrc_t rw = rsrc(W + (int64_t)nwc * K, (int64_t)rows * K);
  const rsrc_t ra = rsrc(A, (int64_t)M * K);
  const rsrc_t rsw = rsrc(sw + (int64_t)(nwc >> 7) * KB, (int64_t)KB * 4);
  const rsrc_t rsa = rsrc(sa, (int64_t)M * KB * 4);
  uint32_t woff[FNW];
#pragma unroll
  for (int f = 0; f < FNW; ++f) woff[f] = (uint32_t)((16 * f + (lane & 15)) * K + q * 16);
  // group chunk e = threadIdx.x + i NT: block e / CHUNKS, row (e % CHUNKS) >> 3,
  // 16-byte column e & 7
  uint32_t aoff[AG];
  int apos[AG];
#pragma unroll
  for (int i = 0; i < AG; ++i) {
    const int e = threadIdx.x + i * NT;
    const int bk = e / CHUNKS, r = (e % CHUNKS) >> 3, col = e & 7;
    const bool ok = e < G * CHUNKS;
    aoff[i] = ok ? (uint32_t)(r * K + bk * 128 + col * 16) : kOob;
    apos[i] = ok ? bk * CHUNKS + r * 8 + (col ^ (r & 7)) : -1;
  }
  const int SST = KB | 1;   // row stride of the staged activation scales

  v4f facc[FNW][MF];
  v4i iacc[FNW][MF];
#pragma unroll
  for (int f = 0; f < FNW; ++f)
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      facc[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};
      iacc[f][j] = (v4i){0, 0, 0, 0};
    }

  v4i areg[AG];
  auto load_act = [&](int g) {  // group g's activations into registers
    const uint32_t ko = g < NG ? (uint32_t)g * G * 128u : kOob;
#pragma unroll
    for (int i = 0; i < AG; ++i) areg[i] = bl16(ra, aoff[i] + ko);
  };
  auto store_act = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AG; ++i)
      if (apos[i] >= 0) as[buf][apos[i]] = areg[i];
  };
  // the activation scales of every K block (MODE 0): flat element e of
  // [ROWS][KB], past M * KB zero; sixteen dword loads per thread at a time
  constexpr int SCH = 16;
  const int stot = ROWS * KB;
  float sv[SCH];
  auto scl_load = [&](int e0) {
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const int e = e0 + i * NT + (int)threadIdx.x;
      sv[i] = blf(rsa, e < stot ? (uint32_t)e * 4u : kOob);
    }
  };
  auto scl_store = [&](int e0) {
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      const int e = e0 + i * NT + (int)threadIdx.x;
      if (e < stot) {
        const int r = e / KB;
        ssa[r * SST + (e - r * KB)] = sv[i];
      }
    }
  };
  v4i wv[PF][FNW][2];
  float swv[PF];
  auto load_w = [&](int P, int kb) {
    const uint32_t ko = kb < KB ? (uint32_t)kb * 128u : kOob;
#pragma unroll
    for (int f = 0; f < FNW; ++f) {
      wv[P][f][0] = bl16(rw, woff[f] + ko);
      wv[P][f][1] = bl16(rw, woff[f] + ko + 64);
    }
    if (MODE == 0) swv[P] = blf(rsw, kb < KB ? (uint32_t)kb * 4u : kOob);
  };

  // prologue, issued in the order the loop issues: group 0 staged, then the
  // weight ring, then group 1 (the scales' first loads go out first and are
  // stored once the ring is on its way)
  if constexpr (MODE == 0) scl_load(0);
  load_act(0);
  store_act(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    load_w(p, p);
    __builtin_amdgcn_sched_barrier(0);
  }
  load_act(1);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MODE == 0) {
    scl_store(0);
    for (int e0 = SCH * NT; e0 < stot; e0 += SCH * NT) {
      scl_load(e0);
      scl_store(e0);
    }
  }
  waitcnt<63, 0>();
  barrier();

  // super-steps of PF K blocks (PF / G activation groups); blocks and groups
  // past the end read as zero
  const int iters = (NG * G + PF - 1) / PF;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int kb = it * PF + p;
      const int g = it * (PF / G) + p / G;
      const int buf = g & 1;
      const int bo = (p % G) * CHUNKS;
      // row groups in chunks of up to four (bounds the fragment registers
      // beyond 64 rows), skipping chunks past the tile's rows
      constexpr int JC = MF <= 4 ? MF : 4;
#pragma unroll
      for (int j0 = 0; j0 < MF; j0 += JC) {
        if (JC < MF && j0 * 16 >= M) continue;
        v4i af[JC][2];
        float saj[JC];
#pragma unroll
        for (int jj = 0; jj < JC; ++jj) {
          const int r = 16 * (j0 + jj) + (lane & 15);
          af[jj][0] = as[buf][bo + r * 8 + (q ^ (r & 7))];
          af[jj][1] = as[buf][bo + r * 8 + ((4 + q) ^ (r & 7))];
          // blocks past the last take a zero scale (past a row's end lie
          // the padding and the next row, whose scale may be infinite and
          // must not meet this row's zero partial)
          if (MODE == 0) saj[jj] = kb < KB ? ssa[r * SST + kb] : 0.f;
        }
#pragma unroll
        for (int f = 0; f < FNW; ++f)
#pragma unroll
          for (int jj = 0; jj < JC; ++jj) {
            const int j = j0 + jj;
            if (MODE == 0) {
              v4i pp = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[p][f][0], af[jj][0], (v4i){0, 0, 0, 0}, 0, 0, 0);
              pp = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[p][f][1], af[jj][1], pp, 0, 0, 0);
              const float s = __fmul_rn(saj[jj], swv[p]);
#pragma unroll
              for (int r = 0; r < 4; ++r) facc[f][j][r] = __builtin_fmaf(s, (float)pp[r], facc[f][j][r]);
            } else {
              iacc[f][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[p][f][0], af[jj][0], iacc[f][j], 0, 0, 0);
              iacc[f][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[p][f][1], af[jj][1], iacc[f][j], 0, 0, 0);
            }
          }
        if (JC < MF) __builtin_amdgcn_sched_barrier(0);
      }
      load_w(p, kb + PF);
      __builtin_amdgcn_sched_barrier(0);
      if (p % G == G - 1) {
        // end of group g: every wave finished reading buffer buf ^ 1
        // (group g - 1) before the previous barrier, so group g + 1 may
        // overwrite it
        store_act(buf ^ 1);
        load_act(g + 2);
        __builtin_amdgcn_sched_barrier(0);
        waitcnt<63, 0>();
        barrier();
      }
    }
  }

  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int f = 0; f < FNW; ++f) {
    const int n = nw + 16 * f + 4 * q;
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      const int m = 16 * j + (lane & 15);
      if (n < N && m < M) {
        float o[4];
        if (MODE == 0) {
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = facc[f][j][r];
          store_out4<OUT>(Y, (int64_t)m * N + n, n, N, vec, o);
        } else if (OUT == OUT_I32) {
          int32_t* y = static_cast<int32_t*>(Y) + (int64_t)m * N + n;
          if (vec && n + 3 < N) {
            *reinterpret_cast<v4i*>(y) = iacc[f][j];
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < N) y[r] = iacc[f][j][r];
          }
        } else {
          const float s_m = sa[m];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            o[r] = n + r < N ? __fmul_rn((float)iacc[f][j][r], __fmul_rn(s_m, sw[n + r])) : 0.f;
          store_out4<OUT>(Y, (int64_t)m * N + n, n, N, vec, o);
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
    const v2h h = __builtin_bit_cast(v2h, w[i]) - bias;
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

// INT4 weights: a 32-bit word holds the codes of 8 consecutive k as
// offset-binary nibbles u = q + 8 (the even k in the low nibble of its byte).
// The nibbles are spread one per byte in k order, then each byte u goes under
// the high byte 0x64 (the fp16 value 1024 + u) and 1032 is subtracted: q
// exactly.
__device__ __forceinline__ v8h i4x8_to_f16(uint32_t w) {
  const uint32_t lo = w & 0x0F0F0F0Fu;           // k = 0, 2, 4, 6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;    // k = 1, 3, 5, 7
  const uint32_t a = __builtin_amdgcn_perm(hi, lo, 0x05010400u);   // k = 0 .. 3
  const uint32_t b = __builtin_amdgcn_perm(hi, lo, 0x07030602u);   // k = 4 .. 7
  uint32_t h2[4];
  h2[0] = __builtin_amdgcn_perm(0x64646464u, a, 0x04010400u);
  h2[1] = __builtin_amdgcn_perm(0x64646464u, a, 0x04030402u);
  h2[2] = __builtin_amdgcn_perm(0x64646464u, b, 0x04010400u);
  h2[3] = __builtin_amdgcn_perm(0x64646464u, b, 0x04030402u);
  v8h r;
  const v2h bias = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v2h h = __builtin_bit_cast(v2h, h2[i]) - bias;
    r[2 * i] = h[0];
    r[2 * i + 1] = h[1];
  }
  return r;
}

// The weight registers of one 128-wide group for one lane: 32 int8 codes
// (two 16-byte loads) or 32 INT4 codes (two 8-byte loads), k = 64 h + 16 q +
// [0, 16) for h = 0, 1; and their fp16 values, 8 per MFMA operand.
template <bool W4>
struct WFrag {
  using T = typename std::conditional<W4, v2i, v4i>::type;
  static constexpr int kBytesPerGroup = W4 ? 64 : 128;   // bytes of one row per 128-wide group
  static constexpr int kLaneBytes = W4 ? 8 : 16;         // bytes of a lane's 16 consecutive k
  __device__ static T load(rsrc_t r, uint32_t off) {
    if constexpr (W4) return bl8(r, off);
    else return bl16(r, off);
  }
  // wh[t]: k = 64 (t / 2) + 16 q + 8 (t % 2) + [0, 8)
  __device__ static void to_f16(const T& w0, const T& w1, v8h (&wh)[4]) {
    if constexpr (W4) {
      wh[0] = i4x8_to_f16((uint32_t)w0[0]);
      wh[1] = i4x8_to_f16((uint32_t)w0[1]);
      wh[2] = i4x8_to_f16((uint32_t)w1[0]);
      wh[3] = i4x8_to_f16((uint32_t)w1[1]);
    } else {
      wh[0] = i8x8_to_f16(w0[0], w0[1]);
      wh[1] = i8x8_to_f16(w0[2], w0[3]);
      wh[2] = i8x8_to_f16(w1[0], w1[1]);
      wh[3] = i8x8_to_f16(w1[2], w1[3]);
    }
  }
};

// v_mfma_f32_16x16x32_f16 with W as operand A.  Per 128-wide group a lane
// loads 32 weight bytes of row n (k = 64 h + 16 q + [0, 16), h = 0, 1) and,
// for MFMA t = 0..3, the 8 activation halves at k = 64 (t/2) + 16 q + 8 (t%2).
// XL (one row fragment, M <= 4): the M x K activations are staged once per
// workgroup in dynamic LDS (M K 2 bytes, then a 256-byte zero region that
// the fragment rows past M read), so a K block costs the weight and scale
// loads and four LDS reads instead of four activation loads per wave.
// W4: INT4 weights, [N][K / 2] bytes (WFrag).
template <int MF, int FNW, int SK, int PF, bool XL, bool W4 = false>
__global__ __launch_bounds__(64 * SK) void k_decode_w8a16(const uint16_t* __restrict__ x, const uint8_t* __restrict__ W,
                                                          const float* __restrict__ ws, uint16_t* __restrict__ Y, int M,
                                                          int N, int K) {
  static_assert(!XL || MF == 1, "staged activations take one row fragment");
  using WF = WFrag<W4>;
  const int KW = W4 ? K >> 1 : K;   // bytes per weight row
  __shared__ v4f red[SK][64];
  extern __shared__ __attribute__((aligned(16))) char xs[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q = lane >> 4;
  const int n0 = blockIdx.x * 16 * FNW;
  const int KB = K >> 7;

  const int rows = N - n0 < 16 * FNW ? N - n0 : 16 * FNW;
  const rsrc_t rw = rsrc(W + (int64_t)n0 * KW, (int64_t)rows * KW);
  const rsrc_t rs = rsrc(ws + (int64_t)n0 * KB, (int64_t)rows * KB * 4);
  const rsrc_t rx = rsrc(x, (int64_t)M * K * 2);
  uint32_t woff[FNW], soff[FNW], xoff[MF];
#pragma unroll
  for (int f = 0; f < FNW; ++f) {
    woff[f] = (uint32_t)((f * 16 + (lane & 15)) * KW + q * WF::kLaneBytes);
    soff[f] = (uint32_t)((f * 16 + 4 * q) * KB * 4);
  }
#pragma unroll
  for (int j = 0; j < MF; ++j) xoff[j] = (uint32_t)(((j * 16 + (lane & 15)) * K + q * 16) * 2);
  // staged activations: row r = lane & 15 at r K 2 bytes (rows past M: the
  // zero region, the same 256 bytes for every K block)
  const int xr = lane & 15;
  const uint32_t xb = XL ? (uint32_t)(xr < M ? xr * K * 2 : M * K * 2) + q * 32 : 0;
  const uint32_t xg = xr < M ? 256u : 0u;
  if constexpr (XL) {
    const int nch = M * K / 8;   // 16-byte chunks of x
    for (int i = threadIdx.x; i < nch; i += 64 * SK) reinterpret_cast<v4i*>(xs)[i] = bl16(rx, (uint32_t)i * 16);
    if (threadIdx.x < 16) reinterpret_cast<v4i*>(xs + M * K * 2)[threadIdx.x] = (v4i){0, 0, 0, 0};
    __syncthreads();
  }

  v4f facc[FNW][MF];
#pragma unroll
  for (int f = 0; f < FNW; ++f)
#pragma unroll
    for (int j = 0; j < MF; ++j) facc[f][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  typename WF::T wv[PF][FNW][2];
  v8h xv[PF][MF][4];
  float sv[PF][FNW][4];
  auto load = [&](int P, int g) {
    const uint32_t ko = g < KB ? (uint32_t)g * WF::kBytesPerGroup : kOob;
    const uint32_t xk = g < KB ? (uint32_t)g * 256u : kOob;   // the group's fp16 activations
    const uint32_t so = g < KB ? (uint32_t)g * 4u : kOob;
#pragma unroll
    for (int f = 0; f < FNW; ++f) {
      wv[P][f][0] = WF::load(rw, woff[f] + ko);
      wv[P][f][1] = WF::load(rw, woff[f] + ko + WF::kBytesPerGroup / 2);
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[P][f][r] = blf(rs, soff[f] + r * KB * 4 + so);
    }
    if constexpr (XL) {
      const uint32_t xo = xb + (uint32_t)(g < KB ? g : 0) * xg;
#pragma unroll
      for (int t = 0; t < 4; ++t) xv[P][0][t] = *reinterpret_cast<const v8h*>(xs + xo + (t >> 1) * 128 + (t & 1) * 16);
    } else {
#pragma unroll
      for (int j = 0; j < MF; ++j)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          xv[P][j][t] = __builtin_bit_cast(v8h, bl16(rx, xoff[j] + xk + (t >> 1) * 128 + (t & 1) * 16));
    }
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    load(p, wave + p * SK);
    __builtin_amdgcn_sched_barrier(0);
  }
  const int nb = (KB - wave + SK - 1) / SK;
  const int iters = (nb + PF - 1) / PF;
  for (int it = 0; it < iters; ++it) {
    const int g0 = wave + it * SK * PF;
#pragma unroll
    for (int p = 0; p < PF; ++p) {
#pragma unroll
      for (int f = 0; f < FNW; ++f) {
        v8h wh[4];
        WF::to_f16(wv[p][f][0], wv[p][f][1], wh);
#pragma unroll
        for (int j = 0; j < MF; ++j) {
          v4f pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int t = 0; t < 4; ++t) pp = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh[t], xv[p][j][t], pp, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) facc[f][j][r] = __builtin_fmaf(sv[p][f][r], pp[r], facc[f][j][r]);
        }
      }
      load(p, g0 + p * SK + SK * PF);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  const bool vec = (N & 3) == 0;
#pragma unroll
  for (int f = 0; f < FNW; ++f)
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      red[wave][lane] = facc[f][j];
      __syncthreads();
      if (wave == ((f * MF + j) % SK)) {
        const int n = n0 + f * 16 + 4 * q;
        const int m = j * 16 + (lane & 15);
        if (n < N && m < M) {
          v4f t = red[0][lane];
#pragma unroll
          for (int w = 1; w < SK; ++w) t += red[w][lane];
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
      __syncthreads();
    }
}

// W8A16 with shared activations: the organisation of k_decode_shared (NWV
// waves of 16 columns walking the same K blocks, activations staged per
// workgroup in groups of G K blocks, weights through a PF-deep register ring)
// with the fragment layout of k_decode_w8a16.  A staged row holds 128 fp16
// values (256 bytes, 16 chunks of 16 bytes); chunk c of row r is stored at
// c ^ (r & 15).
// KPAR = 2: twice the waves, the second NWV taking the odd K blocks (each
// wave's ring then holds every other block, and a staged group of G = 2
// blocks is one step for both halves); the odd sums are added to the even
// ones through LDS at the end (even + odd).
template <int MF, int NWV, int G, int PF, bool W4 = false, int KPAR = 1>
__global__ __launch_bounds__(64 * NWV * KPAR) void k_w8a16_shared(const uint16_t* __restrict__ x,
                                                           const uint8_t* __restrict__ W,
                                                           const float* __restrict__ ws, uint16_t* __restrict__ Y,
                                                           int M, int N, int K) {
  static_assert(KPAR == 1 || (KPAR == 2 && G == 2), "K parity: a staged group is the two halves' blocks");
  using WF = WFrag<W4>;
  const int KW = W4 ? K >> 1 : K;   // bytes per weight row
  constexpr int ROWS = 16 * MF;
  constexpr int CHUNKS = ROWS * 16;
  constexpr int NT = 64 * NWV * KPAR;
  constexpr int AG = (G * CHUNKS + NT - 1) / NT;
  __shared__ v4i xs[2][G * CHUNKS];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wcol = KPAR == 1 ? wave : wave % NWV;   // the wave's 16 columns
  const int par = KPAR == 1 ? 0 : wave / NWV;       // its first K block
  const int q = lane >> 4;
  const int nw = blockIdx.x * 16 * NWV + 16 * wcol;
  const int KBt = K >> 7;
  // split-K: slice blockIdx.y of gridDim.y covers K blocks kbs .. kbe - 1;
  // every descriptor starts at the slice's first block (rows past the end
  // still fall outside), and the slices write fp32 partials
  const int kbs = (int)((int64_t)blockIdx.y * KBt / gridDim.y);
  const int KB = (int)((int64_t)(blockIdx.y + 1) * KBt / gridDim.y) - kbs;
  const int NG = (KB + G - 1) / G;
  int rows = N - nw;
  rows = rows < 0 ? 0 : (rows > 16 ? 16 : rows);
  const int nwc = rows > 0 ? nw : 0;

  const rsrc_t rw = rsrc(W + (int64_t)nwc * KW + kbs * WF::kBytesPerGroup,
                        (int64_t)rows * KW - kbs * WF::kBytesPerGroup);
  const rsrc_t rs = rsrc(ws + (int64_t)nwc * KBt + kbs, (int64_t)rows * KBt * 4 - kbs * 4);
  const rsrc_t rx = rsrc(x + kbs * 128, (int64_t)M * K * 2 - kbs * 256);
  const uint32_t woff = (uint32_t)((lane & 15) * KW + q * WF::kLaneBytes);
  const uint32_t soff = (uint32_t)(4 * q * KBt * 4);
  // activation chunk i of a group: K block xbk[i] of the group; blocks past
  // the slice's last read zero (the bytes there belong to the next slice or,
  // in the last slice, the next row, whose non-finite values must not reach
  // this row through a zero weight)
  uint32_t xoff[AG];
  int xpos[AG], xbk[AG];
#pragma unroll
  for (int i = 0; i < AG; ++i) {
    const int e = threadIdx.x + i * NT;
    const int bk = e / CHUNKS, r = (e % CHUNKS) >> 4, col = e & 15;
    const bool ok = e < G * CHUNKS;
    xoff[i] = ok ? (uint32_t)(r * K * 2 + bk * 256 + col * 16) : kOob;
    xpos[i] = ok ? bk * CHUNKS + r * 16 + (col ^ (r & 15)) : -1;
    xbk[i] = bk;
  }

  v4f facc[MF];
#pragma unroll
  for (int j = 0; j < MF; ++j) facc[j] = (v4f){0.f, 0.f, 0.f, 0.f};

  v4i xreg[AG];
  auto load_act = [&](int g) {
    const int left = KB - g * G;  // K blocks of the slice from this group on
#pragma unroll
    for (int i = 0; i < AG; ++i) {
      const uint32_t ko = xbk[i] < left ? (uint32_t)g * G * 256u : kOob;
      xreg[i] = bl16(rx, xoff[i] + ko);
    }
  };
  auto store_act = [&](int buf) {
#pragma unroll
    for (int i = 0; i < AG; ++i)
      if (xpos[i] >= 0) xs[buf][xpos[i]] = xreg[i];
  };
  // The ring holds the wave's consecutive steps, slot p step it PF + p, step
  // t being K block KPAR t + par.  Slots SB i .. SB i + SB - 1 (SB = 4, or
  // PF if less; 2 with K parity) share the scales sv[i] of their SB blocks
  // for the lane's four columns, loaded with the last of those slots (when
  // all of their previous blocks are done): 4 SB consecutive bytes per
  // column, or with K parity 16 bytes covering the pair's blocks kf and
  // kf + 2; scales past the slice's last block belong to the next row or
  // read zero, and multiply zero products (the activations staged for those
  // blocks read zero; their weight bytes read zero too, which INT4 decodes
  // as code -8, not 0).
  constexpr int SB = KPAR == 2 ? 2 : (PF < 4 ? PF : 4);
  static_assert(PF % SB == 0 && (SB == 4 || SB == 2), "scales load two or four K blocks at a time");
  typename WF::T wv[PF][2];
  float sv[PF / SB][4][SB];
  auto load_w = [&](int P, int t) {
    const int kb = KPAR * t + par;
    const uint32_t ko = kb < KB ? (uint32_t)kb * WF::kBytesPerGroup : kOob;
    wv[P][0] = WF::load(rw, woff + ko);
    wv[P][1] = WF::load(rw, woff + ko + WF::kBytesPerGroup / 2);
    if (P % SB == SB - 1) {
      const int kf = kb - KPAR * (SB - 1);   // the block of the group's first slot
      const uint32_t so = kf < KB ? (uint32_t)kf * 4u : kOob;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (KPAR == 2) {
          const v4f t4 = __builtin_bit_cast(v4f, bl16(rs, soff + r * KBt * 4 + so));
          sv[P / SB][r][0] = t4[0];
          sv[P / SB][r][1] = t4[2];
        } else if constexpr (SB == 4) {
          const v4f t = __builtin_bit_cast(v4f, bl16(rs, soff + r * KBt * 4 + so));
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[P / SB][r][e] = t[e];
        } else {
          const v2i t = bl8(rs, soff + r * KBt * 4 + so);
          sv[P / SB][r][0] = __builtin_bit_cast(float, t[0]);
          sv[P / SB][r][1] = __builtin_bit_cast(float, t[1]);
        }
      }
    }
  };

  load_act(0);
  store_act(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    load_w(p, p);
    __builtin_amdgcn_sched_barrier(0);
  }
  load_act(1);
  __builtin_amdgcn_sched_barrier(0);
  waitcnt<63, 0>();
  barrier();

  // steps: K blocks (K parity: pairs of blocks, one staged group each)
  const int iters = (KPAR == 1 ? NG * G + PF - 1 : NG + PF - 1) / PF;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int t = it * PF + p;
      const int g = KPAR == 1 ? it * (PF / G) + p / G : t;
      const int buf = g & 1;
      const int bo = KPAR == 1 ? (p % G) * CHUNKS : par * CHUNKS;
      v8h wh[4];
      WF::to_f16(wv[p][0], wv[p][1], wh);
#pragma unroll
      for (int j = 0; j < MF; ++j) {
        const int r = 16 * j + (lane & 15);
        v4f pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int c = 8 * (t >> 1) + 2 * q + (t & 1);
          const v8h xv = __builtin_bit_cast(v8h, xs[buf][bo + r * 16 + (c ^ (r & 15))]);
          pp = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh[t], xv, pp, 0, 0, 0);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) facc[j][rr] = __builtin_fmaf(sv[p / SB][rr][p % SB], pp[rr], facc[j][rr]);
      }
      load_w(p, t + PF);
      __builtin_amdgcn_sched_barrier(0);
      if (KPAR == 2 || p % G == G - 1) {
        store_act(buf ^ 1);
        load_act(g + 2);
        __builtin_amdgcn_sched_barrier(0);
        waitcnt<63, 0>();
        barrier();
      }
    }
  }
  if constexpr (KPAR == 2) {
    // every wave is past its reads of xs (the loop ends with a barrier):
    // the odd-block sums through it, added to the even ones (even + odd)
    v4f* red = reinterpret_cast<v4f*>(&xs[0][0]) + wcol * MF * 64 + lane;
    if (par == 1) {
#pragma unroll
      for (int j = 0; j < MF; ++j) red[j * 64] = facc[j];
    }
    barrier();
    if (par == 1) return;
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      const v4f o = red[j * 64];
#pragma unroll
      for (int r = 0; r < 4; ++r) facc[j][r] = __fadd_rn(facc[j][r], o[r]);
    }
  }

  const bool vec = (N & 3) == 0;
  const int n = nw + 4 * q;
  if (gridDim.y > 1) {
    float* yp = reinterpret_cast<float*>(Y) + (int64_t)blockIdx.y * M * N;
#pragma unroll
    for (int j = 0; j < MF; ++j) {
      const int m = 16 * j + (lane & 15);
      if (n >= N || m >= M) continue;
      float* y = yp + (int64_t)m * N + n;
      if (vec && n + 3 < N) {
        *reinterpret_cast<v4f*>(y) = facc[j];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) y[r] = facc[j][r];
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < MF; ++j) {
    const int m = 16 * j + (lane & 15);
    if (n < N && m < M) {
      uint16_t h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = __builtin_bit_cast(uint16_t, (_Float16)facc[j][r]);
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

// Sum of S fp32 W8A16 slices in slice order, rounded to fp16 (4 outputs per
// thread).
__global__ __launch_bounds__(256) void k_w16_slices_sum(const float* __restrict__ part, int S, int M, int N,
                                                        uint16_t* __restrict__ Y) {
  const int64_t q4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nq = (N + 3) >> 2;
  if (q4 >= (int64_t)M * nq) return;
  const int m = (int)(q4 / nq), n = (int)(q4 - (int64_t)m * nq) * 4;
  const int64_t idx = (int64_t)m * N + n, MN = (int64_t)M * N;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  for (int sl = 0; sl < S; ++sl)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) o[r] = __fadd_rn(o[r], part[sl * MN + idx + r]);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (n + r < N) Y[idx + r] = __builtin_bit_cast(uint16_t, (_Float16)o[r]);
}

// Waves per workgroup: as many as keep the whole grid resident given the
// variant's occupancy (waves per SIMD its register use allows), at most 8 and
// no more than there are K blocks.
inline int pick_sk(int64_t workgroups, int64_t kblocks, int max_sk, int waves_per_simd) {
  int sk = (int)((int64_t)kSimds * waves_per_simd / (workgroups > 0 ? workgroups : 1));
  if (sk > max_sk) sk = max_sk;
  if (sk > kblocks) sk = (int)kblocks;
  if (sk >= 8) return 8;
  if (sk >= 4) return 4;
  if (sk >= 2) return 2;
  return 1;
}

// Dynamic LDS of the block-wise decode kernels' staged scales: 16 MF rows of
// activation scales, KB | 1 floats apart.
inline size_t shared_scale_lds(int MF, int64_t K) { return (size_t)16 * MF * ((K >> 7) | 1) * 4; }
constexpr size_t kSharedScaleLdsMax = 64 * 1024;

template <int MODE, int MF, int FNW, int PF, int OUT>
hipError_t decode_launch(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y, int64_t M,
                         int64_t N, int64_t K, int waves_per_simd, hipStream_t st) {
  const int64_t wgs = (N + 16 * FNW - 1) / (16 * FNW);
  const int sk = pick_sk(wgs, K >> 7, 8, waves_per_simd);
  const dim3 g((unsigned)wgs);
  const int m = (int)M, n = (int)N, k = (int)K;
  // block-wise: activation scales staged in LDS where they fit the budget
  // (64-row tiles only with eight waves, whose launch bounds hold the kernel
  // to 208 registers; with fewer it takes 260 and one wave per SIMD)
  const size_t lds = shared_scale_lds(MF, K);
  if (MODE == 0 && lds <= kSharedScaleLdsMax && (MF < 4 || sk == 8)) {
    switch (sk) {
      case 8: hipLaunchKernelGGL((k_decode_w8a8<MODE, MF, FNW, 8, PF, OUT, MODE == 0>), g, dim3(512), lds, st, A, sa, W, sw, Y, m, n, k); break;
      case 4: hipLaunchKernelGGL((k_decode_w8a8<MODE, MF, FNW, 4, PF, OUT, MODE == 0>), g, dim3(256), lds, st, A, sa, W, sw, Y, m, n, k); break;
      case 2: hipLaunchKernelGGL((k_decode_w8a8<MODE, MF, FNW, 2, PF, OUT, MODE == 0>), g, dim3(128), lds, st, A, sa, W, sw, Y, m, n, k); break;
      default: hipLaunchKernelGGL((k_decode_w8a8<MODE, MF, FNW, 1, PF, OUT, MODE == 0>), g, dim3(64), lds, st, A, sa, W, sw, Y, m, n, k); break;
    }
    return hipGetLastError();
  }
  switch (sk) {
    case 8: hipLaunchKernelGGL((k_decode_w8a8<MODE, MF, FNW, 8, PF, OUT>), g, dim3(512), 0, st, A, sa, W, sw, Y, m, n, k); break;
    case 4: hipLaunchKernelGGL((k_decode_w8a8<MODE, MF, FNW, 4, PF, OUT>), g, dim3(256), 0, st, A, sa, W, sw, Y, m, n, k); break;
    case 2: hipLaunchKernelGGL((k_decode_w8a8<MODE, MF, FNW, 2, PF, OUT>), g, dim3(128), 0, st, A, sa, W, sw, Y, m, n, k); break;
    default: hipLaunchKernelGGL((k_decode_w8a8<MODE, MF, FNW, 1, PF, OUT>), g, dim3(64), 0, st, A, sa, W, sw, Y, m, n, k); break;
  }
  return hipGetLastError();
}

// Weight-ring depth for the shared-activation kernels: a CU needs about
// 44 KB of weights in flight (its share of the HBM stream times the loaded
// latency), i.e. 22 K-block slots of 2 KB over its resident waves.
inline int pick_ring_depth(int64_t N, int nwv) {
  const int64_t wgs = (N + 16 * nwv - 1) / (16 * nwv);
  const int64_t waves_per_cu = nwv * ((wgs + kCUs - 1) / kCUs);
  return waves_per_cu <= 4 ? 8 : (waves_per_cu <= 8 ? 4 : 2);
}

template <int MODE, int MF, int NWV, int PF, int OUT>
hipError_t shared_launch(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y, int64_t M,
                         int64_t N, int64_t K, hipStream_t st) {
  const dim3 g((unsigned)((N + 16 * NWV - 1) / (16 * NWV)));
  const size_t lds = MODE == 0 ? shared_scale_lds(MF, K) : 0;
  hipLaunchKernelGGL((k_decode_shared<MODE, MF, NWV, 2, PF, OUT>), g, dim3(64 * NWV), lds, st, A, sa, W, sw, Y,
                     (int)M, (int)N, (int)K);
  return hipGetLastError();
}

template <int MODE, int MF, int NWV, int OUT>
hipError_t shared_depth(int pf, const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y, int64_t M,
                        int64_t N, int64_t K, hipStream_t st) {
  // (only the pairings the depth rule can produce are instantiated)
  if constexpr (NWV <= 4) {
    if (pf == 8) return shared_launch<MODE, MF, NWV, 8, OUT>(A, sa, W, sw, Y, M, N, K, st);
  }
  if constexpr (NWV <= 8) {
    if (pf >= 4) return shared_launch<MODE, MF, NWV, 4, OUT>(A, sa, W, sw, Y, M, N, K, st);
  }
  return shared_launch<MODE, MF, NWV, 2, OUT>(A, sa, W, sw, Y, M, N, K, st);
}

template <int MODE, int MF, int OUT>
hipError_t shared_width(int nwv, const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y, int64_t M,
                        int64_t N, int64_t K, hipStream_t st) {
  const int pf = pick_ring_depth(N, nwv);
  switch (nwv) {
    case 3: return shared_depth<MODE, MF, 3, OUT>(pf, A, sa, W, sw, Y, M, N, K, st);
    case 4: return shared_depth<MODE, MF, 4, OUT>(pf, A, sa, W, sw, Y, M, N, K, st);
    case 6: return shared_depth<MODE, MF, 6, OUT>(pf, A, sa, W, sw, Y, M, N, K, st);
    case 8: return shared_depth<MODE, MF, 8, OUT>(pf, A, sa, W, sw, Y, M, N, K, st);
    default: return shared_depth<MODE, MF, 9, OUT>(pf, A, sa, W, sw, Y, M, N, K, st);
  }
}

// Workgroup width (waves of 16 columns) for the shared-activation kernel:
// the weight stream runs at the pace of the most loaded CU, so pick the width
// whose grid splits most evenly over the CUs (ties go to the wider one, which
// loads the activations fewer times).  0: no width splits evenly enough.
inline int pick_shared_width(int64_t N) {
  static const int widths[] = {9, 8, 6, 4, 3};
  const int64_t frags = (N + 15) / 16;
  int best = 0;
  double best_eff = 0.85;
  for (int w : widths) {
    const int64_t wgs = (frags + w - 1) / w;
    const int64_t per_cu = (wgs + kCUs - 1) / kCUs;
    const double eff = (double)frags / (double)(kCUs * per_cu * w);
    if (eff > best_eff + 0.02) {
      best = w;
      best_eff = eff;
    }
  }
  return best;
}

template <int MODE, int OUT>
hipError_t decode_dispatch(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y, int64_t M,
                           int64_t N, int64_t K, hipStream_t st) {
  int nwv = pick_shared_width(N);
  // block-wise: the staged activation scales must fit their LDS budget
  // (K up to 32640 at 64 rows); longer K runs the split-K decode kernel
  if (MODE == 0 && shared_scale_lds(M <= 16 ? 1 : (M <= 32 ? 2 : 4), K) > kSharedScaleLdsMax) nwv = 0;
  if (nwv > 0) {
    if (M <= 16) return shared_width<MODE, 1, OUT>(nwv, A, sa, W, sw, Y, M, N, K, st);
    if (M <= 32) return shared_width<MODE, 2, OUT>(nwv, A, sa, W, sw, Y, M, N, K, st);
    if constexpr (MODE == 1) {
      if (M > 64) return shared_width<MODE, 8, OUT>(nwv, A, sa, W, sw, Y, M, N, K, st);
    }
    return shared_width<MODE, 4, OUT>(nwv, A, sa, W, sw, Y, M, N, K, st);
  }
  if (M <= 16) return decode_launch<MODE, 1, 1, 4, OUT>(A, sa, W, sw, Y, M, N, K, 3, st);
  if (M <= 32) return decode_launch<MODE, 2, 2, 2, OUT>(A, sa, W, sw, Y, M, N, K, 2, st);
  return decode_launch<MODE, 4, 2, 2, OUT>(A, sa, W, sw, Y, M, N, K, 2, st);
}

template <int MF, int FNW, int PF, bool XL, bool W4>
hipError_t w8a16_launch(const uint16_t* x, const uint8_t* W, const float* s, uint16_t* Y, int M, int64_t N, int64_t K,
                        int waves_per_simd, hipStream_t st) {
  const int64_t wgs = (N + 16 * FNW - 1) / (16 * FNW);
  const int sk = pick_sk(wgs, K >> 7, 8, waves_per_simd);
  const dim3 g((unsigned)wgs);
  const int n = (int)N, k = (int)K;
  const size_t lds = XL ? (size_t)M * K * 2 + 256 : 0;
  switch (sk) {
    case 8: hipLaunchKernelGGL((k_decode_w8a16<MF, FNW, 8, PF, XL, W4>), g, dim3(512), lds, st, x, W, s, Y, M, n, k); break;
    case 4: hipLaunchKernelGGL((k_decode_w8a16<MF, FNW, 4, PF, XL, W4>), g, dim3(256), lds, st, x, W, s, Y, M, n, k); break;
    case 2: hipLaunchKernelGGL((k_decode_w8a16<MF, FNW, 2, PF, XL, W4>), g, dim3(128), lds, st, x, W, s, Y, M, n, k); break;
    default: hipLaunchKernelGGL((k_decode_w8a16<MF, FNW, 1, PF, XL, W4>), g, dim3(64), lds, st, x, W, s, Y, M, n, k); break;
  }
  return hipGetLastError();
}

template <int MF, int NWV, int PF, bool W4, int KPAR>
hipError_t w8a16_shared_launch(const uint16_t* x, const uint8_t* W, const float* s, uint16_t* Y, int M, int64_t N,
                               int64_t K, int S, hipStream_t st) {
  const dim3 g((unsigned)((N + 16 * NWV - 1) / (16 * NWV)), (unsigned)S);
  hipLaunchKernelGGL((k_w8a16_shared<MF, NWV, 2, PF, W4, KPAR>), g, dim3(64 * NWV * KPAR), 0, st, x, W, s, Y, M,
                     (int)N, (int)K);
  return hipGetLastError();
}

template <int MF, int NWV, bool W4, int KPAR>
hipError_t w8a16_shared_depth(int pf, int S, const uint16_t* x, const uint8_t* W, const float* s, uint16_t* Y, int M,
                              int64_t N, int64_t K, hipStream_t st) {
  if constexpr (NWV <= 4) {
    if (pf == 8) return w8a16_shared_launch<MF, NWV, 8, W4, KPAR>(x, W, s, Y, M, N, K, S, st);
  }
  if constexpr (NWV <= 8) {
    if (pf >= 4) return w8a16_shared_launch<MF, NWV, 4, W4, KPAR>(x, W, s, Y, M, N, K, S, st);
  }
  return w8a16_shared_launch<MF, NWV, 2, W4, KPAR>(x, W, s, Y, M, N, K, S, st);
}

template <int MF, bool W4, int KPAR = 1>
hipError_t w8a16_shared_width(int nwv, int pf, int S, const uint16_t* x, const uint8_t* W, const float* s, uint16_t* Y,
                              int M, int64_t N, int64_t K, hipStream_t st) {
  switch (nwv) {
    case 3: return w8a16_shared_depth<MF, 3, W4, KPAR>(pf, S, x, W, s, Y, M, N, K, st);
    case 4: return w8a16_shared_depth<MF, 4, W4, KPAR>(pf, S, x, W, s, Y, M, N, K, st);
    case 6: return w8a16_shared_depth<MF, 6, W4, KPAR>(pf, S, x, W, s, Y, M, N, K, st);
    case 8: return w8a16_shared_depth<MF, 8, W4, KPAR>(pf, S, x, W, s, Y, M, N, K, st);
    default:
      // nine waves twice over would exceed a workgroup's 16 waves
      if constexpr (KPAR == 1) return w8a16_shared_depth<MF, 9, W4, 1>(pf, S, x, W, s, Y, M, N, K, st);
      else return hipErrorInvalidConfiguration;
  }
}

}  // namespace

bool decode_path_takes(int64_t M, int64_t N, bool channel) {
  return M <= 64 || (channel && M <= 128 && pick_shared_width(N) > 0);
}

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

namespace {

template <bool W4>
hipError_t group16_dispatch(const uint16_t* x, const uint8_t* W, const float* s, uint16_t* Y, int64_t M, int64_t N,
                           int64_t K, hipStream_t st) {
  // Per 64-row slice: up to 4 rows the split-K decode kernel with x staged in
  // LDS; 5..16 rows the shared-activation kernel when N balances over the CUs
  // (its activation stage is shared by the workgroup's waves; where N does
  // not balance, its K split and reduction cost more than the decode
  // kernel's per-wave activation loads), else the decode kernel; more rows
  // the shared-activation kernel.  Its width comes from the balance rule (4
  // waves where no width balances), K is split over S workgroups until there
  // are two per CU below 32 rows and one from there (slices of at least 4 K
  // blocks), the ring depth follows the
  // waves per CU, and the slices' fp32 partials go to the split-K workspace
  // and are summed in order.
  const int nwv0 = pick_shared_width(N);
  const int nwv = nwv0 > 0 ? nwv0 : 4;
  const int min_shared = nwv0 > 0 ? 5 : 17;   // fewest rows a slice takes to the shared kernel
  const int64_t wgs1 = (N + 16 * nwv - 1) / (16 * nwv);
  const int64_t KBt = K >> 7;
  // from 17 rows the workgroup runs twice its waves, the second half on the
  // odd K blocks (K parity): more waves per CU to hide the activation
  // staging and load latency without another split of K (a workgroup holds
  // at most 16 waves)
  const int kpar = M >= 17 && nwv <= 8 ? 2 : 1;
  int S = 1;
  // (from 32 rows one workgroup per CU: the slices' partials and their
  // reduction then cost more than the second workgroup's latency hiding)
  const int64_t target = M >= 32 ? kCUs : 2 * kCUs;
  while (wgs1 * S < target && S < 8 && KBt / (2 * S) >= 4) S *= 2;
  const int64_t wpc = nwv * kpar * ((wgs1 * S + kCUs - 1) / kCUs);
  const int pf = wpc <= 4 ? 8 : (wpc <= 8 ? 4 : 2);
  // slices' fp32 partials in the stream's scratch, held until every
  // reduction below is enqueued
  const bool split = S > 1 && M >= min_shared;
  const WsLease lease = stream_workspace(st, 0, split ? (size_t)S * (M < 64 ? M : 64) * N * 4 : 0);
  if (lease.status() != kWsOk) return ws_error(lease);
  float* part = split ? static_cast<float*>(lease.ptr()) : nullptr;
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
    const int mm = (int)(M - m0 < 64 ? M - m0 : 64);
    const uint16_t* xs = x + m0 * K;
    uint16_t* ys = Y + m0 * N;
    hipError_t e;
    if (mm >= min_shared) {
      uint16_t* dst = S > 1 ? reinterpret_cast<uint16_t*>(part) : ys;
      if (kpar == 2)
        e = mm <= 16 ? w8a16_shared_width<1, W4, 2>(nwv, pf, S, xs, W, s, dst, mm, N, K, st)
            : mm <= 32 ? w8a16_shared_width<2, W4, 2>(nwv, pf, S, xs, W, s, dst, mm, N, K, st)
                     : w8a16_shared_width<4, W4, 2>(nwv, pf, S, xs, W, s, dst, mm, N, K, st);
      else
        e = mm <= 16 ? w8a16_shared_width<1, W4>(nwv, pf, S, xs, W, s, dst, mm, N, K, st)
            : mm <= 32 ? w8a16_shared_width<2, W4>(nwv, pf, S, xs, W, s, dst, mm, N, K, st)
                     : w8a16_shared_width<4, W4>(nwv, pf, S, xs, W, s, dst, mm, N, K, st);
      if (e == hipSuccess && S > 1) {
        const dim3 rg((unsigned)((mm * ((N + 3) / 4) + 255) / 256));
        hipLaunchKernelGGL(k_w16_slices_sum, rg, dim3(256), 0, st, part, S, mm, (int)N, ys);
        e = hipGetLastError();
      }
    } else if (mm <= 4 && (int64_t)mm * K * 2 + 256 <= 96 * 1024) {
      e = w8a16_launch<1, 1, 4, true, W4>(xs, W, s, ys, mm, N, K, 3, st);
    } else {
      e = w8a16_launch<1, 1, 4, false, W4>(xs, W, s, ys, mm, N, K, 3, st);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_gemm_w8a16(const uint16_t* x, const int8_t* W, const float* s, uint16_t* Y, int64_t M, int64_t N,
                             int64_t K, hipStream_t st) {
  return group16_dispatch<false>(x, reinterpret_cast<const uint8_t*>(W), s, Y, M, N, K, st);
}

hipError_t launch_gemm_w4a16(const uint16_t* x, const uint8_t* W4, const float* s, uint16_t* Y, int64_t M, int64_t N,
                             int64_t K, hipStream_t st) {
  return group16_dispatch<true>(x, W4, s, Y, M, N, K, st);
}

}  // namespace w8
