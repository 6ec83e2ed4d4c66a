// Quantisation kernels for gfx950: online activation quantisation (per
// token-group and per token) and the offline weight conversions.
//
// Method: "DeepSeek R1 INT8 quantisation in SGLang" (Meituan), section 2.3:
//   - block-wise scheme: 128 x 128 weight tiles, activations per token-group;
//   - channel-wise scheme: one scale per output channel, activations per token;
//   - offline: FP8 checkpoint -> BF16 -> INT8.
// Quantiser: "FP8 vs INT8 quantisation for DeepSeek", section 3.2.1 (int8
// branch): s = amax / 127, q = round(x / s) clamped to +-127.
//
// All kernels are HBM-streaming: every input byte is read once (the token
// and tile quantisers keep their group in registers between the amax pass and
// the quantise pass) and every output byte written once.
#include "common.h"
#include "launch.h"

namespace w8 {
namespace {

// ------------------------------------------------------------------ decode
// OCP FP8-E4M3FN byte J of w -> fp32 (exact: gfx950's v_cvt_f32_fp8 decodes
// the OCP encoding, bias 7, subnormals included; the GPU tests cover every
// finite code), times scale_inv in fp32, rounded to bf16 (nearest even);
// returned as the fp32 value of that bf16 (its bit pattern is the top half).
template <int J>
__device__ __forceinline__ float fp8_to_bf16_value(uint32_t w, float scale_inv) {
  const float p = __fmul_rn(__builtin_amdgcn_cvt_f32_fp8((int)w, J), scale_inv);
  const uint32_t u = __float_as_uint(p);
  return __uint_as_float((u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u);
}

// 16 values from a 16-byte chunk of FP8 codes.
__device__ __forceinline__ void unpack16_fp8(const uint4& c, float scale_inv, float* v) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[4 * i + 0] = fp8_to_bf16_value<0>(w[i], scale_inv);
    v[4 * i + 1] = fp8_to_bf16_value<1>(w[i], scale_inv);
    v[4 * i + 2] = fp8_to_bf16_value<2>(w[i], scale_inv);
    v[4 * i + 3] = fp8_to_bf16_value<3>(w[i], scale_inv);
  }
}

// ------------------------------------------------------- per token-group
// Each group of 128 values (256 bytes) is handled by 8 lanes, 16 values per
// lane (two 16-byte loads), so one wave quantises 8 groups per round and a
// 256-thread workgroup 32 groups per round, 2 rounds per workgroup.
constexpr int kGroupRounds = 2;
constexpr int kGroupsPerBlock = 32 * kGroupRounds;

// I4: the INT4 weight quantiser on the same groups: scale amax / 7, codes
// clamped to [-7, 7] and stored as offset-binary nibbles (q + 8, the even k
// in the low nibble), 64 bytes per group, 8 per lane.
template <bool FP16, bool I4 = false>
__global__ __launch_bounds__(256) void k_quant_group(const uint4* __restrict__ x, int8_t* __restrict__ q,
                                                     float* __restrict__ scale, int64_t G) {
  const int j = threadIdx.x & 7;
  uint4 raw[kGroupRounds][2];
  int64_t gidx[kGroupRounds];
#pragma unroll
  for (int r = 0; r < kGroupRounds; ++r) {
    int64_t g = (int64_t)blockIdx.x * kGroupsPerBlock + r * 32 + (threadIdx.x >> 3);
    gidx[r] = g;
    int64_t gl = g < G ? g : G - 1;             // clamped: tail lanes load a valid group
    const uint4* p = x + gl * 16 + 2 * j;       // 16 chunks of 16 B per group
    raw[r][0] = p[0];
    raw[r][1] = p[1];
  }
#pragma unroll
  for (int r = 0; r < kGroupRounds; ++r) {
    float v[16];
    unpack8<FP16>(raw[r][0], v);
    unpack8<FP16>(raw[r][1], v + 8);
    float a = max8(amax_n(v, 16));
    if constexpr (I4) {
      const QScale sc = make_scale4(a);
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float t = fminf(fmaxf(quant_one(v[i], sc), -7.f), 7.f);
        w[i >> 3] |= (uint32_t)((int)t + 8) << (4 * (i & 7));
      }
      if (gidx[r] < G) {
        reinterpret_cast<uint2*>(q + gidx[r] * 64)[j] = make_uint2(w[0], w[1]);
        if (j == 0) scale[gidx[r]] = sc.s;
      }
      continue;
    }
    QScale sc = make_scale(a);
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = quant_one(v[i], sc);
    if (gidx[r] < G) {
      uint4 o;
      o.x = pack4(t[0], t[1], t[2], t[3]);
      o.y = pack4(t[4], t[5], t[6], t[7]);
      o.z = pack4(t[8], t[9], t[10], t[11]);
      o.w = pack4(t[12], t[13], t[14], t[15]);
      reinterpret_cast<uint4*>(q + gidx[r] * 128)[j] = o;
      if (j == 0) scale[gidx[r]] = sc.s;
    }
  }
}

// ------------------------------------------------------------ per row
// One 256-thread workgroup per row.  A "chunk" is 16 input bytes: 8 bf16 /
// fp16 values, or 16 FP8 codes.  The first CH chunks of every thread stay in
// registers between the amax pass and the quantise pass; rows longer than
// 256 * CH chunks re-read the rest (from L2) in the second pass.
enum { FMT_BF16 = 0, FMT_FP16 = 1, FMT_FP8 = 2 };

template <int FMT>
struct RowFmt {
  static constexpr int EPC = FMT == FMT_FP8 ? 16 : 8;   // elements per chunk
};

template <int FMT>
__device__ __forceinline__ void chunk_values(const uint4& c, float si, float* v) {
  if constexpr (FMT == FMT_FP8) {
    unpack16_fp8(c, si, v);
  } else {
    unpack8<FMT == FMT_FP16>(c, v);
  }
}

template <int FMT, int CH>
__global__ __launch_bounds__(256) void k_quant_row(const uint4* __restrict__ x, const float* __restrict__ scale_inv,
                                                   int8_t* __restrict__ q, float* __restrict__ scale, int K) {
  constexpr int EPC = RowFmt<FMT>::EPC;
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int nch = K / EPC;
  const uint4* xr = x + row * (int64_t)nch;
  // FP8 rows: scale_inv[row / 128][kb]; each 16-code chunk lies in one K block.
  const float* sir = FMT == FMT_FP8 ? scale_inv + (row >> 7) * (int64_t)(K >> 7) : nullptr;
  uint4 keep[CH];
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    int c = threadIdx.x + 256 * i;
    if (c < nch) keep[i] = xr[c];
  }
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    int c = threadIdx.x + 256 * i;
    if (c < nch) {
      float v[EPC];
      chunk_values<FMT>(keep[i], FMT == FMT_FP8 ? sir[(c * EPC) >> 7] : 0.f, v);
      a = fmaxf(a, amax_n(v, EPC));
    }
  }
  for (int c = threadIdx.x + 256 * CH; c < nch; c += 256) {
    float v[EPC];
    chunk_values<FMT>(xr[c], FMT == FMT_FP8 ? sir[(c * EPC) >> 7] : 0.f, v);
    a = fmaxf(a, amax_n(v, EPC));
  }
  a = block_max256(a, red);
  QScale sc = make_scale(a);
  int8_t* qr = q + row * (int64_t)K;
  auto emit = [&](const uint4& raw, int c) {
    float v[EPC];
    chunk_values<FMT>(raw, FMT == FMT_FP8 ? sir[(c * EPC) >> 7] : 0.f, v);
    float t[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) t[e] = quant_one(v[e], sc);
    if constexpr (EPC == 8) {
      uint2 o;
      o.x = pack4(t[0], t[1], t[2], t[3]);
      o.y = pack4(t[4], t[5], t[6], t[7]);
      reinterpret_cast<uint2*>(qr)[c] = o;
    } else {
      uint4 o;
      o.x = pack4(t[0], t[1], t[2], t[3]);
      o.y = pack4(t[4], t[5], t[6], t[7]);
      o.z = pack4(t[8], t[9], t[10], t[11]);
      o.w = pack4(t[12], t[13], t[14], t[15]);
      reinterpret_cast<uint4*>(qr)[c] = o;
    }
  };
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    int c = threadIdx.x + 256 * i;
    if (c < nch) emit(keep[i], c);
  }
  for (int c = threadIdx.x + 256 * CH; c < nch; c += 256) emit(xr[c], c);
  if (threadIdx.x == 0) scale[row] = sc.s;
}

// ---------------------------------------------------------- 128x128 tiles
// One 256-thread workgroup per tile (grid x = kb, y = nb).
// bf16 input: the tile is 128 rows x 256 bytes = 2048 chunks, 8 per thread:
// thread t takes column chunk t & 15 of rows (t >> 4) + 16 i.
__global__ __launch_bounds__(256) void k_quant_tile_bf16(const uint4* __restrict__ w, int8_t* __restrict__ q,
                                                         float* __restrict__ scale, int N, int K) {
  __shared__ float red[4];
  const int KB = K >> 7;
  const int kb = (int)(blockIdx.x % (unsigned)KB), nb = (int)(blockIdx.x / (unsigned)KB);
  const int cc = threadIdx.x & 15;
  const int nchr = K >> 3;   // 16-byte chunks per row
  uint4 raw[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = nb * 128 + (threadIdx.x >> 4) + 16 * i;
    int rl = r < N ? r : N - 1;
    raw[i] = w[(int64_t)rl * nchr + kb * 16 + cc];
  }
  float a = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = nb * 128 + (threadIdx.x >> 4) + 16 * i;
    float v[8];
    unpack8<false>(raw[i], v);
    if (r < N) a = fmaxf(a, amax_n(v, 8));
  }
  a = block_max256(a, red);
  QScale sc = make_scale(a);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = nb * 128 + (threadIdx.x >> 4) + 16 * i;
    float v[8], t[8];
    unpack8<false>(raw[i], v);
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = quant_one(v[e], sc);
    if (r < N) {
      uint2 o;
      o.x = pack4(t[0], t[1], t[2], t[3]);
      o.y = pack4(t[4], t[5], t[6], t[7]);
      reinterpret_cast<uint2*>(q + (int64_t)r * K + kb * 128)[cc] = o;
    }
  }
  if (threadIdx.x == 0) scale[(int64_t)nb * KB + kb] = sc.s;
}

// FP8 input: one 256-thread workgroup per strip of 128 rows x 4 K blocks
// (4 tiles, 64 KB of codes, all loaded up front).  Thread t takes the 16-byte
// column chunk t & 31 of rows (t >> 5) + 8 i, i < 16: every row is read as
// 512 contiguous bytes, and all 16 chunks of a thread lie in tile
// (t & 31) >> 3.  Inside a tile every value is bf16(decode(code) *
// scale_inv) with one scale_inv, so its INT8 code is a function of the FP8
// byte alone: the tile amax comes from the codes (a finite code's magnitude
// increases with its low 7 bits, and the fp32 product and the bf16 rounding
// are monotone, so the largest |value| is that of the largest low-7-bit
// code), then each thread quantises one byte value per tile with the exact
// quotient rule into a 256-entry table, and the elements are looked up.
// (Quantising element by element, FP8 values often sit exactly on a
// half-integer of the grid, e.g. half the tile's largest value lands on 63.5,
// and the exact-quotient fallback then runs for most waves.)
constexpr int kStripTiles = 4;
typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Max over the 8 lanes of each half of a 16-lane DPP row, unsigned integers.
__device__ __forceinline__ uint32_t max8u(uint32_t v) {
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  return v;
}

template <bool WRITE_BF16>
__global__ __launch_bounds__(256) void k_requant_tile_fp8(const uint4* __restrict__ w, const float* __restrict__ scale_inv,
                                                          int8_t* __restrict__ q, float* __restrict__ scale,
                                                          uint16_t* __restrict__ wbf, int N, int K) {
  __shared__ uint32_t red[4][kStripTiles];
  __shared__ uint8_t lut[kStripTiles][256];
  __shared__ uint16_t lutb[WRITE_BF16 ? kStripTiles : 1][256];
  const int KB = K >> 7;
  const int NS = (KB + kStripTiles - 1) / kStripTiles;
  const int sb = (int)(blockIdx.x % (unsigned)NS), nb = (int)(blockIdx.x / (unsigned)NS);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cc = threadIdx.x & 31;
  const int tile = cc >> 3;
  const int kb = sb * kStripTiles + tile;          // this thread's K block
  const bool kok = kb < KB;
  const int kbc = kok ? kb : KB - 1;               // clamped: threads past the last block load a valid one
  const int nchr = K >> 4;
  uint4 raw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = nb * 128 + (threadIdx.x >> 5) + 8 * i;
    const int rl = r < N ? r : N - 1;
    raw[i] = w[(int64_t)rl * nchr + kbc * 8 + (cc & 7)];
  }
  // largest low-7-bit code of this thread's rows (bytes as u16 pairs)
  v2u16 mlo = {0, 0}, mhi = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = nb * 128 + (threadIdx.x >> 5) + 8 * i;
    if (r < N) {
      const uint32_t wv[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t m = wv[k] & 0x7f7f7f7fu;
        mlo = __builtin_elementwise_max(mlo, __builtin_bit_cast(v2u16, m & 0x00ff00ffu));
        mhi = __builtin_elementwise_max(mhi, __builtin_bit_cast(v2u16, (m >> 8) & 0x00ff00ffu));
      }
    }
  }
  const v2u16 mm = __builtin_elementwise_max(mlo, mhi);
  uint32_t code = mm[0] > mm[1] ? mm[0] : mm[1];
  // tile maximum: octet (8 lanes), then octets o and o + 4 of the wave, then waves
  code = max8u(code);
  {
    // lane t < 4 collects tile t from lanes 8 t and 32 + 8 t
    const uint32_t lo = __shfl(code, 8 * (lane & 3), 64), hi = __shfl(code, 32 + 8 * (lane & 3), 64);
    if (lane < kStripTiles) red[wave][lane] = lo > hi ? lo : hi;
  }
  __syncthreads();
  // thread c quantises byte value c for each tile of the strip
#pragma unroll
  for (int tt = 0; tt < kStripTiles; ++tt) {
    const uint32_t mc = umax(umax(red[0][tt], red[1][tt]), umax(red[2][tt], red[3][tt]));
    const int kt = sb * kStripTiles + tt < KB ? sb * kStripTiles + tt : KB - 1;
    const float sit = scale_inv[(int64_t)nb * KB + kt];
    const QScale sc = make_scale(__builtin_fabsf(fp8_to_bf16_value<0>(mc, __builtin_fabsf(sit))));
    const float x = fp8_to_bf16_value<0>(threadIdx.x, sit);
    lut[tt][threadIdx.x] = (uint8_t)(int)quant_one(x, sc);
    if (WRITE_BF16) lutb[tt][threadIdx.x] = (uint16_t)(__float_as_uint(x) >> 16);
    if (threadIdx.x == 0 && sb * kStripTiles + tt < KB) scale[(int64_t)nb * KB + sb * kStripTiles + tt] = sc.s;
  }
  __syncthreads();
  if (!kok) return;
  const uint8_t* lt = lut[tile];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = nb * 128 + (threadIdx.x >> 5) + 8 * i;
    if (r < N) {
      const uint32_t wv[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o[k] = (uint32_t)lt[wv[k] & 0xff] | ((uint32_t)lt[(wv[k] >> 8) & 0xff] << 8) |
               ((uint32_t)lt[(wv[k] >> 16) & 0xff] << 16) | ((uint32_t)lt[wv[k] >> 24] << 24);
      reinterpret_cast<uint4*>(q + (int64_t)r * K + kb * 128)[cc & 7] = make_uint4(o[0], o[1], o[2], o[3]);
      if (WRITE_BF16) {
        const uint16_t* lb = lutb[tile];
        uint32_t h[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          h[2 * k] = (uint32_t)lb[wv[k] & 0xff] | ((uint32_t)lb[(wv[k] >> 8) & 0xff] << 16);
          h[2 * k + 1] = (uint32_t)lb[(wv[k] >> 16) & 0xff] | ((uint32_t)lb[wv[k] >> 24] << 16);
        }
        uint4* dst = reinterpret_cast<uint4*>(wbf + (int64_t)r * K + kb * 128) + 2 * (cc & 7);
        dst[0] = make_uint4(h[0], h[1], h[2], h[3]);
        dst[1] = make_uint4(h[4], h[5], h[6], h[7]);
      }
    }
  }
}

template <int FMT>
hipError_t launch_row(const void* x, const float* si, int64_t M, int64_t K, int8_t* q, float* s, hipStream_t st) {
  constexpr int EPC = RowFmt<FMT>::EPC;
  const int64_t nch = K / EPC;
  const uint4* xp = static_cast<const uint4*>(x);
  dim3 grid((unsigned)M), block(256);
  if (nch <= 256)
    hipLaunchKernelGGL((k_quant_row<FMT, 1>), grid, block, 0, st, xp, si, q, s, (int)K);
  else if (nch <= 512)
    hipLaunchKernelGGL((k_quant_row<FMT, 2>), grid, block, 0, st, xp, si, q, s, (int)K);
  else if (nch <= 1024)
    hipLaunchKernelGGL((k_quant_row<FMT, 4>), grid, block, 0, st, xp, si, q, s, (int)K);
  else if (nch <= 2048)
    hipLaunchKernelGGL((k_quant_row<FMT, 8>), grid, block, 0, st, xp, si, q, s, (int)K);
  else
    hipLaunchKernelGGL((k_quant_row<FMT, 16>), grid, block, 0, st, xp, si, q, s, (int)K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_group(const void* x, bool fp16, int64_t M, int64_t K, int8_t* q, float* s, hipStream_t st) {
  const int64_t G = M * (K >> 7);
  const int64_t blocks = (G + kGroupsPerBlock - 1) / kGroupsPerBlock;
  const uint4* xp = static_cast<const uint4*>(x);
  if (fp16)
    hipLaunchKernelGGL((k_quant_group<true>), dim3((unsigned)blocks), dim3(256), 0, st, xp, q, s, G);
  else
    hipLaunchKernelGGL((k_quant_group<false>), dim3((unsigned)blocks), dim3(256), 0, st, xp, q, s, G);
  return hipGetLastError();
}

hipError_t launch_quant_weight_int4(const void* w, bool fp16, int64_t N, int64_t K, uint8_t* q4, float* s,
                                    hipStream_t st) {
  const int64_t G = N * (K >> 7);
  const int64_t blocks = (G + kGroupsPerBlock - 1) / kGroupsPerBlock;
  const uint4* wp = static_cast<const uint4*>(w);
  int8_t* qp = reinterpret_cast<int8_t*>(q4);
  if (fp16)
    hipLaunchKernelGGL((k_quant_group<true, true>), dim3((unsigned)blocks), dim3(256), 0, st, wp, qp, s, G);
  else
    hipLaunchKernelGGL((k_quant_group<false, true>), dim3((unsigned)blocks), dim3(256), 0, st, wp, qp, s, G);
  return hipGetLastError();
}

hipError_t launch_quant_token(const void* x, bool fp16, int64_t M, int64_t K, int8_t* q, float* s, hipStream_t st) {
  return fp16 ? launch_row<FMT_FP16>(x, nullptr, M, K, q, s, st) : launch_row<FMT_BF16>(x, nullptr, M, K, q, s, st);
}

hipError_t launch_requant_channel(const uint8_t* w, const float* si, int64_t N, int64_t K, int8_t* q, float* s,
                                  hipStream_t st) {
  return launch_row<FMT_FP8>(w, si, N, K, q, s, st);
}

hipError_t launch_quant_weight_block(const void* w, int64_t N, int64_t K, int8_t* q, float* s, hipStream_t st) {
  dim3 grid((unsigned)((K >> 7) * ((N + 127) >> 7)));
  hipLaunchKernelGGL(k_quant_tile_bf16, grid, dim3(256), 0, st, static_cast<const uint4*>(w), q, s, (int)N, (int)K);
  return hipGetLastError();
}

hipError_t launch_requant_block(const uint8_t* w, const float* si, int64_t N, int64_t K, int8_t* q, float* s,
                                uint16_t* wbf, hipStream_t st) {
  const int64_t NS = ((K >> 7) + kStripTiles - 1) / kStripTiles;
  dim3 grid((unsigned)(NS * ((N + 127) >> 7)));
  const uint4* wp = reinterpret_cast<const uint4*>(w);
  if (wbf)
    hipLaunchKernelGGL((k_requant_tile_fp8<true>), grid, dim3(256), 0, st, wp, si, q, s, wbf, (int)N, (int)K);
  else
    hipLaunchKernelGGL((k_requant_tile_fp8<false>), grid, dim3(256), 0, st, wp, si, q, s, wbf, (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace w8
