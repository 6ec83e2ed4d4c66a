// Internal launchers of libw8a8.so (host side).  Each enqueues its kernels on
// the given stream and returns the launch status; argument checks are done by
// the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8 {

enum OutKind { OUT_BF16 = 0, OUT_F32 = 1, OUT_I32 = 2 };

hipError_t launch_quant_group(const void* x, bool fp16, int64_t M, int64_t K, int8_t* q, float* s, hipStream_t st);
hipError_t launch_quant_token(const void* x, bool fp16, int64_t M, int64_t K, int8_t* q, float* s, hipStream_t st);
hipError_t launch_quant_weight_block(const void* w, int64_t N, int64_t K, int8_t* q, float* s, hipStream_t st);
hipError_t launch_requant_block(const uint8_t* w, const float* si, int64_t N, int64_t K, int8_t* q, float* s,
                                uint16_t* wbf, hipStream_t st);
hipError_t launch_requant_channel(const uint8_t* w, const float* si, int64_t N, int64_t K, int8_t* q, float* s,
                                  hipStream_t st);

hipError_t launch_gemm_channel(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                               OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_gemm_block(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                             OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_gemm_block_partials(const int8_t* A, const int8_t* W, int32_t* P, int64_t M, int64_t N, int64_t K,
                                      hipStream_t st);
hipError_t launch_gemm_block_grouped(const int8_t* A, const float* sa, const int8_t* W, const float* sw,
                                     const int32_t* offsets, void* Y, OutKind out, int64_t E, int64_t P, int64_t N,
                                     int64_t K, hipStream_t st);
// Asymmetric per-tensor UINT8 activations (codes stored as q - 128) with
// symmetric per-channel INT8 weights.
hipError_t launch_quant_asym(const void* x, bool fp16, int64_t M, int64_t K, int8_t* q, float* params,
                             hipStream_t st);
// The unsplit channel-wise tile grid serves (M, N, K) (no decode kernel, no
// K split); then the asymmetric epilogue runs inside the tile kernel.
bool channel_tiles_unsplit(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_channel_asym_tiles(const int8_t* A, const float* prm, const int8_t* W, const float* sw,
                                          const int32_t* wsum, void* Y, OutKind out, int64_t M, int64_t N,
                                          int64_t K, hipStream_t st);
hipError_t launch_weight_row_sums(const int8_t* W, int64_t N, int64_t K, int32_t* ws, hipStream_t st);
hipError_t launch_gemm_asym(const int8_t* A, const float* params, const int8_t* W, const float* sw,
                            const int32_t* wsum, void* Y, OutKind out, int64_t M, int64_t N, int64_t K,
                            hipStream_t st);
hipError_t launch_gemm_w8a16(const uint16_t* x, const int8_t* W, const float* s, uint16_t* Y, int64_t M, int64_t N,
                             int64_t K, hipStream_t st);

// Split-K workspace: at least `bytes` of device memory kept for `st` on the
// current device (grown on demand; the growth synchronises `st`).
hipError_t split_workspace(hipStream_t st, size_t bytes, void** out);
// The same for workspace `slot` (0: split-K partials, 1: the asymmetric path).
hipError_t stream_workspace(hipStream_t st, int slot, size_t bytes, void** out);
// Number of K slices (1..16) for a grid of `tiles` workgroups over KB K
// blocks, from a model with t_kb_us microseconds per tile and K block.
int pick_k_slices(int64_t tiles, int64_t KB, int64_t M, int64_t N, double t_kb_us);

// Small-M (weight-streaming) variants, used by the dispatchers above for the
// shapes decode_path_takes accepts: every M <= 64, and channel-wise M <= 128
// where the grid of the workgroup-shared kernel splits evenly over the CUs.
bool decode_path_takes(int64_t M, int64_t N, bool channel);
hipError_t launch_gemm_block_decode(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                                    OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_gemm_channel_decode(const int8_t* A, const float* sa, const int8_t* W, const float* sw, void* Y,
                                      OutKind out, int64_t M, int64_t N, int64_t K, hipStream_t st);

}  // namespace w8
