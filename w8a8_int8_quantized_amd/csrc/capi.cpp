// extern "C" entry points of libw8a8.so (declared in include/w8a8.h).
//
// This layer only validates arguments and dispatches to the launchers; every
// check runs on the host before anything is enqueued, so a failed check
// leaves the stream untouched.  The launchers of the split-K and asymmetric
// paths take the library's per-stream scratch (csrc/workspace.h), which may
// allocate on first use or growth; nothing here or there synchronises.
#include <hip/hip_runtime.h>

#include "../../include/w8a8.h"
#include "launch.h"

namespace {

constexpr int kAbiVersion = 3;
constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxElems = int64_t(1) << 40;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Common shape rule: rows >= 0, 0 <= K <= kMaxK, K % 128 == 0, rows * K < 2^40.
int check_rows_k(int64_t R, int64_t K) {
  if (R < 0 || K < 0 || R > kMaxRows || K > kMaxK || (K & 127) != 0) return W8_ERR_SHAPE;
  if (R > 0 && K > 0 && R > kMaxElems / K) return W8_ERR_SHAPE;
  return W8_OK;
}

int status_of(hipError_t e) {
  if (e == hipSuccess) return W8_OK;
  if (e == hipErrorStreamCaptureUnsupported) {
    (void)hipGetLastError();
    return W8_ERR_CAPTURE;
  }
  return W8_ERR_LAUNCH;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int check_out(int y_dtype, bool allow_i32, w8::OutKind* out) {
  switch (y_dtype) {
    case W8_BF16: *out = w8::OUT_BF16; return W8_OK;
    case W8_FP32: *out = w8::OUT_F32; return W8_OK;
    case W8_I32:
      if (!allow_i32) return W8_ERR_DTYPE;
      *out = w8::OUT_I32;
      return W8_OK;
    default: return W8_ERR_DTYPE;
  }
}

int check_gemm_common(const int8_t* A, const int8_t* W, const void* Y, int64_t M, int64_t N, int64_t K) {
  int rc = check_rows_k(M, K);
  if (rc) return rc;
  rc = check_rows_k(N, K);
  if (rc) return rc;
  if (M > 0 && N > 0 && M > kMaxElems / N) return W8_ERR_SHAPE;
  if (M == 0 || N == 0) return W8_OK;
  if (!A || !W || !Y) return W8_ERR_NULL;
  if (!aligned(A, 16) || !aligned(W, 16) || !aligned(Y, 16)) return W8_ERR_ALIGN;
  return W8_OK;
}

}  // namespace

extern "C" {

int w8_abi_version(void) { return kAbiVersion; }

const char* w8_status_string(int status) {
  switch (status) {
    case W8_OK: return "ok";
    case W8_ERR_NULL: return "null pointer argument";
    case W8_ERR_SHAPE: return "invalid shape (negative size, K not a multiple of 128, or beyond the limits)";
    case W8_ERR_ALIGN: return "misaligned pointer (data 16-byte, scales 4-byte)";
    case W8_ERR_DTYPE: return "unsupported dtype";
    case W8_ERR_LAUNCH: return "kernel launch or workspace allocation failed";
    case W8_ERR_WORKSPACE:
      return "workspace too small (a caller-provided workspace, or the 64 MiB fixed scratch of "
             "gemm_w8a8_channel_noalloc)";
    case W8_ERR_CAPTURE:
      return "the call would allocate its scratch while its stream is being captured "
             "(make one call of the largest shape on the stream before capturing)";
    default: return "unknown status";
  }
}

static int quant_act_common(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q, float* scale, bool group,
                            void* stream) {
  if (x_dtype != W8_BF16 && x_dtype != W8_FP16) return W8_ERR_DTYPE;
  int rc = check_rows_k(M, K);
  if (rc) return rc;
  if (M == 0 || K == 0) return W8_OK;
  if (!x || !q || !scale) return W8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4)) return W8_ERR_ALIGN;
  const bool fp16 = x_dtype == W8_FP16;
  return status_of(group ? w8::launch_quant_group(x, fp16, M, K, q, scale, as_stream(stream))
                         : w8::launch_quant_token(x, fp16, M, K, q, scale, as_stream(stream)));
}

int quant_act_group(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q, float* scale, void* stream) {
  return quant_act_common(x, x_dtype, M, K, q, scale, true, stream);
}

int quant_act_token(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q, float* scale, void* stream) {
  return quant_act_common(x, x_dtype, M, K, q, scale, false, stream);
}

int quant_weight_block(const void* w, int64_t N, int64_t K, int8_t* w_q, float* w_scale, void* stream) {
  int rc = check_rows_k(N, K);
  if (rc) return rc;
  if (N == 0 || K == 0) return W8_OK;
  if (!w || !w_q || !w_scale) return W8_ERR_NULL;
  if (!aligned(w, 16) || !aligned(w_q, 16) || !aligned(w_scale, 4)) return W8_ERR_ALIGN;
  return status_of(w8::launch_quant_weight_block(w, N, K, w_q, w_scale, as_stream(stream)));
}

int requant_fp8_to_int8_block(const uint8_t* w_fp8, const float* scale_inv, int64_t N, int64_t K, int8_t* w_q,
                              float* w_scale, uint16_t* w_bf16_or_null, void* stream) {
  int rc = check_rows_k(N, K);
  if (rc) return rc;
  if (N == 0 || K == 0) return W8_OK;
  if (!w_fp8 || !scale_inv || !w_q || !w_scale) return W8_ERR_NULL;
  if (!aligned(w_fp8, 16) || !aligned(w_q, 16) || !aligned(scale_inv, 4) || !aligned(w_scale, 4) ||
      (w_bf16_or_null && !aligned(w_bf16_or_null, 16)))
    return W8_ERR_ALIGN;
  return status_of(
      w8::launch_requant_block(w_fp8, scale_inv, N, K, w_q, w_scale, w_bf16_or_null, as_stream(stream)));
}

int requant_fp8_to_int8_channel(const uint8_t* w_fp8, const float* scale_inv, int64_t N, int64_t K, int8_t* w_q,
                                float* w_scale, void* stream) {
  int rc = check_rows_k(N, K);
  if (rc) return rc;
  if (N == 0 || K == 0) return W8_OK;
  if (!w_fp8 || !scale_inv || !w_q || !w_scale) return W8_ERR_NULL;
  if (!aligned(w_fp8, 16) || !aligned(w_q, 16) || !aligned(scale_inv, 4) || !aligned(w_scale, 4))
    return W8_ERR_ALIGN;
  return status_of(w8::launch_requant_channel(w_fp8, scale_inv, N, K, w_q, w_scale, as_stream(stream)));
}

int gemm_w8a8_block(const int8_t* A, const float* a_scale, const int8_t* W, const float* w_scale, void* Y,
                    int y_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
  w8::OutKind out;
  int rc = check_out(y_dtype, false, &out);
  if (rc) return rc;
  rc = check_gemm_common(A, W, Y, M, N, K);
  if (rc || M == 0 || N == 0) return rc;
  if (K == 0) return W8_ERR_SHAPE;
  if (!a_scale || !w_scale) return W8_ERR_NULL;
  if (!aligned(a_scale, 4) || !aligned(w_scale, 4)) return W8_ERR_ALIGN;
  return status_of(w8::launch_gemm_block(A, a_scale, W, w_scale, Y, out, M, N, K, as_stream(stream)));
}

int gemm_w8a8_channel(const int8_t* A, const float* a_scale, const int8_t* W, const float* w_scale, void* Y,
                      int y_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
  w8::OutKind out;
  int rc = check_out(y_dtype, true, &out);
  if (rc) return rc;
  rc = check_gemm_common(A, W, Y, M, N, K);
  if (rc || M == 0 || N == 0) return rc;
  if (K == 0 || K > (int64_t(1) << 17)) return W8_ERR_SHAPE;
  if (out != w8::OUT_I32) {
    if (!a_scale || !w_scale) return W8_ERR_NULL;
    if (!aligned(a_scale, 4) || !aligned(w_scale, 4)) return W8_ERR_ALIGN;
  }
  return status_of(w8::launch_gemm_channel(A, a_scale, W, w_scale, Y, out, M, N, K, as_stream(stream)));
}

int gemm_w8a8_channel_noalloc(const int8_t* A, const float* a_scale, const int8_t* W, const float* w_scale,
                              void* Y, int y_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
  w8::OutKind out;
  int rc = check_out(y_dtype, true, &out);
  if (rc) return rc;
  rc = check_gemm_common(A, W, Y, M, N, K);
  if (rc || M == 0 || N == 0) return rc;
  if (K == 0 || K > (int64_t(1) << 17)) return W8_ERR_SHAPE;
  if (out != w8::OUT_I32) {
    if (!a_scale || !w_scale) return W8_ERR_NULL;
    if (!aligned(a_scale, 4) || !aligned(w_scale, 4)) return W8_ERR_ALIGN;
  }
  bool too_big = false;
  const hipError_t e =
      w8::launch_gemm_channel_noalloc(A, a_scale, W, w_scale, Y, out, M, N, K, as_stream(stream), &too_big);
  if (too_big) return W8_ERR_WORKSPACE;
  return status_of(e);
}

int gemm_w8a8_block_quant(const int8_t* A, const float* a_scale, const int8_t* W, const float* w_scale, int8_t* q,
                          float* q_scale, int64_t M, int64_t N, int64_t K, void* stream) {
  int rc = check_gemm_common(A, W, q, M, N, K);
  if (rc || M == 0 || N == 0) return rc;
  if (K == 0 || (N & 127) != 0) return W8_ERR_SHAPE;
  if (!a_scale || !w_scale || !q_scale) return W8_ERR_NULL;
  if (!aligned(a_scale, 4) || !aligned(w_scale, 4) || !aligned(q_scale, 4)) return W8_ERR_ALIGN;
  return status_of(w8::launch_gemm_block_q8(A, a_scale, W, w_scale, q, q_scale, M, N, K, as_stream(stream)));
}

int gemm_w8a8_block_grouped_quant(const int8_t* A, const float* a_scale, const int8_t* W, const float* w_scale,
                                  const int32_t* expert_offsets, int8_t* q, float* q_scale, int64_t E, int64_t P,
                                  int64_t N, int64_t K, void* stream) {
  if (E < 0 || E > 4096) return W8_ERR_SHAPE;
  int rc = check_gemm_common(A, W, q, P, N, K);
  if (rc || P == 0 || N == 0 || E == 0) return rc;
  if (K == 0 || (N & 127) != 0) return W8_ERR_SHAPE;
  if (N * K > kMaxElems / E) return W8_ERR_SHAPE;
  if (!a_scale || !w_scale || !expert_offsets || !q_scale) return W8_ERR_NULL;
  if (!aligned(a_scale, 4) || !aligned(w_scale, 4) || !aligned(expert_offsets, 4) || !aligned(q_scale, 4))
    return W8_ERR_ALIGN;
  return status_of(w8::launch_gemm_block_grouped_q8(A, a_scale, W, w_scale, expert_offsets, q, q_scale, E, P, N, K,
                                                    as_stream(stream)));
}

int gemm_w8a8_block_partials(const int8_t* A, const int8_t* W, int32_t* P, int64_t M, int64_t N, int64_t K,
                             void* stream) {
  int rc = check_gemm_common(A, W, P, M, N, K);
  if (rc || M == 0 || N == 0 || K == 0) return rc;
  return status_of(w8::launch_gemm_block_partials(A, W, P, M, N, K, as_stream(stream)));
}

int gemm_w8a16_group(const uint16_t* x, const int8_t* W, const float* w_scale, uint16_t* Y, int64_t M, int64_t N,
                     int64_t K, void* stream) {
  int rc = check_rows_k(M, K);
  if (rc) return rc;
  rc = check_rows_k(N, K);
  if (rc) return rc;
  if (M > 0 && N > 0 && M > kMaxElems / N) return W8_ERR_SHAPE;
  if (M == 0 || N == 0) return W8_OK;
  if (K == 0) return W8_ERR_SHAPE;
  if (!x || !W || !w_scale || !Y) return W8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(W, 16) || !aligned(Y, 16) || !aligned(w_scale, 4)) return W8_ERR_ALIGN;
  return status_of(w8::launch_gemm_w8a16(x, W, w_scale, Y, M, N, K, as_stream(stream)));
}

int quant_weight_int4_group(const void* w, int w_dtype, int64_t N, int64_t K, uint8_t* w4, float* w_scale,
                            void* stream) {
  if (w_dtype != W8_BF16 && w_dtype != W8_FP16) return W8_ERR_DTYPE;
  int rc = check_rows_k(N, K);
  if (rc) return rc;
  if (N == 0 || K == 0) return W8_OK;
  if (!w || !w4 || !w_scale) return W8_ERR_NULL;
  if (!aligned(w, 16) || !aligned(w4, 16) || !aligned(w_scale, 4)) return W8_ERR_ALIGN;
  return status_of(w8::launch_quant_weight_int4(w, w_dtype == W8_FP16, N, K, w4, w_scale, as_stream(stream)));
}

int gemm_w4a16_group(const uint16_t* x, const uint8_t* W4, const float* w_scale, uint16_t* Y, int64_t M, int64_t N,
                     int64_t K, void* stream) {
  int rc = check_rows_k(M, K);
  if (rc) return rc;
  rc = check_rows_k(N, K);
  if (rc) return rc;
  if (M > 0 && N > 0 && M > kMaxElems / N) return W8_ERR_SHAPE;
  if (M == 0 || N == 0) return W8_OK;
  if (K == 0) return W8_ERR_SHAPE;
  if (!x || !W4 || !w_scale || !Y) return W8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(W4, 16) || !aligned(Y, 16) || !aligned(w_scale, 4)) return W8_ERR_ALIGN;
  return status_of(w8::launch_gemm_w4a16(x, W4, w_scale, Y, M, N, K, as_stream(stream)));
}

int gemm_w8a8_block_grouped(const int8_t* A, const float* a_scale, const int8_t* W, const float* w_scale,
                            const int32_t* expert_offsets, void* Y, int y_dtype, int64_t E, int64_t P, int64_t N,
                            int64_t K, void* stream) {
  w8::OutKind out;
  int rc = check_out(y_dtype, false, &out);
  if (rc) return rc;
  if (E < 0 || E > 4096) return W8_ERR_SHAPE;
  rc = check_gemm_common(A, W, Y, P, N, K);
  if (rc || P == 0 || N == 0 || E == 0) return rc;
  if (K == 0) return W8_ERR_SHAPE;
  if (E > 0 && N * K > kMaxElems / E) return W8_ERR_SHAPE;
  if (!a_scale || !w_scale || !expert_offsets) return W8_ERR_NULL;
  if (!aligned(a_scale, 4) || !aligned(w_scale, 4) || !aligned(expert_offsets, 4)) return W8_ERR_ALIGN;
  return status_of(w8::launch_gemm_block_grouped(A, a_scale, W, w_scale, expert_offsets, Y, out, E, P, N, K,
                                                 as_stream(stream)));
}

int64_t linear_workspace_bytes(int scheme, int64_t M, int64_t K) {
  if (scheme != W8_SCHEME_BLOCK && scheme != W8_SCHEME_CHANNEL) return W8_ERR_DTYPE;
  int rc = check_rows_k(M, K);
  if (rc) return rc;
  const int64_t codes = (M * K + 255) / 256 * 256;
  return codes + 4 * (scheme == W8_SCHEME_BLOCK ? M * (K / 128) : M);
}

static int linear_common(bool block, const void* x, int x_dtype, const int8_t* W, const float* w_scale, void* Y,
                         int y_dtype, int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                         void* stream) {
  if (x_dtype != W8_BF16 && x_dtype != W8_FP16) return W8_ERR_DTYPE;
  w8::OutKind out;
  int rc = check_out(y_dtype, false, &out);
  if (rc) return rc;
  // x takes the place of A in the shape, null and 16-byte alignment checks
  rc = check_gemm_common(static_cast<const int8_t*>(x), W, Y, M, N, K);
  if (rc || M == 0 || N == 0) return rc;
  if (K == 0 || (!block && K > (int64_t(1) << 17))) return W8_ERR_SHAPE;
  if (!w_scale || !workspace) return W8_ERR_NULL;
  if (!aligned(w_scale, 4) || !aligned(workspace, 256)) return W8_ERR_ALIGN;
  const int64_t need = linear_workspace_bytes(block ? W8_SCHEME_BLOCK : W8_SCHEME_CHANNEL, M, K);
  if (workspace_bytes < need) return W8_ERR_WORKSPACE;
  int8_t* q = static_cast<int8_t*>(workspace);
  float* s = reinterpret_cast<float*>(static_cast<char*>(workspace) + (M * K + 255) / 256 * 256);
  const hipStream_t st = as_stream(stream);
  const bool fp16 = x_dtype == W8_FP16;
  const hipError_t e =
      block ? w8::launch_quant_group(x, fp16, M, K, q, s, st) : w8::launch_quant_token(x, fp16, M, K, q, s, st);
  if (e != hipSuccess) return W8_ERR_LAUNCH;
  return status_of(block ? w8::launch_gemm_block(q, s, W, w_scale, Y, out, M, N, K, st)
                         : w8::launch_gemm_channel(q, s, W, w_scale, Y, out, M, N, K, st));
}

int linear_w8a8_block(const void* x, int x_dtype, const int8_t* W, const float* w_scale, void* Y, int y_dtype,
                      int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, void* stream) {
  return linear_common(true, x, x_dtype, W, w_scale, Y, y_dtype, M, N, K, workspace, workspace_bytes, stream);
}

int linear_w8a8_channel(const void* x, int x_dtype, const int8_t* W, const float* w_scale, void* Y, int y_dtype,
                        int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes, void* stream) {
  return linear_common(false, x, x_dtype, W, w_scale, Y, y_dtype, M, N, K, workspace, workspace_bytes, stream);
}

int quant_act_asym(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q_shifted, float* params,
                   void* stream) {
  if (x_dtype != W8_BF16 && x_dtype != W8_FP16) return W8_ERR_DTYPE;
  int rc = check_rows_k(M, K);
  if (rc) return rc;
  if (M == 0 || K == 0) return W8_OK;
  if (!x || !q_shifted || !params) return W8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q_shifted, 16) || !aligned(params, 4)) return W8_ERR_ALIGN;
  return status_of(w8::launch_quant_asym(x, x_dtype == W8_FP16, M, K, q_shifted, params, as_stream(stream)));
}

int weight_row_sums(const int8_t* W, int64_t N, int64_t K, int32_t* w_sum, void* stream) {
  int rc = check_rows_k(N, K);
  if (rc) return rc;
  if (K > (int64_t(1) << 16)) return W8_ERR_SHAPE;
  if (N == 0) return W8_OK;
  if (K == 0) return W8_ERR_SHAPE;
  if (!W || !w_sum) return W8_ERR_NULL;
  if (!aligned(W, 16) || !aligned(w_sum, 4)) return W8_ERR_ALIGN;
  return status_of(w8::launch_weight_row_sums(W, N, K, w_sum, as_stream(stream)));
}

int gemm_w8a8_asym(const int8_t* A_shifted, const float* a_params, const int8_t* W, const float* w_scale,
                   const int32_t* w_sum, void* Y, int y_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
  w8::OutKind out;
  int rc = check_out(y_dtype, false, &out);
  if (rc) return rc;
  rc = check_gemm_common(A_shifted, W, Y, M, N, K);
  if (rc || M == 0 || N == 0) return rc;
  if (K == 0 || K > (int64_t(1) << 16)) return W8_ERR_SHAPE;
  if (!a_params || !w_scale || !w_sum) return W8_ERR_NULL;
  if (!aligned(a_params, 4) || !aligned(w_scale, 4) || !aligned(w_sum, 4)) return W8_ERR_ALIGN;
  return status_of(
      w8::launch_gemm_asym(A_shifted, a_params, W, w_scale, w_sum, Y, out, M, N, K, as_stream(stream)));
}

}  // extern "C"
