/*
 * w8a8.h - C ABI of libw8a8.so: W8A8 INT8 linear layers (block-wise and
 * channel-wise schemes) on AMD Instinct MI355X (gfx950).
 *
 * The method is the one described on the page "DeepSeek R1 INT8 quantisation
 * in SGLang" (Meituan team article), section 2.3 "Quantisation method
 * design", with the symmetric INT8 quantiser of the page "FP8 vs INT8
 * quantisation for DeepSeek", section 3.2.1 (int8 branch):
 *
 *   scale = max(amax, 1e-10f) / 127           fp32 IEEE division
 *   q     = clamp(round_half_even(x / scale), -127, 127)   x / scale in fp32
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  Calls
 *     are thread-safe.  The only state the library keeps is its own scratch
 *     (described at gemm_w8a8_block): a split-K workspace per (device,
 *     stream) for gemm_w8a8_block, gemm_w8a8_channel, gemm_w8a16_group,
 *     gemm_w4a16_group and the linear_* calls, one for quant_act_asym and gemm_w8a8_asym, and the
 *     fixed array of gemm_w8a8_channel_noalloc; every other entry point
 *     allocates nothing.
 *   - Every call enqueues its kernels on `stream` (a hipStream_t passed as
 *     void*; NULL is the default stream) and returns without synchronising.
 *     Results are visible once the stream reaches that point.
 *   - Layouts are row-major and contiguous.  Activations are A[M][K],
 *     weights W[N][K] (nn.Linear layout), outputs Y[M][N] = A . W^T.
 *   - K must be a multiple of 128 (the K block / group size); KB = K / 128,
 *     NB = ceil(N / 128).  M == 0 (or N == 0) is a valid no-op.
 *   - Data pointers (int8, bf16, fp16, fp8, outputs) must be 16-byte aligned;
 *     scale pointers 4-byte aligned.  Outputs must not alias inputs.
 *   - int8 codes are always in [-127, 127] (INT4 codes in [-7, 7]); scales
 *     are fp32.
 *   - bf16 and fp16 values are passed as their 16-bit patterns.
 *   - Inputs are finite.  NaN or infinite inputs (and the FP8 NaN codes
 *     0x7F / 0xFF) give unspecified results but never out-of-bounds access.
 *   - Results are deterministic: no floating-point atomics; rerunning a call
 *     on the same inputs gives the same bits.
 *   - Return 0 (W8_OK) on success, otherwise a negative w8_status; nothing is
 *     enqueued when an argument check fails.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum w8_status {
  W8_OK = 0,
  W8_ERR_NULL = -1,   /* a required pointer is NULL */
  W8_ERR_SHAPE = -2,  /* negative size, K % 128 != 0, or a size beyond the limits below */
  W8_ERR_ALIGN = -3,  /* a pointer is not aligned as required */
  W8_ERR_DTYPE = -4,  /* unsupported dtype code */
  W8_ERR_LAUNCH = -5, /* the HIP runtime rejected a kernel launch or a workspace allocation */
  W8_ERR_WORKSPACE = -6, /* a workspace is smaller than required (a caller-provided one, or the
                            fixed scratch of gemm_w8a8_channel_noalloc) */
  W8_ERR_CAPTURE = -7  /* the call would allocate its scratch while its stream is being captured
                          into a graph; nothing was enqueued */
};

enum w8_dtype { W8_BF16 = 0, W8_FP16 = 1, W8_FP32 = 2, W8_I32 = 3 };

/* Size limits: M, N <= 2^31 - 1 and K <= 2^20, so that every index fits the
   kernels' 32-bit row arithmetic; M * K and N * K < 2^40. */

/* Version of this ABI (bumped on any signature change). */
int w8_abi_version(void);

/* Human-readable text of a w8_status code (static storage). */
const char* w8_status_string(int status);

/*
 * Online per-token-group activation quantisation (block-wise scheme; page 1
 * section 2.3: "each token's vector is split into groups, quantised group by
 * group").  Group = 1 x 128 along K, aligned with the 128-wide weight blocks.
 *   x      [M][K]  bf16 (x_dtype = W8_BF16) or fp16 (W8_FP16) bit patterns
 *   q      [M][K]  int8 out
 *   scale  [M][KB] fp32 out, scale[m][kb] for elements k in [128 kb, 128 kb + 128)
 * With x = W[N][K] in fp16 this is also the group-wise weight quantiser of
 * the W8A16 variant (page 5, symmetric group-wise INT8 weights).
 */
int quant_act_group(const void* x, int x_dtype, int64_t M, int64_t K,
                    int8_t* q, float* scale, void* stream);

/*
 * Online per-token activation quantisation (channel-wise scheme; page 1
 * section 2.3: activations quantised online token by token).  One scale per
 * row over the whole K.  K <= 2^20.
 *   x [M][K] bf16/fp16 -> q [M][K] int8, scale [M] fp32.
 * With x = W[N][K] this is the channel-wise weight quantiser (one scale per
 * output channel: "each column of the weight is one group" in X.W notation).
 */
int quant_act_token(const void* x, int x_dtype, int64_t M, int64_t K,
                    int8_t* q, float* scale, void* stream);

/*
 * Block-wise weight quantisation of bf16 weights in 128 x 128 tiles (page 1
 * section 2.3, block-wise paragraph).  The last tile row may hold fewer than
 * 128 rows; its amax covers the rows that exist.
 *   w [N][K] bf16 -> w_q [N][K] int8, w_scale [NB][KB] fp32.
 */
int quant_weight_block(const void* w, int64_t N, int64_t K,
                       int8_t* w_q, float* w_scale, void* stream);

/*
 * Offline weight conversion of page 1 section 2.3: the FP8 checkpoint is
 * dequantised to BF16, then requantised to INT8 in 128 x 128 tiles.
 *   w_fp8     [N][K]  OCP FP8-E4M3FN codes (bias 7, max 448, S.1111.111 NaN)
 *   scale_inv [NB][KB] fp32: dequantised value = fp8 value * scale_inv
 *   w_q [N][K] int8, w_scale [NB][KB] fp32 out
 *   w_bf16_or_null [N][K] bf16 out (the intermediate) or NULL to skip it
 * BF16 step: bf16_round_nearest_even(fp32(fp8 * scale_inv[n/128][k/128])).
 */
int requant_fp8_to_int8_block(const uint8_t* w_fp8, const float* scale_inv,
                              int64_t N, int64_t K, int8_t* w_q, float* w_scale,
                              uint16_t* w_bf16_or_null, void* stream);

/*
 * Channel-wise counterpart of the offline conversion (page 1 section 2.3,
 * channel-wise paragraph): FP8 -> BF16 as above, then one scale per output
 * channel (row of W).  w_scale [N] fp32.  K <= 2^20.
 */
int requant_fp8_to_int8_channel(const uint8_t* w_fp8, const float* scale_inv,
                                int64_t N, int64_t K, int8_t* w_q, float* w_scale,
                                void* stream);

/*
 * Block-wise W8A8 GEMM (page 1 section 2.3, block-wise paragraph and its
 * Figure 3): int32 partial sums per 128-wide K block, dequantised in fp32
 * inside the K loop:
 *   Y[m][n] = sum_kb a_scale[m][kb] * w_scale[n/128][kb] * P[kb][m][n],
 *   P[kb][m][n] = sum_{k in block kb} A[m][k] * W[n][k]   (exact int32).
 *   A [M][K] int8, a_scale [M][KB], W [N][K] int8, w_scale [NB][KB]
 *   Y [M][N] bf16 (y_dtype W8_BF16) or fp32 (W8_FP32).
 * The bf16 output is the round-to-nearest-even of the fp32 result.
 * Split-K workspace (this call and gemm_w8a8_channel): when the output tile
 * grid is too small to occupy the GPU (few tiles of 256 x 256 for M > 128,
 * or 128 x 256 for M <= 128 block-wise), K is split into S slices whose
 * partial tiles (S x M x N x 4 bytes) go to a device buffer that the library
 * keeps per (device, stream).  It is allocated on the first such call on a
 * stream; a later call that needs more gets a new buffer (size rounded up to
 * a power of two) and the old one is retired, never freed while the process
 * runs, since kernels enqueued earlier (or a graph captured with its
 * address) may still use it.  Nothing synchronises.  A call holds the
 * library's lock from taking its buffer until its kernels are enqueued, so
 * host threads sharing a stream enqueue their sequences one after the other.
 * The slices are summed in slice order, so results stay deterministic.
 * While the stream is being captured into a graph the library allocates
 * nothing: a call whose buffer would have to be allocated or grown returns
 * W8_ERR_CAPTURE with nothing enqueued (make one call of the largest shape
 * on the stream before capturing; the captured graph then uses that
 * stream's buffer, and replaying it while other calls run on that stream
 * races with them).  An allocation failure returns W8_ERR_LAUNCH with
 * nothing enqueued.
 */
int gemm_w8a8_block(const int8_t* A, const float* a_scale,
                    const int8_t* W, const float* w_scale,
                    void* Y, int y_dtype, int64_t M, int64_t N, int64_t K,
                    void* stream);

/*
 * Channel-wise W8A8 GEMM (page 1 section 2.3, channel-wise paragraph): one
 * dequantisation after the INT8 matmul:
 *   ACC[m][n] = sum_k A[m][k] * W[n][k]   (exact int32; K <= 2^17 keeps it
 *                                          inside int32 for codes in +-127)
 *   Y[m][n]   = fp32(fp32(ACC) * fp32(a_scale[m] * w_scale[n]))
 *   A [M][K] int8, a_scale [M], W [N][K] int8, w_scale [N]
 *   Y [M][N] bf16, fp32, or int32 (y_dtype W8_I32: raw ACC, scales unused and
 *   may be NULL).
 * Uses the split-K workspace described at gemm_w8a8_block for small tile
 * grids; the int32 slice sums are exact, so the result is the same as
 * unsplit.
 */
int gemm_w8a8_channel(const int8_t* A, const float* a_scale,
                      const int8_t* W, const float* w_scale,
                      void* Y, int y_dtype, int64_t M, int64_t N, int64_t K,
                      void* stream);

/*
 * gemm_w8a8_channel for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results (bit-identical) as
 * gemm_w8a8_channel; where that call would take its split-K workspace, this
 * one uses a fixed scratch array of 64 MiB compiled into the library (each
 * GPU the library runs on holds its own copy until the process ends).  It
 * calls no allocating routine.  A shape whose split-K partial tiles
 * (S x M x N x 4 bytes) exceed 64 MiB returns W8_ERR_WORKSPACE with nothing
 * enqueued.  Every call of this entry point on one GPU shares that GPU's
 * array: two calls that overlap in time on one GPU (on different streams,
 * or replayed graphs) race and give wrong results; calls on one stream are
 * ordered and safe.
 */
int gemm_w8a8_channel_noalloc(const int8_t* A, const float* a_scale,
                              const int8_t* W, const float* w_scale,
                              void* Y, int y_dtype, int64_t M, int64_t N,
                              int64_t K, void* stream);

/*
 * The block-wise GEMM with the quantiser of the next block-wise layer fused
 * into its epilogue (page 1 section 2.3: activations are quantised online,
 * per token-group, before every INT8 matmul; here the group quantisation of
 * this GEMM's output runs where the output is produced instead of in a
 * separate pass over it).  The result is exactly gemm_w8a8_block with bf16
 * output followed by quant_act_group on that output:
 *   y[m][n]       = bf16 of gemm_w8a8_block's fp32 value
 *   q_scale[m][g] = fp32(max(amax over y[m][128 g .. 128 g + 127], 1e-10) / 127)
 *   q[m][n]       = clamp(round_half_even(fp32(y[m][n] / q_scale[m][n/128])), -127, 127)
 *   A, a_scale, W, w_scale as gemm_w8a8_block; N % 128 == 0 (W8_ERR_SHAPE
 *   otherwise); q [M][N] int8 out, q_scale [M][N/128] fp32 out.
 * The quantisation runs in the tile kernel's epilogue, or, for small tile
 * grids and where gemm_w8a8_block takes its 128 x 192 tiles (whose fp32
 * sums add the odd K blocks' sum to the even ones'), in the pass that sums
 * the fp32 K slices (one slice or more, in the split-K workspace as for
 * gemm_w8a8_block, S x M x N x 4 bytes).  For decode-sized M (the weight-streaming kernels of
 * gemm_w8a8_block, whose waves own 16-column slices of a group) the bf16
 * output goes through the same per-stream scratch (M x N x 2 bytes) to the
 * group quantiser: nothing is saved there, but the result is the same.
 */
int gemm_w8a8_block_quant(const int8_t* A, const float* a_scale,
                          const int8_t* W, const float* w_scale,
                          int8_t* q, float* q_scale,
                          int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The int32 block partial sums of the block-wise GEMM, for bit-exact checks:
 *   P [KB][M][N] int32, P[kb][m][n] as defined for gemm_w8a8_block.
 */
int gemm_w8a8_block_partials(const int8_t* A, const int8_t* W, int32_t* P,
                             int64_t M, int64_t N, int64_t K, void* stream);

/*
 * W8A16 group-wise GEMM (page 5, "DeepSeek-R1-0528-Qwen3-8B Int8 W8A16"
 * release note: symmetric group-wise INT8 weights, fp16 activations), groups
 * of 128 along K:
 *   Y[m][n] = sum_g w_scale[n][g] * sum_{k in group g} x[m][k] * W[n][k]
 *   x [M][K] fp16, W [N][K] int8, w_scale [N][KB] fp32, Y [M][N] fp16.
 * Each x * W product is exact in fp32; sums are fp32.
 * For M > 16 with few output columns per CU, K is split into S slices whose
 * fp32 partials (S x min(M, 64) x N x 4 bytes) go to the split-K workspace
 * described at gemm_w8a8_block and are summed in slice order: the result is
 * deterministic, with the fp32 rounding of that order.
 */
int gemm_w8a16_group(const uint16_t* x, const int8_t* W, const float* w_scale,
                     uint16_t* Y, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * INT4 group-wise weight quantisation.  Page 3 ("DeepSeek-R1-Distill-Llama-8B
 * quantisation practice", section 3.3) reports INT4 against INT8 by
 * measurement only; the scheme here is the group-wise weight scheme of the
 * W8A16 variant (page 5) with a 4-bit range: per row of W and group of 128
 * along K, s = fp32(max(amax, 1e-10) / 7) and q = clamp(rne(fp32(w / s)),
 * -7, 7) (-8 unused).  Codes are stored two per byte in offset binary:
 * byte j of a row holds q[2j] + 8 in its low nibble and q[2j+1] + 8 in its
 * high nibble.
 *   w       [N][K]   bf16 (w_dtype = W8_BF16) or fp16 (W8_FP16)
 *   w4      [N][K/2] uint8 out (16-byte aligned)
 *   w_scale [N][KB]  fp32 out
 */
int quant_weight_int4_group(const void* w, int w_dtype, int64_t N, int64_t K,
                            uint8_t* w4, float* w_scale, void* stream);

/*
 * W4A16 group-wise GEMM: gemm_w8a16_group's formula, with every code read
 * from the INT4 layout of quant_weight_int4_group (nibble value minus 8):
 *   Y[m][n] = sum_g w_scale[n][g] * sum_{k in group g} x[m][k] * q[n][k]
 *   x [M][K] fp16, W4 [N][K/2] uint8, w_scale [N][KB] fp32, Y [M][N] fp16.
 * Products are exact in fp32 and sums fp32; the kernels, the K split and its
 * workspace are those of gemm_w8a16_group, so the same rules apply.
 */
int gemm_w4a16_group(const uint16_t* x, const uint8_t* W4, const float* w_scale,
                     uint16_t* Y, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * Grouped block-wise W8A8 GEMM for mixture-of-experts layers (DeepSeek is an
 * MoE model, page 4 section 1.2).  Rows expert_offsets[e] .. expert_offsets[e+1]-1
 * of the expert-sorted activations are multiplied by expert e's weights with
 * the block-wise formula of gemm_w8a8_block.
 *   A [P][K] int8, a_scale [P][KB], W [E][N][K] int8, w_scale [E][NB][KB]
 *   expert_offsets [E+1] int32 DEVICE array, non-decreasing, offsets[0] = 0,
 *   offsets[E] <= P (rows past offsets[E] are left untouched).
 *   Y [P][N] bf16 or fp32.  E <= 4096.
 * The offsets are read on the device only; offsets that break the contract
 * give unspecified output rows but no out-of-bounds access.
 */
int gemm_w8a8_block_grouped(const int8_t* A, const float* a_scale,
                            const int8_t* W, const float* w_scale,
                            const int32_t* expert_offsets, void* Y, int y_dtype,
                            int64_t E, int64_t P, int64_t N, int64_t K,
                            void* stream);

/*
 * gemm_w8a8_block_grouped with the next layer's group quantisation fused
 * into its epilogue, as gemm_w8a8_block_quant: q [P][N] int8 and
 * q_scale [P][N/128] fp32 out (rows in the same expert-sorted order),
 * N % 128 == 0.
 */
int gemm_w8a8_block_grouped_quant(const int8_t* A, const float* a_scale,
                                  const int8_t* W, const float* w_scale,
                                  const int32_t* expert_offsets,
                                  int8_t* q, float* q_scale,
                                  int64_t E, int64_t P, int64_t N, int64_t K,
                                  void* stream);

/*
 * One-call linear layers (page 1 section 2.3: activations are quantised
 * online, per token group for the block-wise scheme and per token for the
 * channel-wise one, then multiplied by the offline-quantised weights):
 *   linear_w8a8_block   = quant_act_group(x) then gemm_w8a8_block
 *   linear_w8a8_channel = quant_act_token(x) then gemm_w8a8_channel
 * on `stream`, with the same kernels, so Y is bit-identical to the two calls
 * made separately.
 *   x [M][K] bf16 (x_dtype W8_BF16) or fp16 (W8_FP16); W, w_scale as for the
 *   GEMM; Y [M][N] bf16 or fp32 (y_dtype).
 *   workspace: caller-owned device memory of at least
 *   linear_workspace_bytes(scheme, M, K) bytes (workspace_bytes says how
 *   many it holds; fewer gives W8_ERR_WORKSPACE), 256-byte aligned.  It takes
 *   the int8 codes of x ([M][K] at offset 0) and their fp32 scales (at offset
 *   M*K rounded up to 256: [M][KB] for the block-wise scheme, [M] for the
 *   channel-wise one); it must not be used by other work until the stream
 *   has passed this call, and must not overlap x, W, w_scale or Y.  The
 *   GEMM may use the split-K workspace described at gemm_w8a8_block.
 *   Channel-wise: K <= 2^17, as for gemm_w8a8_channel.
 * Argument errors return with nothing enqueued; W8_ERR_LAUNCH may leave the
 * quantisation (which writes only the workspace) enqueued.
 */
enum w8_scheme { W8_SCHEME_BLOCK = 0, W8_SCHEME_CHANNEL = 1 };

/* Workspace bytes for linear_w8a8_block (scheme W8_SCHEME_BLOCK) or
   linear_w8a8_channel (W8_SCHEME_CHANNEL) over M x K activations; a negative
   w8_status for an unknown scheme or a shape the linear calls reject. */
int64_t linear_workspace_bytes(int scheme, int64_t M, int64_t K);

int linear_w8a8_block(const void* x, int x_dtype, const int8_t* W,
                      const float* w_scale, void* Y, int y_dtype,
                      int64_t M, int64_t N, int64_t K, void* workspace,
                      int64_t workspace_bytes, void* stream);

int linear_w8a8_channel(const void* x, int x_dtype, const int8_t* W,
                        const float* w_scale, void* Y, int y_dtype,
                        int64_t M, int64_t N, int64_t K, void* workspace,
                        int64_t workspace_bytes, void* stream);

/*
 * Asymmetric per-tensor activation quantisation, an alternative beside the
 * symmetric scheme above (page 2, Meituan INT8 DeepSeek R1 practice guide,
 * part two, item 1, dynamic range-aware quantisation).  Over the whole
 * M x K tensor, in fp32 IEEE operations:
 *   mn, mx = min(x), max(x)
 *   s = max(mx - mn, 1e-10) / 255,  z = -mn / s   (z is not rounded)
 *   q = clamp(round_half_even((x - mn) / s), 0, 255)
 *   x [M][K] bf16 or fp16 (x_dtype); q_shifted [M][K] int8 out, holding
 *   q - 128 (the byte q ^ 0x80), which the int8 GEMM takes directly;
 *   params [2] fp32 DEVICE out: {s, z}.
 * Two kernel launches; their per-workgroup partial ranges (at most 8 KB) go
 * to a library workspace per (device, stream) like the split-K one (slot of
 * its own).  M * K == 0 is a no-op (params untouched).
 */
int quant_act_asym(const void* x, int x_dtype, int64_t M, int64_t K,
                   int8_t* q_shifted, float* params, void* stream);

/* WS[n] = sum_k W[n][k] (exact int32) of int8 weights W [N][K], for
   gemm_w8a8_asym.  0 < K <= 2^16 (N == 0 is a no-op). */
int weight_row_sums(const int8_t* W, int64_t N, int64_t K, int32_t* w_sum,
                    void* stream);

/*
 * GEMM of asymmetric activations (quant_act_asym) with symmetric
 * per-channel int8 weights (quant_act_token applied to W, page 1 section
 * 2.3 channel-wise scheme):
 *   ACC[m][n] = sum_k q[m][k] W[n][k]   (exact; q = stored code + 128)
 *   Y[m][n]   = fp32(fp32(s * w_scale[n]) * fp32(fp32(ACC) - fp32(z * fp32(w_sum[n]))))
 *   A_shifted [M][K] int8, a_params [2] {s, z} DEVICE, W [N][K] int8,
 *   w_scale [N], w_sum [N] int32 (weight_row_sums), Y [M][N] bf16 or fp32.
 * K <= 2^16 (ACC stays inside int32).  The stored codes' int32 products
 * (the channel-wise GEMM) go to a library workspace of M x N x 4 bytes per
 * (device, stream), grown on demand like the split-K one, then one epilogue
 * launch forms Y.
 */
int gemm_w8a8_asym(const int8_t* A_shifted, const float* a_params,
                   const int8_t* W, const float* w_scale,
                   const int32_t* w_sum, void* Y, int y_dtype,
                   int64_t M, int64_t N, int64_t K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
