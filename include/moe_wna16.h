/*
 * moe_wna16 — fused mixture-of-experts layer with weight-only quantised experts on MI355X (gfx950).
 *
 * The layer: top-k routing -> moe_align_block_size -> one grouped GEMM over all experts for w13 with
 * the weights decoded in registers -> SiLU(gate) * up -> grouped GEMM for w2 -> top-k weighted
 * combine.  The one-launch grouped GEMM over every expert (instead of one launch per expert) is the
 * method of "[Kernel] add triton fused moe kernel for gptq/awq" (PR description); the align step and
 * its graph-capturable form are named in that PR's notes; the weight encodings follow the same PR's
 * review thread (a format that accepts GPTQ/AWQ weights) and the benchmark script of "[Kernel]
 * optimize performance of gptq marlin kernel when n is small" (uint4, group 128, integer zero
 * point).  The int8 variant (w8a16: symmetric, one scale per output channel, no zero point) follows
 * the int8 MoE backend listing (make_int8_moe_quant_config and the int8 weight schema).
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers are caller-owned device buffers; the library never
 *     allocates, frees or synchronises inside these calls, and never reads device data on the host.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*, NULL = default stream) and is
 *     safe to capture in a HIP graph.  Results are available once the stream reaches that point.
 *   - Every output element is written (padding included), so outputs need no initialisation.
 *   - Arguments are checked on the host before anything is enqueued.  A non-zero status means
 *     nothing was enqueued (except MOE_ERR_HIP, a launch failure); moe_last_error() then returns a
 *     message for the calling thread.
 *   - dtype: 0 = fp16, 1 = bf16.  Activations, outputs and weight scales share it.
 *   - Rows are contiguous (row-major).  Alignment: activations, weights and outputs 16 bytes;
 *     uint4 scales 4 bytes; int8 scales and uint4 zero points 2 bytes; int32 and float arrays
 *     4 bytes; workspaces 256 bytes.  A misaligned pointer returns MOE_ERR_INVALID_ARG.
 *   - fp16 with uint4 weights: activations below 2^-10 in magnitude may lose up to 4 low bits of
 *     precision inside the GEMMs, and at block_m 64 / 128 group scales above 273 overflow (decoded
 *     weights beyond about 4000); neither occurs for quantised model weights and activations of
 *     ordinary scale, and bf16 has neither limit.
 *
 * Weight storage (row-major, expert-major; N = output features, K = input features):
 *   int4 (quant {4, 128, 1}): B uint8 [E, N, K/2], byte j of a row holds k = 2j in bits 0-3 and
 *        k = 2j+1 in bits 4-7; scales [E, N, K/128]; zeros uint8 [E, N, K/256], byte j holds the
 *        zero point of group 2j in bits 0-3 and of group 2j+1 in bits 4-7.
 *        Decoded weight w[n][k] = (q - z) * s of its group.
 *   int8 (quant {8, 0, 0}): B int8 [E, N, K]; scales [E, N]; no zeros.  w[n][k] = q * s.
 *   w13 rows [0, I) are the gate projection, rows [I, 2I) the up projection.
 */
#ifndef MOE_WNA16_H
#define MOE_WNA16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, non-positive size, inconsistent args */
  MOE_ERR_UNSUPPORTED = -2,   /* valid request outside what the kernels implement */
  MOE_ERR_CAPACITY = -3,      /* an output buffer is smaller than the worst case needs */
  MOE_ERR_WORKSPACE = -4,     /* workspace smaller than fused_moe_wna16_workspace_size() */
  MOE_ERR_HIP = -5            /* a HIP launch failed (message in moe_last_error) */
};

enum { MOE_DTYPE_FP16 = 0, MOE_DTYPE_BF16 = 1 };
enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum { MOE_ACT_NONE = 0, MOE_ACT_SILU_MUL = 1 };

/* Weight encoding. {4, 128, 1}: uint4 with per-group-of-128 scales and integer zero points.
 * {8, 0, 0}: int8 symmetric with one scale per output channel.  Anything else: UNSUPPORTED. */
typedef struct {
  int32_t bits;
  int32_t group_size;
  int32_t has_zero;
} moe_quant_t;

/* Routing rule.
 * score 0 (softmax): ids = the topk largest logits (descending, ties to the lower expert id);
 *   weight = softmax probability, divided by the sum over the chosen experts if renormalize,
 *   times scale.  num_groups must be 1.
 * score 1 (sigmoid): s = 1/(1+e^-logit) in float32 with a specified exp (Cody-Waite reduction
 *   with C1 = 355/512, degree-7 Taylor polynomial, no fused multiply-add), so ids are reproducible
 *   bit for bit; experts form num_groups contiguous groups scored by the sum of their two largest s;
 *   the topk_groups best groups are kept (ties to the lower group id) and ids are the topk largest
 *   s inside them (ties to the lower id); weight = s / (sum over chosen, if renormalize) * scale.
 * DeepSeek-V3 uses {1, 1, 8, 4, 2.5f}; Mixtral-style top-2 softmax uses {0, 1, 1, 1, 1.0f}. */
typedef struct {
  int32_t score;
  int32_t renormalize;
  int32_t num_groups;
  int32_t topk_groups;
  float scale;
} moe_routing_t;

/* Top-k routing of M tokens over E experts.
 *   logits       device float [M, E]
 *   topk_weights device float [M, topk]   (out)
 *   topk_ids     device int32 [M, topk]   (out; slot s = m*topk + j is token m's j-th choice)
 * Limits: 1 <= E <= 1024, 1 <= topk <= min(E, 32); for sigmoid, E % num_groups == 0,
 * num_groups <= 64, 1 <= topk_groups <= num_groups and topk <= topk_groups * E / num_groups.
 * M == 0 is a no-op.  Logits must be finite. */
int moe_topk_softmax(const float* logits, int M, int E, int topk, const moe_routing_t* routing,
                     float* topk_weights, int32_t* topk_ids, void* stream);

/* Length that sorted_token_ids needs for numel slots: numel + min(E, numel) * (block_m - 1). */
int64_t moe_align_capacity(int numel, int E, int block_m);

/* moe_align_block_size ("[Kernel] add triton fused moe kernel for gptq/awq", PR notes: the
 * shared-memory version for large expert counts that works under graph capture).
 * Groups the numel = M*topk token-slots by expert and pads each group to a multiple of block_m:
 *   sorted_token_ids device int32 [capacity] (out): for experts in ascending order, the slots of
 *     expert e in ascending slot order, then sentinel entries (value numel) up to the next multiple
 *     of block_m; experts with no slots take no space; entries from T to capacity are sentinels.
 *   expert_ids device int32 [ceil(capacity / block_m)] (out): expert of each block, -1 past T.
 *   num_tokens_post_padded device int32 [1] (out): T, the padded total (stays on the device).
 * Ids outside [0, E) are not listed (a slot of another shard).  The result is deterministic.
 * numel = 0 writes T = 0 (and sentinels / -1 over any capacity given); with capacity 0 the
 * sorted_token_ids and expert_ids pointers may be NULL.
 * Limits: 1 <= E <= 1024, block_m in {16, 32, 64, 128, 256}, numel <= 2^24,
 * capacity >= moe_align_capacity(numel, E, block_m) (else MOE_ERR_CAPACITY). */
int moe_align_block_size(const int32_t* topk_ids, int numel, int E, int block_m,
                         int32_t* sorted_token_ids, int32_t* expert_ids,
                         int32_t* num_tokens_post_padded, int64_t capacity, void* stream);

/* Grouped GEMM over all experts in one launch with in-kernel weight decoding (the fused-MoE
 * kernel of "[Kernel] add triton fused moe kernel for gptq/awq"; the K tile always equals the
 * quantisation group, the bug reported in "[Model] Add Support for GPTQ Fused MOE" cannot occur).
 * For every slot s listed at position p < T of sorted_token_ids, with e = expert_ids[p / block_m]:
 *   h = A[s / a_row_div, :] . W[e]^T  (float32 accumulation of the decoded weights)
 *   act 0: C[s, 0:N]   = h                         (C is [num_slots, N])
 *   act 1: C[s, 0:N/2] = SiLU(h[:N/2]) * h[N/2:]   (C is [num_slots, N/2]; w13 gate/up)
 *   then times topk_weights[s] if topk_weights is not NULL; rounded to dtype.
 *   A      device dtype [num_a_rows, K]   (a_row_div = topk for the first GEMM of the layer,
 *                                           1 for the second)
 *   B, scales, zeros: weight storage of E experts with N rows and K columns (zeros NULL for int8)
 *   sorted_token_ids/expert_ids/num_tokens_post_padded: output of moe_align_block_size
 *     with the same block_m; capacity = length of sorted_token_ids.
 * Rows of C whose slot is not listed are not written.  num_slots = 0 returns MOE_OK at once
 * (no pointer is checked or touched).
 * Limits: K % 256 == 0, N % 128 == 0, block_m in {16, 32, 64, 128, 256} (256: N % 256 == 0,
 * else MOE_ERR_UNSUPPORTED), num_a_rows * a_row_div >= num_slots.  uint4 at block_m 16 and 32: a
 * workgroup stages the scales and zero points of its whole K range in LDS beside its activation
 * tiles (160 KiB in all), which allows K up to 36,096 at block_m 16 and 35,840 at block_m 32;
 * longer K returns MOE_ERR_UNSUPPORTED before any launch (block_m 64, 128 and 256 hold two
 * k-blocks of them at a time and have no such limit). */
int moe_wna16_gemm(const void* A, int num_a_rows, int a_row_div, const void* B, const void* scales,
                   const void* zeros, const moe_quant_t* quant, int E, int N, int K, int dtype,
                   const int32_t* sorted_token_ids, const int32_t* expert_ids,
                   const int32_t* num_tokens_post_padded, int64_t capacity, int block_m,
                   int num_slots, const float* topk_weights, int act, void* C, void* stream);

/* Dense GEMM with weights decoded in the kernel: the one-expert, every-row-routed case of
 * moe_wna16_gemm without the align arrays.  "[Kernel] optimize performance of gptq marlin kernel when
 * n is small" benchmarks this operation for uint4 g128 with integer zero points at m = 16,
 * k = 8192, n = 128 ... 32768 (its benchmark script and table), where n alone gives too few
 * workgroups to stream the weights; that PR adds an atomic-add reduction for it.  Here the K range
 * is split across workgroups into float32 partials that a second launch sums in a fixed order
 * (deterministic), and the split is chosen so that about 512 workgroups stream the weights.
 *   C[m, 0:N] = A[m, :] . W^T  (float32 accumulation of the decoded weights), rounded to dtype
 *   A         device dtype [M, K]
 *   B, scales, zeros: weight storage of one expert (E = 1) with N rows and K columns (zeros NULL
 *             for int8)
 *   workspace device buffer of at least moe_wna16_dense_gemm_workspace_size(M, N, K, quant, dtype)
 *             bytes, 256-byte aligned (may be NULL when that size is 0: no split)
 *   C         device dtype [M, N]; every element is written
 * Limits: K % 256 == 0, N % 128 == 0, and the uint4 K limits of moe_wna16_gemm (rows per block:
 * the smallest of 16, 32, 64 (int8: 128) that holds M; larger M runs several blocks). */
int moe_wna16_dense_gemm(const void* A, int M, int K, const void* B, const void* scales,
                         const void* zeros, const moe_quant_t* quant, int N, int dtype,
                         void* workspace, size_t workspace_bytes, void* C, void* stream);

/* Workspace bytes moe_wna16_dense_gemm needs (0 when it does not split K; 0 for invalid sizes). */
size_t moe_wna16_dense_gemm_workspace_size(int M, int N, int K, const moe_quant_t* quant,
                                           int dtype);

/* Grouped GEMM over activations already batched per expert: the BatchedExperts activation format
 * that the int8 MoE backend listing selects for expert-parallel dispatch (select_int8_moe_backend,
 * make_int8_moe_kernel: sized by a per-rank max_num_tokens).  The pages give no layout; the one used
 * here is the plainest reading.  No align step: for every expert e and row r < min(
 * expert_num_tokens[e], max_tokens):
 *   h = A[e, r, :] . W[e]^T  (float32 accumulation of the decoded weights)
 *   act 0: C[e, r, 0:N] = h;  act 1: C[e, r, 0:N/2] = SiLU(h[:N/2]) * h[N/2:]; rounded to dtype.
 *   A     device dtype [E, max_tokens, K]
 *   expert_num_tokens device int32 [E] (read on the device; negative counts as 0)
 *   B, scales, zeros: weight storage of E experts with N rows and K columns (zeros NULL for int8)
 *   C     device dtype [E, max_tokens, N] (act 1: N/2 columns); rows at or past an expert's count
 *         are not written
 *   block_m 0 = the smallest of {16, 32, 64} (int8: 128) that holds max_tokens
 * Limits: 1 <= E <= 1024, K % 256 == 0, N % 128 == 0, the uint4 K limits of moe_wna16_gemm,
 * below 2^31 bytes (32-bit offsets): A (E * max_tokens * K * 2) and one expert's weights. */
int moe_wna16_batched_gemm(const void* A, int E, int max_tokens, int K,
                           const int32_t* expert_num_tokens, const void* B, const void* scales,
                           const void* zeros, const moe_quant_t* quant, int N, int dtype,
                           int block_m, int act, void* C, void* stream);

/* w8a8: the int8 MoE backend listing pairs int8 weights with one symmetric scale per output
 * channel (kInt8StaticChannelSym) with activations quantised per token at run time
 * (kInt8DynamicTokenSym; int8_w8a8_moe_quant_config with per_act_token_quant).  The pages print no
 * formula; the one used is the plain symmetric quantisation, decided in float32.
 *
 * moe_quant_int8_rows: for each row of x (device dtype [rows, K]):
 *   scales[row] = max_k |x[row, k]| / 127 (one correctly rounded float32 division),
 *   q[row, k] = clamp(rint(x[row, k] / scales[row]), -127, 127), rint = round half to even;
 *   a row of zeros gets scale 0 and codes 0.
 *   q device int8 [rows, K]; scales device float [rows].  Limits: K % 256 == 0. */
int moe_quant_int8_rows(const void* x, int rows, int K, int dtype, int8_t* q, float* scales,
                        void* stream);

/* moe_w8a8_gemm: the grouped GEMM of moe_wna16_gemm with int8 activations, on the integer matrix
 * cores.  For every listed slot s (row = s / a_row_div, e = the block's expert):
 *   h[n] = (sum_k A[row, k] * B[e, n, k]) * a_scales[row] * w_scales[e, n]  (exact integer sum)
 *   act 0: C[s, 0:N] = h;  act 1: C[s, 0:N/2] = SiLU(h[:N/2]) * h[N/2:]; times topk_weights[s] if
 *   not NULL; rounded to dtype.
 *   A        device int8 [num_a_rows, K], a_scales device float [num_a_rows] (moe_quant_int8_rows)
 *   B        device int8 [E, N, K], w_scales device dtype [E, N] (the int8 weight storage above)
 *   sorted_token_ids / expert_ids / num_tokens_post_padded: moe_align_block_size with block_m
 * Rows of C whose slot is not listed are not written.  num_slots = 0 returns MOE_OK at once.
 * Limits: block_m in {16, 32, 64, 128}, or 256 where N / 2 (act 1) is a multiple of 128 or N
 * (act 0) a multiple of 256 (the 32x32 integer kernel, one column tile per wavefront), K % 256 == 0,
 * N % 128 == 0, K <= 131072 (the int32 sums of code products stay below 2^31). */
int moe_w8a8_gemm(const int8_t* A, const float* a_scales, int num_a_rows, int a_row_div,
                  const int8_t* B, const void* w_scales, int E, int N, int K, int dtype,
                  const int32_t* sorted_token_ids, const int32_t* expert_ids,
                  const int32_t* num_tokens_post_padded, int64_t capacity, int block_m,
                  int num_slots, const float* topk_weights, int act, void* C, void* stream);

/* The whole layer with w8a8 experts: routing and align as in fused_moe_wna16, x quantised per
 * token (moe_quant_int8_rows), w8a8 GEMM1 with SiLU(gate) * up into dtype rows, those rows
 * quantised per slot, w8a8 GEMM2 into float32 rows, top-k weighted combine in float32 (fixed order).
 *   w13 device int8 [E, 2I, H], w13_scales device dtype [E, 2I]; w2 int8 [E, H, I], w2_scales [E, H]
 *   workspace: at least fused_moe_w8a8_workspace_size(...) bytes, 256-byte aligned
 *   block_m 0 = the library's choice (moe_pick_block_m for int8 weights; 128 where it picks 256 and
 *   256 is not available)
 * Deterministic.  Limits: H % 256 == 0, I % 256 == 0, H and I <= 131072 (int32 sums), block_m
 * in {0, 16, 32, 64, 128}, or 256 where I % 128 == 0 (always, given I % 256 == 0), M * topk <=
 * 2^24, and below 2^31 (32-bit offsets): M * H, M * topk * I and 2I * H. */
int fused_moe_w8a8(const void* x, const float* router_logits, int M, int H, int I, int E, int topk,
                   const moe_routing_t* routing, const int8_t* w13, const void* w13_scales,
                   const int8_t* w2, const void* w2_scales, int dtype, int block_m,
                   void* workspace, size_t workspace_bytes, void* out, float* topk_weights_out,
                   int32_t* topk_ids_out, void* stream);

/* Workspace bytes fused_moe_w8a8 needs (0 for invalid sizes). */
size_t fused_moe_w8a8_workspace_size(int M, int H, int I, int E, int topk, int dtype, int block_m);

/* The whole layer with GPTQ act-order uint4 experts: the group of an input column is given per
 * column (g_idx) rather than by its position.  The GEMM of "[Kernel] optimize performance of gptq
 * marlin kernel when n is small" takes g_idx and sort_indices for this (its benchmark passes them
 * empty); here the experts arrive in the sorted storage: for expert e, w13_perm[e] (int32 [H]) lists
 * the original input columns in group order (group g = w13_perm[e][128g : 128g+128], i.e. a stable
 * argsort of g_idx), and w13 / w13_scales / w13_zeros are the uint4 storage above of the weights
 * with their columns in that order; likewise w2_perm [E, I] for w2.  The layer gathers each slot's
 * activation row through its expert's permutation before each GEMM, and is otherwise
 * fused_moe_wna16 (the same result as decoding w[n, k] = (q - z[g_idx[k]]) * s[g_idx[k]] in the
 * original column order).  Permutation entries outside [0, H) (or [0, I)) read as zero.
 *   workspace: at least fused_moe_wna16_act_order_workspace_size(...) bytes.
 * Limits: those of fused_moe_wna16 for uint4 weights, and the gathered rows of the first GEMM
 * below 2^31 bytes (M * topk * H * 2, 32-bit offsets). */
int fused_moe_wna16_act_order(const void* x, const float* router_logits, int M, int H, int I,
                              int E, int topk, const moe_routing_t* routing, const void* w13,
                              const void* w13_scales, const void* w13_zeros,
                              const int32_t* w13_perm, const void* w2, const void* w2_scales,
                              const void* w2_zeros, const int32_t* w2_perm, int dtype,
                              int block_m, void* workspace, size_t workspace_bytes, void* out,
                              float* topk_weights_out, int32_t* topk_ids_out, void* stream);

/* Workspace bytes fused_moe_wna16_act_order needs (0 for invalid sizes). */
size_t fused_moe_wna16_act_order_workspace_size(int M, int H, int I, int E, int topk, int dtype,
                                                int block_m);

/* GPTQ / AWQ checkpoint storage of E experts -> the canonical uint4 storage above, on the device.
 * "[Kernel] add triton fused moe kernel for gptq/awq" (review thread) asks for a weight format that
 * accepts GPTQ and AWQ checkpoints; the pages print neither checkpoint's packing, and the layouts
 * read here are the ones those checkpoint families ship, per expert (N output rows, K inputs):
 *   format 0 (GPTQ): qweight int32 [E, K/8, N], code (k, n) in bits 4 (k % 8) .. + 3 of word
 *     [k / 8, n]; qzeros int32 [E, K/128, N/8], zero (g, n) in bits 4 (n % 8) of word [g, n / 8];
 *     scales dtype [E, K/128, N]; g_idx int32 [E, K] (act-order: input column k is in group
 *     g_idx[k]) or NULL.
 *   format 1 (AWQ): qweight int32 [E, K, N/8], code (k, n) in nibble j of word [k, n / 8] where
 *     n % 8 = (0, 2, 4, 6, 1, 3, 5, 7)[j]; qzeros int32 [E, K/128, N/8] packed the same way;
 *     scales dtype [E, K/128, N]; g_idx must be NULL.
 *   Zero points are taken as stored (decoded weight (q - z) * s; no "z - 1" offset).
 * Writes B uint8 [E, N, K/2], scales_out dtype [E, N, K/128], zeros_out uint8 [E, N, K/256].  With
 * g_idx it also writes perm_out int32 [E, K], the stable argsort of each expert's g_idx, and B holds
 * the columns in that order: the sorted storage fused_moe_wna16_act_order takes (w13 of a gate and
 * an up matrix sharing one g_idx: repack each into its rows of w13, or repack a [E, 2I]-row
 * checkpoint).  Each group must hold exactly 128 columns; otherwise a short group is padded with the
 * column index K (read as zero by the act-order layer), columns past a full group or with g_idx
 * outside [0, K/128) are left out, and each such column adds 1 to *invalid_out (a device int32 the
 * caller zeroes first; NULL: not counted).
 * Limits: K % 256 == 0, N % 8 == 0, K <= 16384 with g_idx.  Alignment: B 16 bytes, scales_out 4,
 * zeros_out and scales 2, int32 arrays 4.  Asynchronous on stream; allocates nothing. */
enum { MOE_FORMAT_GPTQ = 0, MOE_FORMAT_AWQ = 1 };
int moe_repack_uint4(int format, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                     const int32_t* g_idx, int E, int N, int K, int dtype, uint8_t* B,
                     void* scales_out, uint8_t* zeros_out, int32_t* perm_out, int32_t* invalid_out,
                     void* stream);

/* The block_m fused_moe_wna16 uses when called with block_m = 0, for weights of `bits` (4 or 8)
 * bits and activations of `dtype`: the smallest of {16, 32, 64, 128, 256} that holds 1.5x the
 * average number of slots per active expert (min(E, M*topk) experts), so a typical expert's slots
 * share one block and its weights are streamed and decoded once; bf16 uint4 keeps 64 up to 128
 * needed rows; fp16 uint4 stops at 64, and takes 32 where up to 128 rows would be needed (its
 * 64-row kernel stages activations through registers, which measured slower than two 32-row
 * blocks).  128- and 256-row blocks run on the 32x32 matrix cores (for fused_moe_w8a8 too).
 * Returns -1 for non-positive sizes, other bit widths or other dtypes. */
int moe_pick_block_m(int M, int E, int topk, int bits, int dtype);

/* Workspace bytes fused_moe_wna16 needs for these sizes (block_m 0 = library's choice). */
size_t fused_moe_wna16_workspace_size(int M, int H, int I, int E, int topk, const moe_quant_t* quant,
                                      int dtype, int block_m);

/* The whole layer:  out[m] = sum_j w[m,j] * W2[e_mj] (SiLU(gate_e x_m) * up_e x_m), with (e_mj, w[m,j])
 * from the routing rule applied to router_logits.
 *   x             device dtype [M, H]
 *   router_logits device float [M, E]
 *   w13*          weight storage of E experts, N = 2I rows, K = H columns
 *   w2*           weight storage of E experts, N = H rows, K = I columns
 *   workspace     device buffer of at least fused_moe_wna16_workspace_size(...) bytes
 *   out           device dtype [M, H]
 *   topk_weights_out / topk_ids_out: optional device [M, topk] copies of the routing result
 *   block_m       0 = library's choice, else one of {16, 32, 64, 128, 256}
 * Launches, by the path fused_moe_wna16_path names:
 *   MOE_PATH_GROUPED: routing and align (one launch for M <= 4; align over many workgroups in two
 *     launches from 8192 slots, its counts in the workspace), GEMM1 (+SiLU*up; split over K
 *     into float32 partials and a SiLU*up pass when its workgroups would not fill the chip), GEMM2
 *     (split over K into float32 partials at small M; unsplit with block_m 64, it writes dtype rows
 *     times the routing weight), combine (float32 sums in a fixed order);
 *   MOE_PATH_ONE_TOKEN: two launches of one dot product per weight row (the routing inside the
 *     first, SiLU*up; the top-k combine inside the second);
 *   MOE_PATH_FEW_TOKENS: routing, then the same two launches, each workgroup grouping the slots by
 *     expert so that each distinct expert's rows are read once for all its slots.
 * Deterministic: identical inputs give bitwise identical outputs.
 * Limits: those of the calls above with N = 2I and N = H; H % 256 == 0, I % 256 == 0,
 * M * topk <= 2^24, and below 2^31 bytes (32-bit offsets): x (M * H * 2), the intermediate rows
 * (M * topk * I * 2) and one expert's w13. */
int fused_moe_wna16(const void* x, const float* router_logits, int M, int H, int I, int E, int topk,
                    const moe_routing_t* routing, const void* w13, const void* w13_scales,
                    const void* w13_zeros, const void* w2, const void* w2_scales,
                    const void* w2_zeros, const moe_quant_t* quant, int dtype, int block_m,
                    void* workspace, size_t workspace_bytes, void* out, float* topk_weights_out,
                    int32_t* topk_ids_out, void* stream);

/* The launch sequence fused_moe_wna16 takes for these sizes (act_order: the act-order entry point),
 * decided from the sizes alone:
 *   MOE_PATH_ONE_TOKEN  M = 1, uint4, block_m 0, E <= 256, the staged vectors within LDS
 *                       (topk * I up to about 60 K columns);
 *   MOE_PATH_FEW_TOKENS 2 <= M <= 5, uint4, block_m 0, I <= 512, H <= 8192, M * topk <= 256 (on the
 *                       DeepSeek-V3 tensor-parallel share it measured 7 to 25 % faster than the
 *                       grouped GEMMs; slower with wider I or more tokens);
 *   MOE_PATH_GROUPED    otherwise.
 * Returns -1 for sizes fused_moe_wna16 rejects. */
#define MOE_PATH_GROUPED 0
#define MOE_PATH_ONE_TOKEN 1
#define MOE_PATH_FEW_TOKENS 2
int fused_moe_wna16_path(int M, int H, int I, int E, int topk, const moe_quant_t* quant,
                         int block_m, int act_order);

/* Bytes of the static device scratch that fused_moe_wna16_noalloc uses as its workspace. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* fused_moe_wna16 for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments, result and determinism as
 * fused_moe_wna16, without the workspace: the library keeps MOE_NOALLOC_SCRATCH_BYTES (64 MiB) of
 * device memory in a static array, one per GPU it runs on, held until the process ends, and calls
 * no allocator.  That covers every decode batch (M <= 64) of the Mixtral-, Qwen2- and DeepSeek-V3-
 * shaped layers and batches up to about 128-256 tokens; a batch whose
 * fused_moe_wna16_workspace_size exceeds it returns MOE_ERR_WORKSPACE before anything is enqueued.
 * The stream must belong to the current device.  All calls on one GPU share that GPU's scratch:
 * calls that overlap in time on one GPU (different streams or threads) race on it and must be
 * serialised by the caller; calls in order on one stream are safe (each writes every scratch
 * element it reads). */
int fused_moe_wna16_noalloc(const void* x, const float* router_logits, int M, int H, int I, int E,
                            int topk, const moe_routing_t* routing, const void* w13,
                            const void* w13_scales, const void* w13_zeros, const void* w2,
                            const void* w2_scales, const void* w2_zeros, const moe_quant_t* quant,
                            int dtype, int block_m, void* out, float* topk_weights_out,
                            int32_t* topk_ids_out, void* stream);

/* Message for the last non-zero status returned on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_WNA16_H */
