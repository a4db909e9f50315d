// Host-side launchers implemented by the .hip translation units; the C ABI in api.cpp validates
// arguments and then calls these.  Each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct RoutingParams {
  int score;        // 0 softmax, 1 sigmoid
  int renormalize;
  int num_groups;
  int topk_groups;
  float scale;
};

hipError_t launch_routing(const float* logits, int M, int E, int topk, const RoutingParams& p,
                          float* topk_w, int32_t* topk_ids, hipStream_t stream);

// Routing and align in one launch for small batches (route_align_fits(M, E): M <= 4, E <= 256).
bool route_align_fits(int M, int E);
hipError_t launch_route_align(const float* logits, int M, int E, int topk, const RoutingParams& p,
                              float* topk_w, int32_t* topk_ids, int block_m, int32_t* sorted_ids,
                              int32_t* expert_ids, int32_t* num_post, int64_t capacity,
                              hipStream_t stream);
hipError_t launch_align(const int32_t* topk_ids, int numel, int E, int block_m,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_post,
                        int64_t capacity, hipStream_t stream);
// The same output by two launches over many workgroups (for many slots: align_multi_pays);
// scratch: device int32 of align_multi_scratch_bytes(numel, E) bytes.
bool align_multi_pays(int numel);
size_t align_multi_scratch_bytes(int numel, int E);
hipError_t launch_align_multi(const int32_t* topk_ids, int numel, int E, int block_m,
                              int32_t* sorted_ids, int32_t* expert_ids, int32_t* num_post,
                              int64_t capacity, int32_t* scratch, hipStream_t stream);

struct GemmParams {
  const void* A;              // dtype [num_a_rows, K]
  int num_a_rows;
  int a_row_div;
  const uint8_t* B;           // int4: uint8 [E, N, K/2]; int8: int8 [E, N, K]
  const void* scales;         // int4: [E, N, K/128]; int8: [E, N]
  const uint8_t* zeros;       // int4: uint8 [E, N, K/256]; int8: unused
  int E, N, K;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* num_post;
  int num_blocks;             // floor(capacity / block_m): grid extent over blocks
  int num_slots;              // sentinel value (M * topk)
  const float* topk_w;        // nullable: scale output row s by topk_w[s]
  void* C;                    // act: dtype [num_slots, N/2]; out_f32: float [split, num_slots, N];
                              // else dtype [num_slots, N]
  int split_k;                // K split count (out_f32 only, else 1)
  int dense;                  // 1: slot r of block b is row b * block_m + r (< num_slots), expert
                              // 0; sorted_ids, expert_ids and num_post are not read
  int batched;                // 1: A and C hold E blocks of max_tokens rows; block b covers rows
                              // (b % bpe) * block_m .. of expert b / bpe, valid below
                              // min(expert_counts[e], max_tokens); align arrays are not read
  const int32_t* expert_counts;
  int max_tokens;
  int bpe;                    // blocks per expert: ceil(max_tokens / block_m)
  uint32_t dec_mask;          // set by launch_gemm: low nibble-pair mask of the decode
  uint32_t dec_mask_hi;       // set by launch_gemm: high nibble-pair mask (fp16 uint4 decode)
  uint32_t dec_magic;         // set by launch_gemm: magic bias in both 16-bit halves
  int cgroup;                 // set by launch_gemm: column chunks per workgroup (GemmConfig)
};

struct GemmConfig {
  int dtype;     // 0 fp16, 1 bf16
  int bits;      // 4 or 8
  int block_m;   // 16, 32, 64, 128, 256
  int act;       // 0 none, 1 silu-mul
  int out_f32;   // 1: float partials [split, num_slots, N]
  int ntw;       // column tiles of 16 per wavefront: 2, or 4 (block_m 16 only)
  int waves = 4; // wavefronts per workgroup: 4, or 8 (block_m 32 with 2 tiles only; honoured there)
  // column chunks one workgroup streams in turn, its activation rows staged once (1: one chunk).
  // > 1 only where gemm_cgroup_fits: a short K whose whole range is one activation chunk.
  int cgroup = 1;
};

// Column chunks per workgroup > 1 is possible: uint4, block_m 16, no SiLU epilogue, float32
// partials, unsplit, and K within one activation chunk of the 16-row kernel (256).
bool gemm_cgroup_fits(const GemmConfig& c, int K, int split_k);

// Columns of output one workgroup covers (N % this must be 0; act: gate columns).
int gemm_wg_cols(const GemmConfig& c);
// Dynamic LDS of one workgroup for the staged uint4 scales and zero points of its K range.
size_t gemm_meta_lds_bytes(int K, int split_k, const GemmConfig& c);
// All LDS of one workgroup (activation tiles + staged metadata); at most kGemmLdsLimit.
size_t gemm_lds_bytes(int K, int split_k, const GemmConfig& c);
constexpr size_t kGemmLdsLimit = 160 * 1024;
hipError_t launch_gemm(const GemmParams& p, const GemmConfig& c, hipStream_t stream);

// The prefill tiling (prefill.hip): block_m 128 and 256 on the 32x32 matrix cores, 8 wavefronts
// of prefill_nt(c, N) column tiles of 32.  launch_gemm takes it wherever prefill_fits(c, N).
bool prefill_fits(const GemmConfig& c, int N);
int prefill_nt(const GemmConfig& c, int N);
int prefill_wg_cols(const GemmConfig& c, int N);
size_t prefill_lds_bytes(const GemmConfig& c);
hipError_t launch_prefill(const GemmParams& p, const GemmConfig& c, hipStream_t stream);

// out[r, c] = sum_z partial[z, r, c] (z ascending) over rows x cols, rounded to dtype.
hipError_t launch_split_reduce(const float* partial, int split, int rows, int cols, int dtype,
                               void* out, hipStream_t stream);
// w8a8: int8 activations (one float32 scale per row) x int8 weights (one dtype scale per column)
struct W8A8Params {
  const int8_t* A;            // [num_a_rows, K]
  const float* a_scales;      // [num_a_rows]
  int num_a_rows;
  int a_row_div;
  const int8_t* B;            // [E, N, K]
  const void* w_scales;       // dtype [E, N]
  int E, N, K;
  const int32_t* sorted_ids;
  const int32_t* expert_ids;
  const int32_t* num_post;
  int num_blocks;
  int num_slots;
  const float* topk_w;        // nullable
  void* C;                    // dtype [num_slots, N] (act: N/2)
};
hipError_t launch_quant_rows(const void* x, int rows, int K, int dtype, int8_t* q, float* scales,
                             hipStream_t stream);
// out_f32 (act 0 only): C is float [num_slots, N] (the fused layer's second GEMM, combined later)
hipError_t launch_w8a8_gemm(const W8A8Params& p, int block_m, int act, int dtype,
                            hipStream_t stream, int out_f32 = 0);
// The same GEMM on the 32x32x32 integer matrix cores (prefill.hip), block_m 64, 128 and 256;
// launch_w8a8_gemm takes it wherever w8a8_mma32_fits.
bool w8a8_mma32_fits(int block_m, int act, int N);
hipError_t launch_w8a8_mma32(const W8A8Params& p, int block_m, int act, int dtype, int out_f32,
                             hipStream_t stream);

// out[s, j] = in[s / div, perm[ids[s], j]] for slots s < slots, columns j < K (dtype elements); a
// permutation entry outside [0, K) or an expert id outside [0, E) gives zero.
hipError_t launch_gather_cols(const void* in, int div, const int32_t* ids, int E,
                              const int32_t* perm, int K, int slots, int dtype, void* out,
                              hipStream_t stream);
// GPTQ (format 0) / AWQ (format 1) checkpoint storage of E experts -> canonical uint4 storage;
// g_idx non-NULL (GPTQ act-order): perm_out [E, K] and the sorted storage (repack.hip)
hipError_t launch_repack_uint4(int format, const int32_t* qweight, const int32_t* qzeros,
                               const void* scales, const int32_t* g_idx, int E, int N, int K,
                               uint8_t* B, void* scales_out, uint8_t* zeros_out, int32_t* perm_out,
                               int32_t* invalid, hipStream_t stream);
hipError_t launch_combine(const float* partial, int split, const float* topk_w, int M, int topk,
                          int H, int dtype, void* out, hipStream_t stream);
// out[m] = sum_j y[m * topk + j] (j ascending, float32) for dtype rows y [M * topk, H] that already
// carry their routing weight (the second GEMM unsplit); H % 8 == 0
hipError_t launch_combine_rows(const void* y, int M, int topk, int H, int dtype, void* out,
                               hipStream_t stream);
// inter[s, i] = SiLU(sum_z partial[z, s, i]) * sum_z partial[z, s, I + i] (first GEMM split over K)
hipError_t launch_act_combine(const float* partial, int split, int slots, int I, int dtype,
                              void* inter, hipStream_t stream);

// The layer for one token with uint4 g128 experts (gemv.hip), two launches.  up routes the token
// (every workgroup for itself, the first one writing topk_w and topk_ids) and writes
// inter[j, n] = SiLU(gate) * up for the topk slots; down writes out[n] = sum_j topk_w[j] *
// (W2 row n of expert topk_ids[j] . inter[j]) in the activation dtype.
struct SingleParams {
  const void* x;              // dtype [H]
  const float* logits;        // [E]
  RoutingParams rp;
  float* topk_w;              // [topk], written by up
  int32_t* topk_ids;          // [topk], written by up
  const uint8_t* w13;         // [E, 2I, H/2]
  const void* s13;            // dtype [E, 2I, H/128]
  const uint8_t* z13;         // [E, 2I, H/256]
  const uint8_t* w2;          // [E, H, I/2]
  const void* s2;             // dtype [E, H, I/128]
  const uint8_t* z2;          // [E, H, I/256]
  int E, H, I, topk;
  void* inter;                // dtype [topk, I]
  void* out;                  // dtype [H]
  int upw;                    // set by launch_single / launch_few
  int lanes_per_row;          // set by launch_single / launch_few
  int rows_per_wg;            // set by launch_single / launch_few
  int M;                      // launch_few: tokens (x is [M, H], out [M, H], inter [M * topk, I])
};
// E <= 256, topk <= E, H and I multiples of 256 up to 32768, the staged vectors within LDS
bool single_fits(int H, int I, int E, int topk);
hipError_t launch_single(const SingleParams& p, int dtype, hipStream_t stream);
// The layer for a few tokens (2 <= M <= 8, M * topk <= 256, H and I <= 8192) after routing
// (topk_w / topk_ids [M, topk] given): up and down as above, each workgroup grouping the slots by
// expert so that every distinct expert's rows are read once for all its slots.
bool few_fits(int M, int H, int I, int E, int topk);
hipError_t launch_few(const SingleParams& p, int dtype, hipStream_t stream);

}  // namespace moe
