// C ABI of the moe_wna16 library: argument checks (host only, no device access), the tile plan,
// the workspace layout of the fused layer, and the launch sequence.  Declarations and the full
// contract of every entry point are in include/moe_wna16.h.
#include "moe_wna16.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "api_internal.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

int vfail(int code, const char* fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof(buf), fmt, ap);
  g_err = buf;
  return code;
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(code, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_block_m(int bm) { return bm == 16 || bm == 32 || bm == 64 || bm == 128; }
// uint4 / int8 weight-only GEMMs and layers also take 256-row blocks (the 32x32 prefill kernel)
bool valid_block_m_wna16(int bm) { return valid_block_m(bm) || bm == 256; }

int check_dtype(int dtype) {
  if (dtype != MOE_DTYPE_FP16 && dtype != MOE_DTYPE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "dtype %d is not fp16 (0) or bf16 (1)", dtype);
  return MOE_OK;
}

int check_quant(const moe_quant_t* q) {
  if (!q) return fail(MOE_ERR_INVALID_ARG, "quant is NULL");
  if (q->bits == 4) {
    if (q->group_size != 128)
      return fail(MOE_ERR_UNSUPPORTED, "uint4 weights need group_size 128 (got %d)", q->group_size);
    if (!q->has_zero)
      return fail(MOE_ERR_UNSUPPORTED, "uint4 weights need integer zero points (has_zero = 1)");
    return MOE_OK;
  }
  if (q->bits == 8) {
    if (q->group_size != 0)
      return fail(MOE_ERR_UNSUPPORTED, "int8 weights use one scale per output channel (group_size 0)");
    if (q->has_zero)
      return fail(MOE_ERR_UNSUPPORTED, "int8 weights are symmetric (has_zero = 0)");
    return MOE_OK;
  }
  return fail(MOE_ERR_UNSUPPORTED, "bits = %d (supported: 4, 8)", q->bits);
}

int check_routing(const moe_routing_t* r, int E, int topk) {
  if (!r) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
  if (E <= 0 || topk <= 0) return fail(MOE_ERR_INVALID_ARG, "E = %d, topk = %d", E, topk);
  if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E = %d > 1024", E);
  if (topk > E || topk > 32)
    return fail(MOE_ERR_INVALID_ARG, "topk = %d must be <= min(E, 32)", topk);
  if (r->score == MOE_SCORE_SOFTMAX) {
    if (r->num_groups != 1)
      return fail(MOE_ERR_UNSUPPORTED, "softmax routing takes num_groups = 1 (got %d)", r->num_groups);
    return MOE_OK;
  }
  if (r->score != MOE_SCORE_SIGMOID) return fail(MOE_ERR_INVALID_ARG, "score = %d", r->score);
  if (r->num_groups < 1 || r->num_groups > 64 || E % r->num_groups)
    return fail(MOE_ERR_INVALID_ARG, "num_groups = %d must divide E = %d and be <= 64",
                r->num_groups, E);
  if (r->topk_groups < 1 || r->topk_groups > r->num_groups)
    return fail(MOE_ERR_INVALID_ARG, "topk_groups = %d not in [1, num_groups]", r->topk_groups);
  if (topk > r->topk_groups * (E / r->num_groups))
    return fail(MOE_ERR_INVALID_ARG, "topk = %d exceeds the experts of %d kept groups", topk,
                r->topk_groups);
  return MOE_OK;
}

// Longest K of the int8 x int8 GEMMs: their int32 sums of products of codes in [-127, 127]
// stay below 2^31 (127^2 * 131072 = 2,114,060,288).
constexpr int kW8A8MaxK = 131072;

int64_t align_capacity(int64_t numel, int E, int bm) {
  return numel + std::min<int64_t>(E, numel) * (bm - 1);
}

// ------------------------------------------------------------------------------------------------
// tile plan of the fused layer
// ------------------------------------------------------------------------------------------------
struct Plan {
  int bm;
  int64_t cap;
  int nblk;
  int split1;  // > 1: the first GEMM writes float32 partials, a second pass applies SiLU(gate) * up
  int split2;
  int ntw1, ntw2, wv1, wv2;
  size_t off_w, off_ids, off_sorted, off_eids, off_npost, off_inter, off_part, total;
};

// fp16 uint4 stops at 64 (the 16-row kernel at 128 rows stages activations through registers at
// two wavefronts per SIMD: Qwen2-shaped layer at M = 512, GEMMs 798 us at 128 rows, 497 us at 64).
// fp16 uint4 where 64 rows would be picked for up to 128 needed: 32 rows (the fp16 64-row kernel
// also stages activations through registers; Qwen2 shape at M = 512, ~72 slots per expert: 555 ->
// 529 us per layer; bf16 and int8 measured equal or slower at 32).  bf16 uint4 and int8 beyond 128
// needed rows: 256-row blocks, which hold a whole expert's slots at the DeepSeek-V3 prefill shape
// (101 to 159 slots per expert at 4096 tokens), so each weight is decoded once for all of them
// (first GEMM, uint4: 2.90 ms at 128 rows, where about half the experts spill a short second block
// that decodes every weight again, 2.63 ms at 256; int8 weights 2.91 -> 2.83 ms); int8 takes 128
// rows from 64 needed, bf16 uint4 keeps 64 rows up to 128 needed (measured against 128).
int pick_block_m(int M, int topk, int E, int bits, int dtype) {
  const int64_t slots = (int64_t)M * topk;
  const int64_t active = std::max<int64_t>(1, std::min<int64_t>(E, slots));
  const int64_t avg = (slots + active - 1) / active;
  const int64_t need = avg + avg / 2;
  for (int bm : {16, 32})
    if (need <= bm) return bm;
  if (bits == 4 && dtype == MOE_DTYPE_FP16) return need <= 128 ? 32 : 64;
  if (need <= 64 || (bits == 4 && need <= 128)) return 64;
  return need <= 128 ? 128 : 256;
}

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

// The few-token dot-product path: up to 5 tokens with I <= 512 (a tensor-parallel share of many
// experts).  Measured against the grouped GEMMs on the DeepSeek-V3 TP share (graph replays, layer
// us): M = 2 26.4 against 35.1, M = 3 35.0 / 40.0, M = 4 38.2 / 47.2; with both routing launches
// ranking per workgroup, M = 5 45.8 / 49.3, M = 6 60.0 / 53.6, M = 7 67.3 / 54.7, M = 8 70.0 /
// 61.0; with I = 2560 (Qwen2 shape) M = 2 83 / 63 and M = 3 112 / 74, so there it stays off.
constexpr int kFewMaxTokens = 5;
constexpr int kFewMaxI = 512;

// The launch sequence of the fused uint4/int8 layer (valid sizes assumed).
int layer_path(int M, int H, int I, int E, int topk, int bits, int block_m, bool act_order) {
  if (bits != 4 || act_order || block_m != 0) return MOE_PATH_GROUPED;
  if (M == 1 && moe::single_fits(H, I, E, topk)) return MOE_PATH_ONE_TOKEN;
  if (M >= 2 && M <= kFewMaxTokens && I <= kFewMaxI && moe::few_fits(M, H, I, E, topk))
    return MOE_PATH_FEW_TOKENS;
  return MOE_PATH_GROUPED;
}

// Column tiles of 16 per wavefront for a grouped GEMM with N weight rows.  Four tiles halve the
// activation traffic per weight byte; they need block_m 16 (at 32 the 4-tile kernel takes 211
// registers, two wavefronts per SIMD, against 128 and four with 2 tiles, and more wavefronts stream
// faster), N divisible by the wider workgroup, and (for the SiLU epilogue, whose grid is narrower)
// enough workgroups to fill the chip.
int pick_ntw(int act, int N, int bm, int64_t est_blocks) {
  if (bm > 16) return 2;
  if (act) return ((N / 2) % 128 == 0 && est_blocks * ((N / 2) / 128) >= 1024) ? 4 : 2;
  return N % 256 == 0 ? 4 : 2;
}

// Wavefronts per workgroup.  8 share one activation tile, so each issues half the activation loads
// per weight byte of a 4-wavefront workgroup:
//   - the second GEMM at block_m 32 (2 column tiles) where N divides the wider workgroup (measured
//     on the fused layer: Mixtral shape at M = 64 -2.2 %, Qwen2 shape at M = 128 -1.3 %);
//   - the first GEMM at block_m 32 for wide experts (I >= 8192: Mixtral shape at M = 64, three
//     alternating runs each, 202-203 -> 196-199 us per layer); for narrower ones (Qwen2 shape, I =
//     2560, M = 128: 237.6 -> 244.9 us) it keeps 4;
//   - both GEMMs at block_m 64 and 128 when the activations go straight from memory into LDS
//     (bf16 activations or int8 weights), where the activation loads are two to four times the
//     weight loads (DeepSeek-V3-shaped prefill layers: -2 to -5 %); with fp16 uint4 weights, whose
//     activations are staged through registers, it measured 4 % slower and keeps 4.
int pick_waves(int act, int N, int bm, int ntw, int dtype, int bits) {
  if (ntw != 2) return 4;
  if (bm >= 64) {
    if (dtype != 1 && bits != 8) return 4;
    return (act ? (N / 2) % 128 : N % 256) == 0 ? 8 : 4;
  }
  if (bm != 32) return 4;
  if (act) return (N / 2 >= 8192 && (N / 2) % 128 == 0) ? 8 : 4;
  return N % 256 == 0 ? 8 : 4;
}

// The uint4 scales and zero points of a workgroup's whole K range are staged in LDS, so a long K
// may not fit beside the activation tiles: fall back to two column tiles per wavefront and four
// wavefronts (fewer rows per workgroup), and reject the shape if even that does not fit.
int fit_lds(int K, int split, moe::GemmConfig& c, const char* what) {
  if (moe::gemm_lds_bytes(K, split, c) > moe::kGemmLdsLimit) {
    c.ntw = 2;
    c.waves = 4;
  }
  const size_t need = moe::gemm_lds_bytes(K, split, c);
  if (need > moe::kGemmLdsLimit)
    return fail(MOE_ERR_UNSUPPORTED, "%s: K = %d needs %zu bytes of LDS per workgroup (limit %zu)",
                what, K, need, moe::kGemmLdsLimit);
  return MOE_OK;
}

// Split count over K for a grouped GEMM with `wgs` workgroups per split: the smallest divisor of
// the k-block count that reaches target_wgs workgroups while leaving every split at least min_kb
// k-blocks (start-up is paid per workgroup), else the largest such divisor.
int pick_split(int kb_total, int64_t wgs, int min_kb, int64_t target_wgs) {
  int best = 1;
  for (int d = 1; d <= kb_total; ++d) {
    if (kb_total % d || kb_total / d < min_kb) continue;
    best = d;
    if (wgs * d >= target_wgs) break;
  }
  return best;
}

int64_t estimate_blocks(int64_t slots, int E, int bm) {
  return std::max<int64_t>(std::min<int64_t>(E, slots), slots / bm);
}

// Blocks a batch of M tokens is expected to fill when each token picks topk of E experts evenly:
// E * (1 - (1 - topk/E)^M) distinct experts, at least M * topk / bm blocks.  min(E, M * topk)
// overestimates at small M (Mixtral shape, M = 4: 8 assumed, 5.5 expected), which left the split
// second GEMM with about one workgroup per compute unit (measured: 4 % slower layer).
int64_t estimate_active_blocks(int64_t M, int topk, int E, int bm) {
  const double act = E * (1.0 - std::pow(1.0 - (double)topk / E, (double)M));
  return std::max<int64_t>(std::max<int64_t>(1, (int64_t)(act + 0.5)), M * topk / bm);
}

Plan make_plan(int M, int H, int I, int E, int topk, int bits, int dtype, int block_m) {
  Plan p{};
  const int64_t slots = (int64_t)M * topk;
  p.bm = block_m > 0 ? block_m : pick_block_m(M, topk, E, bits, dtype);
  p.cap = align_capacity(slots, E, p.bm);
  p.nblk = (int)((p.cap + p.bm - 1) / p.bm);
  const int kb = bits == 4 ? 128 : 64;
  const int64_t est_blocks = estimate_blocks(slots, E, p.bm);
  p.ntw1 = pick_ntw(1, 2 * I, p.bm, est_blocks);
  p.ntw2 = pick_ntw(0, H, p.bm, est_blocks);
  p.wv1 = pick_waves(1, 2 * I, p.bm, p.ntw1, dtype, bits);
  p.wv2 = pick_waves(0, H, p.bm, p.ntw2, dtype, bits);
  // The first GEMM (K = H) keeps SiLU in its epilogue unless its workgroups cannot fill the chip:
  // then it is split over K into float32 partials and a second pass applies SiLU(gate) * up.
  //   - under 256 workgroups (few experts and a narrow I, as in a tensor-parallel share of many
  //     small experts at M = 1): split to ~512;
  //   - under one round of resident workgroups (~1024): split towards ~1024, keeping >= 14
  //     k-blocks per split so the extra pass stays small against the stream (measured: DeepSeek-V3
  //     TP share M = 16 107 -> 103 us, M = 64 199 -> 190 us, Qwen2 shape M = 1 62 -> 59 us; the
  //     Mixtral shape at M = 1, 448 workgroups of 32 k-blocks, is 1-4 % slower split in two);
  //   - otherwise unsplit: with more workgroups than that the extra pass costs what the split
  //     gains (Mixtral shape at M = 16 and 64: 3-6 % slower split).
  const int64_t blocks = estimate_active_blocks(M, topk, E, p.bm);
  const int64_t wgs1 = blocks * (I / (p.ntw1 / 2 * 16 * p.wv1));  // unsplit SiLU workgroups
  const int64_t wgs1_split = blocks * (I / 64);                   // per split (128 columns of 2I)
  if (wgs1 < 256)
    p.split1 = pick_split(H / kb, wgs1_split, 4, 512);
  else if (wgs1 < 1024)
    p.split1 = pick_split(H / kb, wgs1_split, 14, 1024);
  else
    p.split1 = 1;
  // The second GEMM (K = I) writes float32 partials anyway; split it to about two workgroups per
  // compute unit (more, shorter workgroups pay their start-up more often and write more partials)
  const int64_t wgs2 = estimate_active_blocks(M, topk, E, p.bm) * (H / (p.ntw2 * 16 * p.wv2));
  p.split2 = pick_split(I / kb, wgs2, 4, 512);
  size_t off = 0;
  p.off_w = off;      off += up256((size_t)slots * 4);
  p.off_ids = off;    off += up256((size_t)slots * 4);
  p.off_sorted = off; off += up256((size_t)p.cap * 4);
  p.off_eids = off;   off += up256((size_t)p.nblk * 4);
  p.off_npost = off;  off += 256;
  p.off_inter = off;  off += up256((size_t)slots * I * 2);
  p.off_part = off;
  off += up256(std::max((size_t)p.split1 * slots * 2 * I, (size_t)p.split2 * slots * H) * 4);
  p.total = off;
  return p;
}

// Column chunks per second-GEMM workgroup.  With K = I = 256 (a tensor-parallel share of many
// small experts) a 16-row workgroup streams two k-blocks per column chunk, and its start-up (slot
// ids, activation rows, metadata, the first weight latency) costs as much as the stream; streaming
// several chunks against one staged activation tile pays it once.  Four chunks where that still
// leaves >= 512 workgroups, else two, else one (measured on the DeepSeek-V3 TP share, layer per
// call: M = 16 103 -> 95 us, M = 64 189 -> 175 us, M = 256 249 -> 233 us at four; two at M = 1,
// 224 -> 112 workgroups, 29.8 -> 31.7 us, so none there; seven or fourteen slower).
int pick_cgroup(const moe::GemmConfig& c, int N, int K, int split, int64_t blocks) {
  if (!moe::gemm_cgroup_fits(c, K, split)) return 1;
  const int n_chunks = N / moe::gemm_wg_cols(c);
  for (int g : {4, 2})
    if (n_chunks % g == 0 && blocks * (n_chunks / g) >= 512) return g;
  return 1;
}

// ------------------------------------------------------------------------------------------------
// dense GEMM (one expert, every row a slot)
// ------------------------------------------------------------------------------------------------
struct DensePlan {
  moe::GemmConfig c;
  int nblk;
  int split;
  size_t ws;  // float32 partials [split, M, N] when split > 1
};

// Rows per block: the smallest of {16, 32, 64} (int8: up to 128) that holds M, so short batches
// stream every weight once.  Column tiles and split as for the grouped GEMM: four tiles at 16 rows
// only while four-tile workgroups can still reach ~512 with splits of >= 4 k-blocks (a short N, as in
// n = 4096 at k = 8192, keeps two tiles and so twice the workgroups), then split K to ~512
// workgroups.
DensePlan make_dense_plan(int M, int N, int K, int bits, int dtype) {
  DensePlan d{};
  int bm = 16;
  const int top = bits == 4 ? 64 : 128;
  while (bm < M && bm < top) bm *= 2;
  d.nblk = (M + bm - 1) / bm;
  const int kb_total = K / (bits == 4 ? 128 : 64);
  int ntw = 2;
  if (bm == 16 && N % 256 == 0 && (int64_t)(N / 256) * d.nblk * std::max(1, kb_total / 4) >= 512)
    ntw = 4;
  const int wv = pick_waves(0, N, bm, ntw, dtype, bits);
  const int64_t wgs = (int64_t)d.nblk * (N / (ntw * 16 * wv));
  d.split = pick_split(kb_total, wgs, 4, 512);
  d.c = moe::GemmConfig{dtype, bits, bm, 0, d.split > 1 ? 1 : 0, ntw, wv};
  d.ws = d.split > 1 ? up256((size_t)d.split * M * N * 4) : 0;
  return d;
}

}  // namespace

extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

int moe_pick_block_m(int M, int E, int topk, int bits, int dtype) {
  if (M <= 0 || E <= 0 || topk <= 0 || (bits != 4 && bits != 8)) return -1;
  if (dtype != MOE_DTYPE_FP16 && dtype != MOE_DTYPE_BF16) return -1;
  return pick_block_m(M, topk, E, bits, dtype);
}

int64_t moe_align_capacity(int numel, int E, int block_m) {
  if (numel < 0 || E <= 0 || block_m <= 0) return -1;
  return align_capacity(numel, E, block_m);
}

int moe_topk_softmax(const float* logits, int M, int E, int topk, const moe_routing_t* routing,
                     float* topk_weights, int32_t* topk_ids, void* stream) {
  if (M < 0) return fail(MOE_ERR_INVALID_ARG, "M = %d", M);
  if (int rc = check_routing(routing, E, topk)) return rc;
  if (M == 0) return MOE_OK;
  if (!logits || !topk_weights || !topk_ids)
    return fail(MOE_ERR_INVALID_ARG, "NULL logits / topk_weights / topk_ids");
  if (!aligned(logits, 4) || !aligned(topk_weights, 4) || !aligned(topk_ids, 4))
    return fail(MOE_ERR_INVALID_ARG, "routing buffers must be 4-byte aligned");
  const moe::RoutingParams rp{routing->score, routing->renormalize, routing->num_groups,
                              routing->topk_groups, routing->scale};
  hipError_t e = moe::launch_routing(logits, M, E, topk, rp, topk_weights, topk_ids,
                                     (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "routing launch");
}

int moe_align_block_size(const int32_t* topk_ids, int numel, int E, int block_m,
                         int32_t* sorted_token_ids, int32_t* expert_ids,
                         int32_t* num_tokens_post_padded, int64_t capacity, void* stream) {
  if (numel < 0 || E <= 0) return fail(MOE_ERR_INVALID_ARG, "numel = %d, E = %d", numel, E);
  if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E = %d > 1024", E);
  if (!valid_block_m_wna16(block_m))
    return fail(MOE_ERR_UNSUPPORTED, "block_m = %d (supported: 16, 32, 64, 128, 256)", block_m);
  if (numel > (1 << 24)) return fail(MOE_ERR_UNSUPPORTED, "numel = %d > 2^24", numel);
  // an empty batch still gets its padded total (0) written; its id buffers may then be empty
  if ((numel > 0 && !topk_ids) || (capacity > 0 && (!sorted_token_ids || !expert_ids)) ||
      !num_tokens_post_padded)
    return fail(MOE_ERR_INVALID_ARG, "NULL align buffer");
  if (!aligned(topk_ids, 4) || !aligned(sorted_token_ids, 4) || !aligned(expert_ids, 4) ||
      !aligned(num_tokens_post_padded, 4))
    return fail(MOE_ERR_INVALID_ARG, "align buffers must be 4-byte aligned");
  const int64_t need = align_capacity(numel, E, block_m);
  if (capacity < need)
    return fail(MOE_ERR_CAPACITY, "capacity %lld < %lld needed", (long long)capacity,
                (long long)need);
  if (capacity > (int64_t)1 << 30) return fail(MOE_ERR_UNSUPPORTED, "capacity too large");
  hipError_t e = moe::launch_align(topk_ids, numel, E, block_m, sorted_token_ids, expert_ids,
                                   num_tokens_post_padded, capacity, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "align launch");
}

static int check_weights(const void* B, const void* scales, const void* zeros,
                         const moe_quant_t* q) {
  if (!B || !scales) return fail(MOE_ERR_INVALID_ARG, "NULL weight or scale pointer");
  if (q->has_zero && !zeros) return fail(MOE_ERR_INVALID_ARG, "zeros are NULL but has_zero = 1");
  if (!q->has_zero && zeros)
    return fail(MOE_ERR_INVALID_ARG, "zeros given but has_zero = 0 (both or neither)");
  if (!aligned(B, 16)) return fail(MOE_ERR_INVALID_ARG, "weights must be 16-byte aligned");
  // uint4 scales are read two k-blocks at a time (4-byte loads at even k-blocks; a row of K/128
  // scales is a multiple of 4 bytes since K % 256 == 0); int8 scales and zero points in 2 bytes
  const size_t salign = q->bits == 4 ? 4 : 2;
  if (!aligned(scales, salign))
    return fail(MOE_ERR_INVALID_ARG, "scales must be %zu-byte aligned", salign);
  if (zeros && !aligned(zeros, 2)) return fail(MOE_ERR_INVALID_ARG, "zeros must be 2-byte aligned");
  return MOE_OK;
}

int moe_wna16_gemm(const void* A, int num_a_rows, int a_row_div, const void* B, const void* scales,
                   const void* zeros, const moe_quant_t* quant, int E, int N, int K, int dtype,
                   const int32_t* sorted_token_ids, const int32_t* expert_ids,
                   const int32_t* num_tokens_post_padded, int64_t capacity, int block_m,
                   int num_slots, const float* topk_weights, int act, void* C, void* stream) {
  if (int rc = check_dtype(dtype)) return rc;
  if (int rc = check_quant(quant)) return rc;
  if (E <= 0 || N <= 0 || K <= 0 || num_a_rows < 0 || a_row_div <= 0 || num_slots < 0 ||
      capacity < 0)
    return fail(MOE_ERR_INVALID_ARG, "E=%d N=%d K=%d rows=%d a_row_div=%d slots=%d", E, N, K,
                num_a_rows, a_row_div, num_slots);
  if (act != MOE_ACT_NONE && act != MOE_ACT_SILU_MUL)
    return fail(MOE_ERR_INVALID_ARG, "act = %d", act);
  if (!valid_block_m_wna16(block_m))
    return fail(MOE_ERR_UNSUPPORTED, "block_m = %d (supported: 16, 32, 64, 128, 256)", block_m);
  if (K % 256) return fail(MOE_ERR_UNSUPPORTED, "K = %d must be a multiple of 256", K);
  if (N % 128) return fail(MOE_ERR_UNSUPPORTED, "N = %d must be a multiple of 128", N);
  if (block_m == 256 && N % 256)
    return fail(MOE_ERR_UNSUPPORTED, "block_m 256 needs N = %d to be a multiple of 256", N);
  if ((int64_t)num_a_rows * K * 2 >= ((int64_t)1 << 31) ||
      (int64_t)N * (quant->bits == 4 ? K / 2 : K) >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "A or one expert's weights exceed 2 GiB");
  if ((int64_t)num_a_rows * a_row_div < num_slots)
    return fail(MOE_ERR_INVALID_ARG, "A has %d rows, slots need %lld", num_a_rows,
                (long long)((num_slots + a_row_div - 1) / a_row_div));
  if (num_slots == 0) return MOE_OK;  // nothing to read or write
  if (int rc = check_weights(B, scales, zeros, quant)) return rc;
  if (!A || !C || !sorted_token_ids || !expert_ids || !num_tokens_post_padded)
    return fail(MOE_ERR_INVALID_ARG, "NULL A / C / align buffer");
  if (!aligned(A, 16) || !aligned(C, 16))
    return fail(MOE_ERR_INVALID_ARG, "A and C must be 16-byte aligned");
  if (topk_weights && !aligned(topk_weights, 4))
    return fail(MOE_ERR_INVALID_ARG, "topk_weights must be 4-byte aligned");
  if (num_slots == 0 || capacity == 0) return MOE_OK;
  moe::GemmParams p{};
  p.A = A;
  p.num_a_rows = num_a_rows;
  p.a_row_div = a_row_div;
  p.B = (const uint8_t*)B;
  p.scales = scales;
  p.zeros = (const uint8_t*)zeros;
  p.E = E;
  p.N = N;
  p.K = K;
  p.sorted_ids = sorted_token_ids;
  p.expert_ids = expert_ids;
  p.num_post = num_tokens_post_padded;
  // T is a multiple of block_m and <= capacity, so whole blocks below capacity cover every real
  // block; a corrupt num_tokens_post_padded then cannot push reads past sorted_token_ids
  p.num_blocks = (int)(capacity / block_m);
  p.num_slots = num_slots;
  p.topk_w = topk_weights;
  p.C = C;
  p.split_k = 1;
  const int ntw = pick_ntw(act, N, block_m, estimate_blocks(num_slots, E, block_m));
  moe::GemmConfig c{dtype, quant->bits, block_m, act, 0, ntw,
                    pick_waves(act, N, block_m, ntw, dtype, quant->bits)};
  if (int rc = fit_lds(K, 1, c, "gemm")) return rc;
  hipError_t e = moe::launch_gemm(p, c, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "gemm launch");
}

size_t moe_wna16_dense_gemm_workspace_size(int M, int N, int K, const moe_quant_t* quant,
                                           int dtype) {
  if (M <= 0 || N <= 0 || K <= 0 || !quant || (quant->bits != 4 && quant->bits != 8)) return 0;
  return make_dense_plan(M, N, K, quant->bits, dtype).ws;
}

int moe_wna16_dense_gemm(const void* A, int M, int K, const void* B, const void* scales,
                         const void* zeros, const moe_quant_t* quant, int N, int dtype,
                         void* workspace, size_t workspace_bytes, void* C, void* stream) {
  if (int rc = check_dtype(dtype)) return rc;
  if (int rc = check_quant(quant)) return rc;
  if (M < 0 || N <= 0 || K <= 0) return fail(MOE_ERR_INVALID_ARG, "M=%d N=%d K=%d", M, N, K);
  if (K % 256) return fail(MOE_ERR_UNSUPPORTED, "K = %d must be a multiple of 256", K);
  if (N % 128) return fail(MOE_ERR_UNSUPPORTED, "N = %d must be a multiple of 128", N);
  if ((int64_t)M * K * 2 >= ((int64_t)1 << 31) ||
      (int64_t)N * (quant->bits == 4 ? K / 2 : K) >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "A or the weights exceed 2 GiB");
  if (int rc = check_weights(B, scales, zeros, quant)) return rc;
  if (M == 0) return MOE_OK;
  if (!A || !C) return fail(MOE_ERR_INVALID_ARG, "NULL A / C");
  if (!aligned(A, 16) || !aligned(C, 16))
    return fail(MOE_ERR_INVALID_ARG, "A and C must be 16-byte aligned");
  DensePlan d = make_dense_plan(M, N, K, quant->bits, dtype);
  if (workspace_bytes < d.ws)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, d.ws);
  if (d.ws && (!workspace || !aligned(workspace, 256)))
    return fail(MOE_ERR_INVALID_ARG, "workspace must be a 256-byte aligned device buffer");
  if (int rc = fit_lds(K, d.split, d.c, "dense gemm")) return rc;
  moe::GemmParams p{};
  p.A = A;
  p.num_a_rows = M;
  p.a_row_div = 1;
  p.B = (const uint8_t*)B;
  p.scales = scales;
  p.zeros = (const uint8_t*)zeros;
  p.E = 1;
  p.N = N;
  p.K = K;
  p.num_blocks = d.nblk;
  p.num_slots = M;
  p.C = d.split > 1 ? workspace : C;
  p.split_k = d.split;
  p.dense = 1;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = moe::launch_gemm(p, d.c, st);
  if (e != hipSuccess) return hip_fail(e, "dense gemm launch");
  if (d.split > 1) {
    e = moe::launch_split_reduce((const float*)workspace, d.split, M, N, dtype, C, st);
    if (e != hipSuccess) return hip_fail(e, "dense split reduce launch");
  }
  return MOE_OK;
}

int moe_wna16_batched_gemm(const void* A, int E, int max_tokens, int K,
                           const int32_t* expert_num_tokens, const void* B, const void* scales,
                           const void* zeros, const moe_quant_t* quant, int N, int dtype,
                           int block_m, int act, void* C, void* stream) {
  if (int rc = check_dtype(dtype)) return rc;
  if (int rc = check_quant(quant)) return rc;
  if (E <= 0 || max_tokens < 0 || K <= 0 || N <= 0)
    return fail(MOE_ERR_INVALID_ARG, "E=%d max_tokens=%d K=%d N=%d", E, max_tokens, K, N);
  if (E > 1024) return fail(MOE_ERR_UNSUPPORTED, "E = %d > 1024", E);
  if (act != MOE_ACT_NONE && act != MOE_ACT_SILU_MUL)
    return fail(MOE_ERR_INVALID_ARG, "act = %d", act);
  if (block_m != 0 && !valid_block_m(block_m))
    return fail(MOE_ERR_UNSUPPORTED, "block_m = %d (supported: 0, 16, 32, 64, 128)", block_m);
  if (K % 256) return fail(MOE_ERR_UNSUPPORTED, "K = %d must be a multiple of 256", K);
  if (N % 128) return fail(MOE_ERR_UNSUPPORTED, "N = %d must be a multiple of 128", N);
  const int64_t rows = (int64_t)E * max_tokens;
  // 32-bit buffer offsets: A and one expert's weights (C is written with 64-bit addresses)
  if (rows * K * 2 >= ((int64_t)1 << 31) ||
      (int64_t)N * (quant->bits == 4 ? K / 2 : K) >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "A or one expert's weights exceed 2 GiB");
  if (int rc = check_weights(B, scales, zeros, quant)) return rc;
  if (max_tokens == 0) return MOE_OK;
  if (!A || !C || !expert_num_tokens) return fail(MOE_ERR_INVALID_ARG, "NULL A / C / counts");
  if (!aligned(A, 16) || !aligned(C, 16) || !aligned(expert_num_tokens, 4))
    return fail(MOE_ERR_INVALID_ARG, "A and C need 16-byte, counts 4-byte alignment");
  // rows per block: the smallest of {16, 32, 64} (int8: 128) that holds a full batch, so an expert
  // with a full batch streams its weights once
  int bm = block_m;
  if (bm == 0) {
    bm = 16;
    const int top = quant->bits == 4 ? 64 : 128;
    while (bm < max_tokens && bm < top) bm *= 2;
  }
  const int bpe = (max_tokens + bm - 1) / bm;
  const int64_t nblk = (int64_t)E * bpe;
  const int ntw = pick_ntw(act, N, bm, nblk);
  moe::GemmConfig c{dtype, quant->bits, bm, act, 0, ntw,
                    pick_waves(act, N, bm, ntw, dtype, quant->bits)};
  if (int rc = fit_lds(K, 1, c, "batched gemm")) return rc;
  moe::GemmParams p{};
  p.A = A;
  p.num_a_rows = (int)rows;
  p.a_row_div = 1;
  p.B = (const uint8_t*)B;
  p.scales = scales;
  p.zeros = (const uint8_t*)zeros;
  p.E = E;
  p.N = N;
  p.K = K;
  p.num_blocks = (int)nblk;
  p.num_slots = (int)rows;
  p.C = C;
  p.split_k = 1;
  p.batched = 1;
  p.expert_counts = expert_num_tokens;
  p.max_tokens = max_tokens;
  p.bpe = bpe;
  hipError_t e = moe::launch_gemm(p, c, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "batched gemm launch");
}

int moe_quant_int8_rows(const void* x, int rows, int K, int dtype, int8_t* q, float* scales,
                        void* stream) {
  if (int rc = check_dtype(dtype)) return rc;
  if (rows < 0 || K <= 0) return fail(MOE_ERR_INVALID_ARG, "rows=%d K=%d", rows, K);
  if (K % 256) return fail(MOE_ERR_UNSUPPORTED, "K = %d must be a multiple of 256", K);
  if ((int64_t)rows * K * 2 >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "x exceeds 2 GiB");
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scales) return fail(MOE_ERR_INVALID_ARG, "NULL x / q / scales");
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4))
    return fail(MOE_ERR_INVALID_ARG, "x and q need 16-byte, scales 4-byte alignment");
  hipError_t e = moe::launch_quant_rows(x, rows, K, dtype, q, scales, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "quant launch");
}

int moe_w8a8_gemm(const int8_t* A, const float* a_scales, int num_a_rows, int a_row_div,
                  const int8_t* B, const void* w_scales, int E, int N, int K, int dtype,
                  const int32_t* sorted_token_ids, const int32_t* expert_ids,
                  const int32_t* num_tokens_post_padded, int64_t capacity, int block_m,
                  int num_slots, const float* topk_weights, int act, void* C, void* stream) {
  if (int rc = check_dtype(dtype)) return rc;
  if (E <= 0 || N <= 0 || K <= 0 || num_a_rows < 0 || a_row_div <= 0 || num_slots < 0 ||
      capacity < 0)
    return fail(MOE_ERR_INVALID_ARG, "E=%d N=%d K=%d rows=%d a_row_div=%d slots=%d", E, N, K,
                num_a_rows, a_row_div, num_slots);
  if (act != MOE_ACT_NONE && act != MOE_ACT_SILU_MUL)
    return fail(MOE_ERR_INVALID_ARG, "act = %d", act);
  if (!valid_block_m(block_m) && !(block_m == 256 && moe::w8a8_mma32_fits(256, act, N)))
    return fail(MOE_ERR_UNSUPPORTED,
                "block_m = %d (supported: 16, 32, 64, 128; 256 where N / 2 (act) or N is a "
                "multiple of 128 or 256)", block_m);
  if (K % 256) return fail(MOE_ERR_UNSUPPORTED, "K = %d must be a multiple of 256", K);
  if (N % 128) return fail(MOE_ERR_UNSUPPORTED, "N = %d must be a multiple of 128", N);
  if ((int64_t)num_a_rows * K >= ((int64_t)1 << 31) || (int64_t)N * K >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "A or one expert's weights exceed 2 GiB");
  // int32 accumulation of products of codes in [-127, 127]: 127^2 * K stays below 2^31
  if (K > kW8A8MaxK) return fail(MOE_ERR_UNSUPPORTED, "K = %d > %d (int32 sums)", K, kW8A8MaxK);
  if ((int64_t)num_a_rows * a_row_div < num_slots)
    return fail(MOE_ERR_INVALID_ARG, "A has %d rows, slots need %lld", num_a_rows,
                (long long)((num_slots + a_row_div - 1) / a_row_div));
  if (num_slots == 0) return MOE_OK;  // nothing to read or write
  if (!A || !a_scales || !B || !w_scales || !C || !sorted_token_ids || !expert_ids ||
      !num_tokens_post_padded)
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(a_scales, 4) ||
      !aligned(w_scales, 2))
    return fail(MOE_ERR_INVALID_ARG, "A, B and C need 16-byte alignment");
  if (topk_weights && !aligned(topk_weights, 4))
    return fail(MOE_ERR_INVALID_ARG, "topk_weights must be 4-byte aligned");
  if (num_slots == 0 || capacity == 0) return MOE_OK;
  moe::W8A8Params p{};
  p.A = A;
  p.a_scales = a_scales;
  p.num_a_rows = num_a_rows;
  p.a_row_div = a_row_div;
  p.B = B;
  p.w_scales = w_scales;
  p.E = E;
  p.N = N;
  p.K = K;
  p.sorted_ids = sorted_token_ids;
  p.expert_ids = expert_ids;
  p.num_post = num_tokens_post_padded;
  p.num_blocks = (int)(capacity / block_m);
  p.num_slots = num_slots;
  p.topk_w = topk_weights;
  p.C = C;
  hipError_t e = moe::launch_w8a8_gemm(p, block_m, act, dtype, (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "w8a8 gemm launch");
}

// ------------------------------------------------------------------------------------------------
// the fused w8a8 layer
// ------------------------------------------------------------------------------------------------
namespace {
struct PlanW8 {
  int bm;
  int64_t cap;
  size_t off_w, off_ids, off_sorted, off_eids, off_npost, off_xq, off_xs, off_inter, off_iq, off_is,
      off_y, total;
};
// 256-row blocks for both w8a8 GEMMs: the 32x32 integer kernel with one column tile per wavefront
bool w8a8_fits_256(int H, int I) {
  return moe::w8a8_mma32_fits(256, 1, 2 * I) && moe::w8a8_mma32_fits(256, 0, H);
}

PlanW8 make_plan_w8(int M, int H, int I, int E, int topk, int dtype, int block_m) {
  PlanW8 p{};
  const int64_t slots = (int64_t)M * topk;
  // the int8 block-size rule; 256 rows (a whole expert's slots: each weight read once, where 128
  // rows read about half the experts' weights twice) where both GEMMs take them, else 128
  p.bm = block_m > 0 ? block_m : pick_block_m(M, topk, E, 8, dtype);
  if (block_m == 0 && p.bm == 256 && !w8a8_fits_256(H, I)) p.bm = 128;
  p.cap = align_capacity(slots, E, p.bm);
  const int64_t nblk = (p.cap + p.bm - 1) / p.bm;
  size_t off = 0;
  p.off_w = off;      off += up256((size_t)slots * 4);
  p.off_ids = off;    off += up256((size_t)slots * 4);
  p.off_sorted = off; off += up256((size_t)p.cap * 4);
  p.off_eids = off;   off += up256((size_t)nblk * 4);
  p.off_npost = off;  off += 256;
  p.off_xq = off;     off += up256((size_t)M * H);
  p.off_xs = off;     off += up256((size_t)M * 4);
  p.off_inter = off;  off += up256((size_t)slots * I * 2);
  p.off_iq = off;     off += up256((size_t)slots * I);
  p.off_is = off;     off += up256((size_t)slots * 4);
  p.off_y = off;      off += up256((size_t)slots * H * 4);
  p.total = off;
  return p;
}
}  // namespace

size_t fused_moe_w8a8_workspace_size(int M, int H, int I, int E, int topk, int dtype, int block_m) {
  if (M < 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0) return 0;
  if (block_m != 0 && !valid_block_m(block_m) && !(block_m == 256 && w8a8_fits_256(H, I))) return 0;
  return make_plan_w8(M, H, I, E, topk, dtype, block_m).total;
}

int fused_moe_w8a8(const void* x, const float* router_logits, int M, int H, int I, int E, int topk,
                   const moe_routing_t* routing, const int8_t* w13, const void* w13_scales,
                   const int8_t* w2, const void* w2_scales, int dtype, int block_m,
                   void* workspace, size_t workspace_bytes, void* out, float* topk_weights_out,
                   int32_t* topk_ids_out, void* stream) {
  if (int rc = check_dtype(dtype)) return rc;
  if (M < 0 || H <= 0 || I <= 0) return fail(MOE_ERR_INVALID_ARG, "M=%d H=%d I=%d", M, H, I);
  if (int rc = check_routing(routing, E, topk)) return rc;
  if (H % 256 || I % 256)
    return fail(MOE_ERR_UNSUPPORTED, "H = %d and I = %d must be multiples of 256", H, I);
  if (block_m != 0 && !valid_block_m(block_m) && !(block_m == 256 && w8a8_fits_256(H, I)))
    return fail(MOE_ERR_UNSUPPORTED, "block_m = %d (supported: 0, 16, 32, 64, 128, 256)", block_m);
  if (H > kW8A8MaxK || I > kW8A8MaxK)
    return fail(MOE_ERR_UNSUPPORTED, "H = %d or I = %d > %d (int32 sums)", H, I, kW8A8MaxK);
  if ((int64_t)M * topk > (1 << 24)) return fail(MOE_ERR_UNSUPPORTED, "M * topk > 2^24");
  // 32-bit buffer offsets: the int8 activations of either GEMM, one expert's weights (the rows the
  // second GEMM writes and the combine reads use 64-bit addresses)
  if ((int64_t)M * H >= ((int64_t)1 << 31) || (int64_t)M * topk * I >= ((int64_t)1 << 31) ||
      (int64_t)2 * I * H >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "int8 activations or one expert's weights exceed 2 GiB");
  if (M == 0) return MOE_OK;
  if (!x || !router_logits || !out || !workspace || !w13 || !w13_scales || !w2 || !w2_scales)
    return fail(MOE_ERR_INVALID_ARG, "NULL pointer argument");
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, 256) ||
      !aligned(router_logits, 4) || !aligned(w13, 16) || !aligned(w2, 16) ||
      !aligned(w13_scales, 2) || !aligned(w2_scales, 2))
    return fail(MOE_ERR_INVALID_ARG, "misaligned pointer argument");
  if ((topk_weights_out && !aligned(topk_weights_out, 4)) ||
      (topk_ids_out && !aligned(topk_ids_out, 4)))
    return fail(MOE_ERR_INVALID_ARG, "routing outputs must be 4-byte aligned");
  const PlanW8 pl = make_plan_w8(M, H, I, E, topk, dtype, block_m);
  if (workspace_bytes < pl.total)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, pl.total);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* tw = topk_weights_out ? topk_weights_out : (float*)(ws + pl.off_w);
  int32_t* ids = topk_ids_out ? topk_ids_out : (int32_t*)(ws + pl.off_ids);
  int32_t* sorted = (int32_t*)(ws + pl.off_sorted);
  int32_t* eids = (int32_t*)(ws + pl.off_eids);
  int32_t* npost = (int32_t*)(ws + pl.off_npost);
  int8_t* xq = (int8_t*)(ws + pl.off_xq);
  float* xs = (float*)(ws + pl.off_xs);
  void* inter = ws + pl.off_inter;
  int8_t* iq = (int8_t*)(ws + pl.off_iq);
  float* is = (float*)(ws + pl.off_is);
  float* y = (float*)(ws + pl.off_y);
  const int slots = M * topk;

  const moe::RoutingParams rp{routing->score, routing->renormalize, routing->num_groups,
                              routing->topk_groups, routing->scale};
  hipError_t e;
  if (moe::route_align_fits(M, E)) {
    e = moe::launch_route_align(router_logits, M, E, topk, rp, tw, ids, pl.bm, sorted, eids, npost,
                                pl.cap, st);
    if (e != hipSuccess) return hip_fail(e, "routing + align launch");
  } else {
    e = moe::launch_routing(router_logits, M, E, topk, rp, tw, ids, st);
    if (e != hipSuccess) return hip_fail(e, "routing launch");
    // many slots: the many-workgroup align, its counts in the float32 row buffer (not yet in use)
    if (moe::align_multi_pays(slots) &&
        moe::align_multi_scratch_bytes(slots, E) <= pl.total - pl.off_y)
      e = moe::launch_align_multi(ids, slots, E, pl.bm, sorted, eids, npost, pl.cap,
                                  (int32_t*)(ws + pl.off_y), st);
    else
      e = moe::launch_align(ids, slots, E, pl.bm, sorted, eids, npost, pl.cap, st);
    if (e != hipSuccess) return hip_fail(e, "align launch");
  }
  e = moe::launch_quant_rows(x, M, H, dtype, xq, xs, st);
  if (e != hipSuccess) return hip_fail(e, "quant launch");
  moe::W8A8Params g1{};
  g1.A = xq;
  g1.a_scales = xs;
  g1.num_a_rows = M;
  g1.a_row_div = topk;
  g1.B = w13;
  g1.w_scales = w13_scales;
  g1.E = E;
  g1.N = 2 * I;
  g1.K = H;
  g1.sorted_ids = sorted;
  g1.expert_ids = eids;
  g1.num_post = npost;
  g1.num_blocks = (int)(pl.cap / pl.bm);
  g1.num_slots = slots;
  g1.C = inter;
  e = moe::launch_w8a8_gemm(g1, pl.bm, 1, dtype, st);
  if (e != hipSuccess) return hip_fail(e, "w8a8 gemm1 launch");
  e = moe::launch_quant_rows(inter, slots, I, dtype, iq, is, st);
  if (e != hipSuccess) return hip_fail(e, "quant launch");
  moe::W8A8Params g2 = g1;
  g2.A = iq;
  g2.a_scales = is;
  g2.num_a_rows = slots;
  g2.a_row_div = 1;
  g2.B = w2;
  g2.w_scales = w2_scales;
  g2.N = H;
  g2.K = I;
  g2.C = y;
  e = moe::launch_w8a8_gemm(g2, pl.bm, 0, dtype, st, 1);
  if (e != hipSuccess) return hip_fail(e, "w8a8 gemm2 launch");
  e = moe::launch_combine(y, 1, tw, M, topk, H, dtype, out, st);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return MOE_OK;
}

int moe_repack_uint4(int format, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                     const int32_t* g_idx, int E, int N, int K, int dtype, uint8_t* B,
                     void* scales_out, uint8_t* zeros_out, int32_t* perm_out,
                     int32_t* invalid_out, void* stream) {
  if (format != MOE_FORMAT_GPTQ && format != MOE_FORMAT_AWQ)
    return fail(MOE_ERR_INVALID_ARG, "format = %d (0 GPTQ, 1 AWQ)", format);
  if (int rc = check_dtype(dtype)) return rc;
  if (E <= 0 || N <= 0 || K <= 0) return fail(MOE_ERR_INVALID_ARG, "E=%d N=%d K=%d", E, N, K);
  if (K % 256) return fail(MOE_ERR_UNSUPPORTED, "K = %d must be a multiple of 256", K);
  if (N % 8) return fail(MOE_ERR_UNSUPPORTED, "N = %d must be a multiple of 8", N);
  if (format == MOE_FORMAT_AWQ && g_idx)
    return fail(MOE_ERR_UNSUPPORTED, "AWQ checkpoints carry no g_idx (act-order is GPTQ's)");
  if ((g_idx == nullptr) != (perm_out == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "g_idx and perm_out go together (both or neither)");
  if (g_idx && K > 16384)
    return fail(MOE_ERR_UNSUPPORTED, "act-order repack: K = %d > 16384 (group ids staged in LDS)", K);
  if (!qweight || !qzeros || !scales || !B || !scales_out || !zeros_out)
    return fail(MOE_ERR_INVALID_ARG, "NULL checkpoint or output pointer");
  if (!aligned(qweight, 4) || !aligned(qzeros, 4) || !aligned(scales, 2) || !aligned(B, 16) ||
      !aligned(scales_out, 4) || !aligned(zeros_out, 2) || (g_idx && !aligned(g_idx, 4)) ||
      (perm_out && !aligned(perm_out, 4)) || (invalid_out && !aligned(invalid_out, 4)))
    return fail(MOE_ERR_INVALID_ARG, "misaligned pointer argument");
  hipError_t e = moe::launch_repack_uint4(format, qweight, qzeros, scales, g_idx, E, N, K, B,
                                          scales_out, zeros_out, perm_out, invalid_out,
                                          (hipStream_t)stream);
  return e == hipSuccess ? MOE_OK : hip_fail(e, "repack launch");
}

size_t fused_moe_wna16_workspace_size(int M, int H, int I, int E, int topk,
                                      const moe_quant_t* quant, int dtype, int block_m) {
  if (M < 0 || H <= 0 || I <= 0 || E <= 0 || topk <= 0 || !quant) return 0;
  if (block_m != 0 && !valid_block_m_wna16(block_m)) return 0;
  return make_plan(M, H, I, E, topk, quant->bits, dtype, block_m).total;
}

}  // extern "C"

namespace {

// Extra workspace of the act-order layer: each slot's activation row gathered through its expert's
// input-column permutation, for both GEMMs.
size_t act_order_bytes(int M, int H, int I, int topk) {
  return up256((size_t)M * topk * H * 2) + up256((size_t)M * topk * I * 2);
}

// The fused layer; w13_perm / w2_perm non-NULL: act-order experts (the activation rows are
// gathered per slot through the expert's permutation before each GEMM).
int fused_impl(const void* x, const float* router_logits, int M, int H, int I, int E, int topk,
               const moe_routing_t* routing, const void* w13, const void* w13_scales,
               const void* w13_zeros, const void* w2, const void* w2_scales, const void* w2_zeros,
               const moe_quant_t* quant, int dtype, int block_m, void* workspace,
               size_t workspace_bytes, void* out, float* topk_weights_out, int32_t* topk_ids_out,
               const int32_t* w13_perm, const int32_t* w2_perm, void* stream) {
  if (int rc = check_dtype(dtype)) return rc;
  if (int rc = check_quant(quant)) return rc;
  if (M < 0 || H <= 0 || I <= 0) return fail(MOE_ERR_INVALID_ARG, "M=%d H=%d I=%d", M, H, I);
  if (int rc = check_routing(routing, E, topk)) return rc;
  if (block_m != 0 && !valid_block_m_wna16(block_m))
    return fail(MOE_ERR_UNSUPPORTED, "block_m = %d (supported: 0, 16, 32, 64, 128, 256)", block_m);
  if (H % 256 || I % 256)
    return fail(MOE_ERR_UNSUPPORTED, "H = %d and I = %d must be multiples of 256", H, I);
  if ((int64_t)M * topk > (1 << 24)) return fail(MOE_ERR_UNSUPPORTED, "M * topk > 2^24");
  if ((int64_t)M * topk * I * 2 >= ((int64_t)1 << 31) || (int64_t)M * H * 2 >= ((int64_t)1 << 31) ||
      (int64_t)2 * I * (quant->bits == 4 ? H / 2 : H) >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "activations or one expert's weights exceed 2 GiB");
  // act-order: the first GEMM reads the gathered rows [M * topk, H] instead of x
  if (w13_perm && (int64_t)M * topk * H * 2 >= ((int64_t)1 << 31))
    return fail(MOE_ERR_UNSUPPORTED, "gathered activation rows (M * topk * H) exceed 2 GiB");
  if (M == 0) return MOE_OK;
  if (int rc = check_weights(w13, w13_scales, w13_zeros, quant)) return rc;
  if (int rc = check_weights(w2, w2_scales, w2_zeros, quant)) return rc;
  if (!x || !router_logits || !out || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "NULL x / router_logits / out / workspace");
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, 256) || !aligned(router_logits, 4))
    return fail(MOE_ERR_INVALID_ARG, "x/out need 16-byte, workspace 256-byte alignment");
  if ((topk_weights_out && !aligned(topk_weights_out, 4)) ||
      (topk_ids_out && !aligned(topk_ids_out, 4)))
    return fail(MOE_ERR_INVALID_ARG, "routing outputs must be 4-byte aligned");
  const Plan pl = make_plan(M, H, I, E, topk, quant->bits, dtype, block_m);
  const bool act_order = w13_perm != nullptr;
  const size_t need = pl.total + (act_order ? act_order_bytes(M, H, I, topk) : 0);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* tw = topk_weights_out ? topk_weights_out : (float*)(ws + pl.off_w);
  int32_t* ids = topk_ids_out ? topk_ids_out : (int32_t*)(ws + pl.off_ids);
  void* inter = ws + pl.off_inter;
  const moe::RoutingParams rp{routing->score, routing->renormalize, routing->num_groups,
                              routing->topk_groups, routing->scale};
  hipError_t e;

  const int path = layer_path(M, H, I, E, topk, quant->bits, block_m, act_order);
  // one token: one dot product per weight row in two launches (gemv.hip), the routing inside the
  // first, the top-k combine inside the second
  if (path == MOE_PATH_ONE_TOKEN) {
    moe::SingleParams sp{};
    sp.x = x;
    sp.logits = router_logits;
    sp.rp = rp;
    sp.topk_ids = ids;
    sp.topk_w = tw;
    sp.w13 = (const uint8_t*)w13;
    sp.s13 = w13_scales;
    sp.z13 = (const uint8_t*)w13_zeros;
    sp.w2 = (const uint8_t*)w2;
    sp.s2 = w2_scales;
    sp.z2 = (const uint8_t*)w2_zeros;
    sp.E = E;
    sp.H = H;
    sp.I = I;
    sp.topk = topk;
    sp.inter = inter;
    sp.out = out;
    e = moe::launch_single(sp, dtype, st);
    if (e != hipSuccess) return hip_fail(e, "single-token launch");
    return MOE_OK;
  }

  // a few tokens: routing, then the two dot-product launches, each grouping the slots by expert
  if (path == MOE_PATH_FEW_TOKENS) {
    e = moe::launch_routing(router_logits, M, E, topk, rp, tw, ids, st);
    if (e != hipSuccess) return hip_fail(e, "routing launch");
    moe::SingleParams sp{};
    sp.x = x;
    sp.topk_ids = ids;
    sp.topk_w = tw;
    sp.w13 = (const uint8_t*)w13;
    sp.s13 = w13_scales;
    sp.z13 = (const uint8_t*)w13_zeros;
    sp.w2 = (const uint8_t*)w2;
    sp.s2 = w2_scales;
    sp.z2 = (const uint8_t*)w2_zeros;
    sp.E = E;
    sp.H = H;
    sp.I = I;
    sp.topk = topk;
    sp.M = M;
    sp.inter = inter;
    sp.out = out;
    e = moe::launch_few(sp, dtype, st);
    if (e != hipSuccess) return hip_fail(e, "few-token launch");
    return MOE_OK;
  }

  const bool split1 = pl.split1 > 1;
  // split: plain columns (gate rows, then up rows) into float32 partials, 2 column tiles per
  // wavefront so the workgroup count matches the estimate the split was chosen for
  moe::GemmConfig c1{dtype, quant->bits, pl.bm, split1 ? 0 : 1, split1 ? 1 : 0,
                     split1 ? 2 : pl.ntw1, split1 ? 4 : pl.wv1};
  // second GEMM unsplit with 64-row blocks: rows weighted in its epilogue and written in the
  // activation dtype, half the bytes of float32 rows for the combine to read back (DeepSeek-V3
  // prefill at 1024 tokens: layer -1.2 to -1.6 %, same box, same process).  Not with 128-row
  // blocks, whose 32x32 result layout leaves each lane one 2-byte column per row: there the
  // half-line writes cost more than the bytes saved (4096 tokens: +1 to +3 %).
  const bool rows2 = pl.split2 == 1 && pl.bm == 64;
  moe::GemmConfig c2{dtype, quant->bits, pl.bm, 0, rows2 ? 0 : 1, pl.ntw2, pl.wv2};
  c2.cgroup = pick_cgroup(c2, H, I, pl.split2, estimate_active_blocks(M, topk, E, pl.bm));
  if (int rc = fit_lds(H, pl.split1, c1, "gemm1")) return rc;
  if (int rc = fit_lds(I, pl.split2, c2, "gemm2")) return rc;

  int32_t* sorted = (int32_t*)(ws + pl.off_sorted);
  int32_t* eids = (int32_t*)(ws + pl.off_eids);
  int32_t* npost = (int32_t*)(ws + pl.off_npost);
  float* part = (float*)(ws + pl.off_part);
  const int slots = M * topk;

  if (moe::route_align_fits(M, E)) {
    e = moe::launch_route_align(router_logits, M, E, topk, rp, tw, ids, pl.bm, sorted, eids, npost,
                                pl.cap, st);
    if (e != hipSuccess) return hip_fail(e, "routing + align launch");
  } else {
    e = moe::launch_routing(router_logits, M, E, topk, rp, tw, ids, st);
    if (e != hipSuccess) return hip_fail(e, "routing launch");
    // many slots: the many-workgroup align, its counts in the float32 partial buffer (not yet in
    // use)
    if (moe::align_multi_pays(slots) &&
        moe::align_multi_scratch_bytes(slots, E) <= pl.total - pl.off_part)
      e = moe::launch_align_multi(ids, slots, E, pl.bm, sorted, eids, npost, pl.cap,
                                  (int32_t*)part, st);
    else
      e = moe::launch_align(ids, slots, E, pl.bm, sorted, eids, npost, pl.cap, st);
    if (e != hipSuccess) return hip_fail(e, "align launch");
  }

  // act-order: slot s reads x[s / topk] through its expert's permutation of the H input columns
  void* xa = act_order ? (void*)(ws + pl.total) : nullptr;
  void* ia = act_order ? (void*)(ws + pl.total + up256((size_t)M * topk * H * 2)) : nullptr;
  if (act_order) {
    e = moe::launch_gather_cols(x, topk, ids, E, w13_perm, H, slots, dtype, xa, st);
    if (e != hipSuccess) return hip_fail(e, "gather launch");
  }

  moe::GemmParams g1{};
  g1.A = act_order ? xa : x;
  g1.num_a_rows = act_order ? slots : M;
  g1.a_row_div = act_order ? 1 : topk;
  g1.B = (const uint8_t*)w13;
  g1.scales = w13_scales;
  g1.zeros = (const uint8_t*)w13_zeros;
  g1.E = E;
  g1.N = 2 * I;
  g1.K = H;
  g1.sorted_ids = sorted;
  g1.expert_ids = eids;
  g1.num_post = npost;
  g1.num_blocks = (int)(pl.cap / pl.bm);
  g1.num_slots = slots;
  g1.topk_w = nullptr;
  g1.C = split1 ? (void*)part : inter;
  g1.split_k = pl.split1;
  e = moe::launch_gemm(g1, c1, st);
  if (e != hipSuccess) return hip_fail(e, "gemm1 launch");
  if (split1) {
    e = moe::launch_act_combine(part, pl.split1, slots, I, dtype, inter, st);
    if (e != hipSuccess) return hip_fail(e, "gemm1 combine launch");
  }

  if (act_order) {
    e = moe::launch_gather_cols(inter, 1, ids, E, w2_perm, I, slots, dtype, ia, st);
    if (e != hipSuccess) return hip_fail(e, "gather launch");
  }

  moe::GemmParams g2 = g1;
  g2.A = act_order ? ia : inter;
  g2.num_a_rows = slots;
  g2.a_row_div = 1;
  g2.B = (const uint8_t*)w2;
  g2.scales = w2_scales;
  g2.zeros = (const uint8_t*)w2_zeros;
  g2.N = H;
  g2.K = I;
  g2.C = part;
  g2.split_k = pl.split2;
  g2.topk_w = rows2 ? tw : nullptr;
  e = moe::launch_gemm(g2, c2, st);
  if (e != hipSuccess) return hip_fail(e, "gemm2 launch");

  e = rows2 ? moe::launch_combine_rows(part, M, topk, H, dtype, out, st)
            : moe::launch_combine(part, pl.split2, tw, M, topk, H, dtype, out, st);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return MOE_OK;
}

}  // namespace

namespace moe {

int api_fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vfail(code, fmt, ap);
  va_end(ap);
  return code;
}

int fused_wna16(const void* x, const float* router_logits, int M, int H, int I, int E, int topk,
                const moe_routing_t* routing, const void* w13, const void* w13_scales,
                const void* w13_zeros, const void* w2, const void* w2_scales, const void* w2_zeros,
                const moe_quant_t* quant, int dtype, int block_m, void* workspace,
                size_t workspace_bytes, void* out, float* topk_weights_out, int32_t* topk_ids_out,
                void* stream) {
  return fused_impl(x, router_logits, M, H, I, E, topk, routing, w13, w13_scales, w13_zeros, w2,
                    w2_scales, w2_zeros, quant, dtype, block_m, workspace, workspace_bytes, out,
                    topk_weights_out, topk_ids_out, nullptr, nullptr, stream);
}

}  // namespace moe

extern "C" {

int fused_moe_wna16(const void* x, const float* router_logits, int M, int H, int I, int E, int topk,
                    const moe_routing_t* routing, const void* w13, const void* w13_scales,
                    const void* w13_zeros, const void* w2, const void* w2_scales,
                    const void* w2_zeros, const moe_quant_t* quant, int dtype, int block_m,
                    void* workspace, size_t workspace_bytes, void* out, float* topk_weights_out,
                    int32_t* topk_ids_out, void* stream) {
  return fused_impl(x, router_logits, M, H, I, E, topk, routing, w13, w13_scales, w13_zeros, w2,
                    w2_scales, w2_zeros, quant, dtype, block_m, workspace, workspace_bytes, out,
                    topk_weights_out, topk_ids_out, nullptr, nullptr, stream);
}

int fused_moe_wna16_path(int M, int H, int I, int E, int topk, const moe_quant_t* quant,
                         int block_m, int act_order) {
  if (M <= 0 || H <= 0 || I <= 0 || H % 256 || I % 256 || !quant) return -1;
  if (E <= 0 || E > 1024 || topk <= 0 || topk > E || topk > 32) return -1;
  if (quant->bits != 4 && quant->bits != 8) return -1;
  if (block_m != 0 && !valid_block_m_wna16(block_m)) return -1;
  return layer_path(M, H, I, E, topk, quant->bits, block_m, act_order != 0);
}

size_t fused_moe_wna16_act_order_workspace_size(int M, int H, int I, int E, int topk,
                                                int dtype, int block_m) {
  const moe_quant_t q{4, 128, 1};
  const size_t base = fused_moe_wna16_workspace_size(M, H, I, E, topk, &q, dtype, block_m);
  return base ? base + act_order_bytes(M, H, I, topk) : 0;
}

int fused_moe_wna16_act_order(const void* x, const float* router_logits, int M, int H, int I,
                              int E, int topk, const moe_routing_t* routing, const void* w13,
                              const void* w13_scales, const void* w13_zeros,
                              const int32_t* w13_perm, const void* w2, const void* w2_scales,
                              const void* w2_zeros, const int32_t* w2_perm, int dtype,
                              int block_m, void* workspace, size_t workspace_bytes, void* out,
                              float* topk_weights_out, int32_t* topk_ids_out, void* stream) {
  if (!w13_perm || !w2_perm) return fail(MOE_ERR_INVALID_ARG, "NULL permutation");
  if (!aligned(w13_perm, 4) || !aligned(w2_perm, 4))
    return fail(MOE_ERR_INVALID_ARG, "permutations must be 4-byte aligned");
  const moe_quant_t q{4, 128, 1};
  return fused_impl(x, router_logits, M, H, I, E, topk, routing, w13, w13_scales, w13_zeros, w2,
                    w2_scales, w2_zeros, &q, dtype, block_m, workspace, workspace_bytes, out,
                    topk_weights_out, topk_ids_out, w13_perm, w2_perm, stream);
}

}  // extern "C"
