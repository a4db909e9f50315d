// Host-side pieces of the C ABI shared between its translation units (api.cpp and noalloc.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "moe_wna16.h"

namespace moe {

// Records the message for moe_last_error() on the calling thread and returns code.
int api_fail(int code, const char* fmt, ...);

// fused_moe_wna16 with its argument checks, on a workspace the caller supplies.
int fused_wna16(const void* x, const float* router_logits, int M, int H, int I, int E, int topk,
                const moe_routing_t* routing, const void* w13, const void* w13_scales,
                const void* w13_zeros, const void* w2, const void* w2_scales, const void* w2_zeros,
                const moe_quant_t* quant, int dtype, int block_m, void* workspace,
                size_t workspace_bytes, void* out, float* topk_weights_out, int32_t* topk_ids_out,
                void* stream);

}  // namespace moe
