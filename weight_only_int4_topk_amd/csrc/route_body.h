// Top-k routing of one token, on one 64-lane wavefront (route_token: topk rounds of a wavefront-wide
// arg-best) or on a workgroup of 256 threads (route_single: each candidate ranked by 64-bit order
// keys), shared by the routing launches and the single-token layer; both give the same ids and
// weights.
//
// Softmax rule: ids are the topk largest logits (ties to the lower expert id); ranking logits ranks
// softmax probabilities without any rounding, so ids are exact.  Sigmoid rule (DeepSeek-V3 style):
// scores s = 1/(1+e^-x) computed with a fully specified float32 exp so that every IEEE-754
// implementation gets the same bits, group score = sum of the two largest s of a contiguous group,
// keep topk_groups groups, then the topk largest s inside them.  The pages do not describe the
// routing; this is the rule of the Mixtral-, Qwen2- and DeepSeek-V3-shaped layers the library serves.
#pragma once

#include "common.h"
#include "launch.h"

namespace moe {
namespace {

// e^x in float32: clamp to [-80, 80]; n = rint(x * log2 e); r = (x - n*C1) - n*C2 with
// C1 = 355/512 (exact, so n*C1 is exact) and C2 = ln 2 - C1 rounded to float32 (Cody & Waite's
// two-constant reduction); p = Taylor polynomial of degree 7 in Horner form with coefficients 1/i!
// rounded to float32; result p * 2^n.  Each operation is a separately rounded float32 operation.
__device__ float exp_spec(float x) {
#pragma clang fp contract(off)
  const float kLog2e = 0x1.715476p+0f;
  const float kC1 = 0x1.63p-1f;
  const float kC2 = -0x1.bd0106p-13f;
  x = fminf(fmaxf(x, -80.0f), 80.0f);
  const float n = __builtin_rintf(x * kLog2e);
  const float r = (x - n * kC1) - n * kC2;
  float p = 0x1.a01a02p-13f;   // 1/7!
  p = p * r + 0x1.6c16c2p-10f; // 1/6!
  p = p * r + 0x1.111112p-7f;  // 1/5!
  p = p * r + 0x1.555556p-5f;  // 1/4!
  p = p * r + 0x1.555556p-3f;  // 1/3!
  p = p * r + 0x1.0p-1f;       // 1/2!
  p = p * r + 1.0f;            // 1/1!
  p = p * r + 1.0f;            // 1/0!
  return ldexpf(p, (int)n);
}

__device__ float sigmoid_spec(float x) {
#pragma clang fp contract(off)
  const float e = exp_spec(-x);
  return 1.0f / (1.0f + e);  // correctly rounded division (HIP default)
}

// Merge (t1 >= t2) with the partner lane's pair into the two largest of the four values.
__device__ __forceinline__ void top2_merge(float& t1, float& t2, float o1, float o2) {
  const float n2 = fmaxf(fminf(t1, o1), fmaxf(t2, o2));
  t1 = fmaxf(t1, o1);
  t2 = n2;
}
template <int CTRL>
__device__ __forceinline__ void top2_step(float& t1, float& t2) {
  top2_merge(t1, t2, dpp_f<CTRL>(t1), dpp_f<CTRL>(t2));
}

// One token on one wavefront: row = its E logits, sc = this wave's LDS scratch (EPL * 64 floats,
// used by the general group-limited rule), w_out / ids_out = its topk outputs; ids_lds (nullable)
// receives a copy of the ids.
template <int EPL>
__device__ void route_token(const float* __restrict__ row, int E, int topk, const RoutingParams& p,
                            float* sc, float* __restrict__ w_out, int32_t* __restrict__ ids_out,
                            int32_t* ids_lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const float kNone = -__builtin_inff();

  // expert e = lane + 64*i lives in v[i]
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    v[i] = e < E ? row[e] : kNone;
  }

  uint32_t taken[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) taken[i] = 0;
  // lane j (< topk) keeps the j-th winner; every lane sees every winner through the reduction
  float my_val = 0.0f;
  int my_id = 0;
  float denom = 0.0f;

  if (p.score == 0) {
    // softmax: rank raw logits; the first winner is the maximum logit
    float mx = 0.0f;
    for (int j = 0; j < topk; ++j) {
      float bv = kNone;
      int bi = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        if (e < E && !taken[i] && better(v[i], e, bv, bi)) {
          bv = v[i];
          bi = e;
        }
      }
      wave_argbest(bv, bi);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i == bi) taken[i] = 1;
      if (j == 0) mx = bv;
      const float ej = expf(bv - mx);
      denom += ej;
      if (lane == j) {
        my_val = ej;
        my_id = bi;
      }
    }
    if (!p.renormalize) {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (lane + kWave * i < E) part += expf(v[i] - mx);
      denom = wave_sum(part);
    }
    if (lane < topk) {
      w_out[lane] = my_val / denom * p.scale;
      ids_out[lane] = my_id;
      if (ids_lds) ids_lds[lane] = my_id;
    }
    return;
  }

  // sigmoid scores (exact spec)
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + kWave * i < E) v[i] = sigmoid_spec(v[i]);

  const int ng = p.num_groups;
  const int gs = E / ng;
  uint64_t kept = ~0ull;
  if (EPL == 4 && E == 256 && ng == 8 && p.topk_groups < ng) {
    // 8 groups of 32 (the DeepSeek-V3 layout): group 2i + h holds the experts of v[i] in half h
    // of the wave, so a butterfly inside each half (DPP in rows, a row swap across them) leaves
    // every lane with the two largest scores of its half's four groups; one half swap then gives
    // every lane all eight group scores, which it ranks by itself (ties -> lower group id).
    float gsc[8];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      float t1 = v[i], t2 = kNone;
      top2_step<kDppXor1>(t1, t2);
      top2_step<kDppXor2>(t1, t2);
      top2_step<kDppHalfMirror>(t1, t2);
      top2_step<kDppMirror>(t1, t2);
      uint32_t a1, b1, a2, b2;
      swap_pair<false>(__float_as_uint(t1), a1, b1);
      swap_pair<false>(__float_as_uint(t2), a2, b2);
      t1 = __uint_as_float(a1);
      t2 = __uint_as_float(a2);
      top2_merge(t1, t2, __uint_as_float(b1), __uint_as_float(b2));
      uint32_t lo, hi;
      swap_pair<true>(__float_as_uint(t1 + t2), lo, hi);
      gsc[2 * i] = __uint_as_float(lo);
      gsc[2 * i + 1] = __uint_as_float(hi);
    }
    kept = 0;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      int rank = 0;
#pragma unroll
      for (int o = 0; o < 8; ++o) rank += (o != g && better(gsc[o], o, gsc[g], g)) ? 1 : 0;
      if (rank < p.topk_groups) kept |= 1ull << g;
    }
  } else if (p.topk_groups < ng) {
    // publish scores to LDS; lane g < ng scores group g by the sum of its two largest values
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E) sc[e] = v[i];
    }
    __builtin_amdgcn_wave_barrier();  // a wave's LDS accesses complete in program order
    float gscore = kNone;
    if (lane < ng) {
      float b1 = kNone, b2 = kNone;
#pragma unroll 8
      for (int t = 0; t < gs; ++t) {
        const float s = sc[lane * gs + t];
        if (s > b1) {
          b2 = b1;
          b1 = s;
        } else if (s > b2) {
          b2 = s;
        }
      }
      gscore = gs >= 2 ? b1 + b2 : b1;
    }
    // keep the topk_groups best groups (ties -> lower group id)
    kept = 0;
    bool gtaken = false;
    for (int r = 0; r < p.topk_groups; ++r) {
      float bv = (lane < ng && !gtaken) ? gscore : kNone;
      int bi = (lane < ng && !gtaken) ? lane : 0x7fffffff;
      wave_argbest(bv, bi);
      kept |= 1ull << bi;
      if (lane == bi) gtaken = true;
    }
  }
  // topk largest scores inside kept groups (ties -> lower expert id)
  for (int j = 0; j < topk; ++j) {
    float bv = kNone;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + kWave * i;
      if (e < E && !taken[i] && ((kept >> (e / gs)) & 1ull) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
    wave_argbest(bv, bi);
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + kWave * i == bi) taken[i] = 1;
    denom += bv;
    if (lane == j) {
      my_val = bv;
      my_id = bi;
    }
  }
  if (!p.renormalize) denom = 1.0f;
  if (lane < topk) {
    w_out[lane] = my_val / denom * p.scale;
    ids_out[lane] = my_id;
    if (ids_lds) ids_lds[lane] = my_id;
  }
}


// The token's routing by the whole workgroup (E <= 256, topk <= 32): the same selection and
// weights as route_token, without its topk rounds of a wave-wide arg-best.  Every candidate gets
// a 64-bit key, its score mapped to an unsigned integer of the same order above its complemented
// id, so that key order is route_token's order (larger score first, equal scores to the lower
// id) and all keys differ; ineligible candidates (experts of dropped groups, NaN scores) get key
// 0, below every other.  A candidate's place is the number of larger keys: first within its
// wavefront's 64 candidates, then, for the topk best of each wavefront (which hold every
// candidate of the overall top-k), among those.  `v` is the thread's logit (threads t < E).
// Leaves the ids in wid[0, topk) (0x7fffffff where fewer candidates are eligible) and returns
// the weight of place t to the threads t < topk.  Ends with a barrier.
struct __attribute__((aligned(16))) RouteLds {
  uint64_t key[256];
  uint64_t surv[4 * 32];  // the topk best keys of each wavefront (0: none)
  float gsc[64];
  float val[256];
  int wid[32];
  float wval[32];
};

__device__ __forceinline__ uint64_t route_key(float v, int t) {
  const uint32_t b = __float_as_uint(v + 0.0f);  // -0 -> +0: equal scores stay equal
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)t);
}

__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t ord = (uint32_t)(k >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

__device__ float route_single(float v, int E, int topk, const RoutingParams& rp, RouteLds& r) {
  const int t = threadIdx.x;
  const int lane = t & (kWave - 1);
  const int wave = t / kWave;
  const float kNone = -__builtin_inff();
  if (rp.score == 1 && t < E) v = sigmoid_spec(v);
  if (t < 256) r.val[t] = t < E ? v : 0.0f;  // the scores (softmax without renormalisation)
  if (t < 4 * 32) r.surv[t] = 0;
  if (t < topk) {
    r.wid[t] = 0x7fffffff;
    r.wval[t] = kNone;
  }
  bool elig = t < E && v == v;
  const int ng = rp.num_groups;
  if (rp.score == 1 && rp.topk_groups < ng) {
    // group score: sum of the two largest scores of the group's contiguous experts
    const int gs = E / ng;
    if ((gs & (gs - 1)) == 0 && gs <= kWave) {
      // groups of a power of two lanes: top-2 merges across the group's lanes (DPP within rows of
      // 16, then row and half swaps), every lane of the group ends with the pair
      float t1 = t < E ? v : kNone, t2 = kNone;
      if (gs >= 2) top2_step<kDppXor1>(t1, t2);
      if (gs >= 4) top2_step<kDppXor2>(t1, t2);
      if (gs >= 8) top2_step<kDppHalfMirror>(t1, t2);
      if (gs >= 16) top2_step<kDppMirror>(t1, t2);
      if (gs >= 32) {
        uint32_t a1, b1, a2, b2;
        swap_pair<false>(__float_as_uint(t1), a1, b1);
        swap_pair<false>(__float_as_uint(t2), a2, b2);
        t1 = __uint_as_float(a1);
        t2 = __uint_as_float(a2);
        top2_merge(t1, t2, __uint_as_float(b1), __uint_as_float(b2));
      }
      if (gs >= 64) {
        uint32_t a1, b1, a2, b2;
        swap_pair<true>(__float_as_uint(t1), a1, b1);
        swap_pair<true>(__float_as_uint(t2), a2, b2);
        t1 = __uint_as_float(a1);
        t2 = __uint_as_float(a2);
        top2_merge(t1, t2, __uint_as_float(b1), __uint_as_float(b2));
      }
      if (t < E && t % gs == 0) r.gsc[t / gs] = gs >= 2 ? t1 + t2 : t1;
      __syncthreads();
    } else {
      __syncthreads();  // the scores in val
      if (t < ng) {
        float b1 = kNone, b2 = kNone;
        for (int i = 0; i < gs; ++i) {
          const float x = r.val[t * gs + i];
          if (x > b1) {
            b2 = b1;
            b1 = x;
          } else if (x > b2) {
            b2 = x;
          }
        }
        r.gsc[t] = gs >= 2 ? b1 + b2 : b1;
      }
      __syncthreads();
    }
    // keep the topk_groups best groups (ties -> lower group id); each thread ranks its own group
    if (t < E) {
      const int g = t / gs;
      const float mine = r.gsc[g];
      int rank = 0;
#pragma unroll 8
      for (int o = 0; o < ng; ++o) rank += (o != g && better(r.gsc[o], o, mine, g)) ? 1 : 0;
      if (rank >= rp.topk_groups) elig = false;
    }
  }
  const uint64_t key = elig ? route_key(v, t) : 0ull;
  if (t < 256) r.key[t] = key;
  __syncthreads();
  // place within the wavefront's 64 candidates (waves past E hold key 0 only)
  if (elig) {
    const uint64_t* kw = r.key + wave * kWave;
    int c0 = 0, c1 = 0;
#pragma unroll 8
    for (int u = 0; u < kWave; u += 2) {
      c0 += kw[u] > key ? 1 : 0;
      c1 += kw[u + 1] > key ? 1 : 0;
    }
    const int lr = c0 + c1;
    if (lr < topk) r.surv[wave * topk + lr] = key;
  }
  __syncthreads();
  // place among the survivors
  const int ns = ((E + kWave - 1) / kWave) * topk;
  if (t < ns) {
    const uint64_t k = r.surv[t];
    if (k != 0) {
      int c0 = 0, c1 = 0;
      int u = 0;
      for (; u + 1 < ns; u += 2) {
        c0 += r.surv[u] > k ? 1 : 0;
        c1 += r.surv[u + 1] > k ? 1 : 0;
      }
      if (u < ns) c0 += r.surv[u] > k ? 1 : 0;
      const int rank = c0 + c1;
      if (rank < topk) {
        r.wid[rank] = (int)(0xFFFFFFFFu - (uint32_t)k);
        r.wval[rank] = key_value(k);
      }
    }
  }
  __syncthreads();
  if (t >= kWave) return 0.0f;
  // weights, in route_token's order of operations
  float denom = 0.0f, my = 0.0f;
  if (rp.score == 0) {
    const float mx = r.wval[0];
    for (int j = 0; j < topk; ++j) {
      const float ej = expf(r.wval[j] - mx);
      denom += ej;
      if (j == lane) my = ej;
    }
    if (!rp.renormalize) {
      float part = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + kWave * i < E) part += expf(r.val[lane + kWave * i] - mx);
      denom = wave_sum(part);
    }
  } else {
    for (int j = 0; j < topk; ++j) {
      denom += r.wval[j];
      if (j == lane) my = r.wval[j];
    }
    if (!rp.renormalize) denom = 1.0f;
  }
  return my / denom * rp.scale;
}

}  // namespace
}  // namespace moe
