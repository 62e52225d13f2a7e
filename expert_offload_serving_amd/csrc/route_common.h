// Wave-level primitives shared by the routing kernels (decode and prefill):
// DPP reductions and scans, order-preserving float keys, per-token top-k.
#pragma once

#include "moe_internal.h"

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Wave-wide reductions on DPP (row shifts, then row broadcasts 15 and 31);
// the full result lands in lane 63.  The combination order is fixed.
template <int CTRL, int ROWS = 0xF, int BANKS = 0xF>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return __builtin_amdgcn_update_dpp(0u, v, CTRL, ROWS, BANKS, false);
}
template <int CTRL, int ROWS = 0xF, int BANKS = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t r = ((uint64_t)dpp<CTRL, ROWS, BANKS>((uint32_t)(u >> 32)) << 32) |
                     dpp<CTRL, ROWS, BANKS>((uint32_t)u);
  return __builtin_bit_cast(double, r);
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dpp_f64<0x111>(v);          // row_shr:1
  v += dpp_f64<0x112>(v);          // row_shr:2
  v += dpp_f64<0x114>(v);          // row_shr:4
  v += dpp_f64<0x118>(v);          // row_shr:8
  v += dpp_f64<0x142, 0xA>(v);     // row_bcast:15
  v += dpp_f64<0x143, 0xC>(v);     // row_bcast:31
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t r = ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(u >> 32), 63) << 32) |
                     (uint32_t)__builtin_amdgcn_readlane((uint32_t)u, 63);
  return __builtin_bit_cast(double, r);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint64_t max_step(uint64_t v) {
  const uint64_t o = ((uint64_t)dpp<CTRL, ROWS>((uint32_t)(v >> 32)) << 32) |
                     dpp<CTRL, ROWS>((uint32_t)v);
  return o > v ? o : v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_step<0x111>(v);
  v = max_step<0x112>(v);
  v = max_step<0x114>(v);
  v = max_step<0x118>(v);
  v = max_step<0x142, 0xA>(v);
  v = max_step<0x143, 0xC>(v);
  return ((uint64_t)__builtin_amdgcn_readlane((uint32_t)(v >> 32), 63) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((uint32_t)v, 63);
}

// Inclusive scan of one int per lane (DPP, fixed order).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += (int)dpp<0x111>((uint32_t)v);
  v += (int)dpp<0x112>((uint32_t)v);
  v += (int)dpp<0x114>((uint32_t)v);
  v += (int)dpp<0x118>((uint32_t)v);
  v += (int)dpp<0x142, 0xA>((uint32_t)v);
  v += (int)dpp<0x143, 0xC>((uint32_t)v);
  return v;
}

// Exclusive scan of one int per thread over the block; *total gets the sum.
__device__ int block_excl_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) s_tmp[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < nw; i++) {
    const int s = s_tmp[i];
    if (i < w) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Order-preserving map of a finite fp32 to uint32.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

struct TopkArgs {
  int E, k, renorm;
  const float* logits;   // [T][E]
  int32_t* ids;          // [T][k]
  float* gates;          // [T][k]
  int32_t* user_ids;     // optional copies
  float* user_gates;
};

// Top-k of one token in one wave.  Lane l holds the keys of experts
// l, l+64, ... (NK of them) as (ordered logit << 32 | ~expert): the largest
// key is the largest logit, ties to the lower expert.  Each round takes the
// wave maximum of the lanes' current maxima; only the winner lane clears
// that key and recomputes its maximum.
template <int NK>
__device__ void topk_token(const TopkArgs& a, int t, int* s_ids) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  uint64_t keys[NK];
#pragma unroll
  for (int i = 0; i < NK; i++) {
    const int e = lane + 64 * i;
    keys[i] = e < E ? ((uint64_t)ordered_bits(a.logits[(size_t)t * E + e]) << 32) |
                          (uint64_t)(0xFFFFFFFFu - (uint32_t)e)
                    : 0ull;
  }
  uint64_t lmax = 0;
#pragma unroll
  for (int i = 0; i < NK; i++) lmax = keys[i] > lmax ? keys[i] : lmax;
  float my_l = 0.f, l0 = 0.f;
  for (int j = 0; j < k; j++) {
    const uint64_t best = wave_max_u64(lmax);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const float l = from_ordered_bits((uint32_t)(best >> 32));
    if (lmax == best) {  // the winner lane (keys are unique)
      lmax = 0;
#pragma unroll
      for (int i = 0; i < NK; i++) {
        if (keys[i] == best) keys[i] = 0ull;
        lmax = keys[i] > lmax ? keys[i] : lmax;
      }
    }
    if (lane == j) my_l = l;
    if (j == 0) l0 = l;
    if (lane == 0) {
      a.ids[t * k + j] = e;
      if (s_ids) s_ids[t * k + j] = e;
      if (a.user_ids) a.user_ids[t * k + j] = e;
    }
  }
  double z = 0.0, denom;
  if (a.renorm) {
    z = lane < k ? exp((double)my_l - (double)l0) : 0.0;
    denom = wave_sum_f64(z);
  } else {
    double part = 0.0;
#pragma unroll
    for (int i = 0; i < NK; i++) {
      const int e = lane + 64 * i;
      if (e < E) part += exp((double)a.logits[(size_t)t * E + e] - (double)l0);
    }
    denom = wave_sum_f64(part);
    z = lane < k ? exp((double)my_l - (double)l0) : 0.0;
  }
  if (lane < k) {
    const float g = (float)(z / denom);
    a.gates[t * k + lane] = g;
    if (a.user_gates) a.user_gates[t * k + lane] = g;
  }
}

}  // namespace moe
