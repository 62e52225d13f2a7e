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

// Workgroup barrier for LDS traffic only: it waits for the wave's LDS (and
// scalar) operations but not for its global stores, which stay in flight.
// __syncthreads() would also drain every store before the barrier, about a
// microsecond per barrier after a store.  Only for code in which no thread
// reads global memory that another thread of the workgroup wrote during the
// same launch.
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Exclusive scan of one int per thread over the block (at most 64 waves);
// *total gets the sum.  The wave totals go through LDS once and are scanned
// by every wave with the same DPP scan (lane i holds wave i's total), so
// the cost does not grow with the wave count.  Synchronises through LDS only
// (lds_sync).
__device__ int block_excl_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int x = wave_incl_scan(v);
  if (lane == 63) s_tmp[w] = x;
  lds_sync();
  const int wsum = wave_incl_scan(lane < nw ? s_tmp[lane] : 0);
  lds_sync();  // s_tmp may be rewritten by the next scan
  *total = __builtin_amdgcn_readlane(wsum, 63);
  const int base = w > 0 ? __builtin_amdgcn_readlane(wsum, w - 1) : 0;
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

// Top-k of one token in one wave.  Lane l holds the ordered-logit keys of
// experts l, l+64, ... (NK of them; 0 for experts past E, below every finite
// logit) and its best one (the first maximum, so the lowest expert among
// equal logits).  Each round reduces the lanes' best keys to the wave
// maximum on 32-bit DPP steps; a ballot finds the lanes that hold it, and
// when more than one does (equal logits in several lanes) the lowest expert
// among them wins, as in the (logit descending, expert ascending) order.  The
// winner lane clears that key and recomputes its best.  topk_load issues the
// logit loads (so a caller can start them early), topk_select does the rest.
template <int NK>
__device__ __forceinline__ void topk_load(const TopkArgs& a, int t, uint32_t (&keys)[NK]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < NK; i++) {
    const int e = lane + 64 * i;
    keys[i] = e < a.E ? ordered_bits(a.logits[(size_t)t * a.E + e]) : 0u;
  }
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ uint32_t max_step_u32(uint32_t v) {
  const uint32_t o = dpp<CTRL, ROWS>(v);
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max_step_u32<0x111>(v);
  v = max_step_u32<0x112>(v);
  v = max_step_u32<0x114>(v);
  v = max_step_u32<0x118>(v);
  v = max_step_u32<0x142, 0xA>(v);
  v = max_step_u32<0x143, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}
// Wave minimum through the maximum of the complements.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return ~wave_max_u32(~v); }

template <int NK>
__device__ __forceinline__ void best_key(const uint32_t (&keys)[NK], uint32_t& bv, int& bi) {
  bv = keys[0];
  bi = 0;
#pragma unroll
  for (int i = 1; i < NK; i++)
    if (keys[i] > bv) {
      bv = keys[i];
      bi = i;
    }
}

template <int NK>
__device__ void topk_select(const TopkArgs& a, int t, uint32_t (&keys)[NK], int* s_ids) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, k = a.k;
  uint32_t bv;
  int bi;
  best_key<NK>(keys, bv, bi);
  // Round j's expert and logit stay in lane j; no branch on the winner lane,
  // one store per output at the end.
  int my_e = 0;
  float my_l = 0.f, l0 = 0.f;
  for (int j = 0; j < k; j++) {
    const uint32_t m = wave_max_u32(bv);
    const uint64_t holders = __ballot(bv == m);
    int e;
    if (__popcll(holders) == 1)
      e = __builtin_amdgcn_readlane(lane + 64 * bi, (int)__builtin_ctzll(holders));
    else  // equal logits in several lanes: the lowest expert
      e = (int)wave_min_u32(bv == m ? (uint32_t)(lane + 64 * bi) : 0xFFFFFFFFu);
    const bool winner = lane == (e & 63);
#pragma unroll
    for (int i = 0; i < NK; i++) keys[i] = (winner && i == (e >> 6)) ? 0u : keys[i];
    best_key<NK>(keys, bv, bi);
    const float l = from_ordered_bits(m);
    if (lane == j) {
      my_e = e;
      my_l = l;
    }
    if (j == 0) l0 = l;
  }
  if (lane < k) {
    a.ids[t * k + lane] = my_e;
    if (s_ids) s_ids[t * k + lane] = my_e;
    if (a.user_ids) a.user_ids[t * k + lane] = my_e;
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

template <int NK>
__device__ void topk_token(const TopkArgs& a, int t, int* s_ids) {
  uint32_t keys[NK];
  topk_load<NK>(a, t, keys);
  topk_select<NK>(a, t, keys, s_ids);
}

}  // namespace moe
