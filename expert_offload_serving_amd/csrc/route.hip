// Routing for the decode forward: router logits, top-k, gates, dispatch
// permutation and the global LRU cache lookup, all on the device.
//
// The router is unchanged by offloading (jansverre.net FreeToken article,
// section "Hva er FreeToken?"); the cache is one LRU shared by all MoE
// layers (same article, section "Hvorfor er båndbredden viktigere enn antall
// kjerner?"), exploiting overlap between adjacent tokens (aipolix.com
// FreeToken article, fifth paragraph).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterRows = 32;   // H rows per router workgroup
constexpr int kFinalizeThreads = 1024;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// partials[chunk][t][e] = sum over the chunk's H rows of x[t][h] * W_r[h][e],
// in fp64.  bf16 x fp32 products are exact in fp64.
template <int TG>
__global__ __launch_bounds__(256) void router_partial_kernel(
    const uint16_t* __restrict__ x, int T, int H, int E,
    const float* __restrict__ wr, double* __restrict__ partials) {
  const int chunk = blockIdx.x;
  const int h0 = chunk * kRouterRows;
  const int hn = min(kRouterRows, H - h0);
  __shared__ float xs[TG][kRouterRows];
  for (int tg = 0; tg < T; tg += TG) {
    const int tn = min(TG, T - tg);
    __syncthreads();
    for (int i = threadIdx.x; i < TG * kRouterRows; i += blockDim.x) {
      const int t = i / kRouterRows, hh = i % kRouterRows;
      xs[t][hh] = (t < tn && hh < hn) ? bf16_bits_to_f32(x[(size_t)(tg + t) * H + h0 + hh]) : 0.f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
      double acc[TG];
#pragma unroll
      for (int t = 0; t < TG; t++) acc[t] = 0.0;
      for (int hh = 0; hh < hn; hh++) {
        const double wv = (double)wr[(size_t)(h0 + hh) * E + e];
#pragma unroll
        for (int t = 0; t < TG; t++) acc[t] = fma((double)xs[t][hh], wv, acc[t]);
      }
#pragma unroll
      for (int t = 0; t < TG; t++)
        if (t < tn) partials[((size_t)chunk * T + tg + t) * E + e] = acc[t];
    }
  }
}

// Exclusive scan of one int per thread over the block; *total gets the sum.
__device__ int block_excl_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, d, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// Block-wide LRU lookup of the n unique experts in s_U (ascending).
// Slot codes go to s_slot[u]; fills (cache and staging copies) to a.fills.
// See the rule in moe.h (moe_layer_forward).
__device__ void block_lookup(const LookupArgs& a, const int* s_U, int n, int* s_slot,
                             int* s_tmp, int* s_evict) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int C = a.C;
  const uint64_t clock0 = a.cache->clock;
  if (tid == 0) *s_evict = 0;
  for (int s = tid; s < C; s += nt) a.hitflag[s] = 0;
  __syncthreads();

  const int u = tid;
  const int e = u < n ? s_U[u] : -1;
  const bool valid = e >= 0 && e < a.E;
  const int key = valid ? a.layer * a.E + e : -1;
  const int slot = valid ? a.map[key] : -1;
  const bool hit = valid && slot >= 0;
  const bool miss = valid && !hit;
  int n_hit, n_miss;
  const int hrank = block_excl_scan(hit ? 1 : 0, s_tmp, &n_hit);
  const int mrank = block_excl_scan(miss ? 1 : 0, s_tmp, &n_miss);
  const int n_fill = min(n_miss, C - n_hit);
  if (hit) {
    a.hitflag[slot] = 1;
    a.stamp[slot] = clock0 + 1 + (uint64_t)hrank;
    s_slot[u] = slot;
  }
  __syncthreads();

  // Victims: non-hit slots in recency order; untouched ones keep their order.
  int carry = 0, carry_keep = 0;
  for (int p0 = 0; p0 < C; p0 += nt) {
    const int p = p0 + tid;
    const int s = p < C ? a.order[p] : -1;
    const bool nonhit = p < C && !a.hitflag[s];
    int tot, ktot;
    const int r = block_excl_scan(nonhit ? 1 : 0, s_tmp, &tot) + carry;
    const bool victim = nonhit && r < n_fill;
    if (victim) a.victim[r] = s;
    const bool keep = nonhit && !victim;
    const int kr = block_excl_scan(keep ? 1 : 0, s_tmp, &ktot) + carry_keep;
    if (keep) a.order_tmp[kr] = s;
    carry += tot;
    carry_keep += ktot;
  }
  __syncthreads();
  const int n_keep = C - n_hit - n_fill;
  if (hit) a.order_tmp[n_keep + hrank] = slot;
  if (miss) {
    const uint8_t* src = a.pool + (size_t)key * a.stride;
    if (mrank < n_fill) {
      const int s = a.victim[mrank];
      const int old = a.key[s];
      if (old >= 0) {
        a.map[old] = -1;
        atomicAdd(s_evict, 1);
      }
      a.key[s] = key;
      a.map[key] = s;
      a.stamp[s] = clock0 + (uint64_t)n_hit + 1 + (uint64_t)mrank;
      a.order_tmp[n_keep + n_hit + mrank] = s;
      a.fills[mrank] = FillEntry{src, a.slots + (size_t)s * a.stride};
      s_slot[u] = s;
    } else {
      const int b = mrank - n_fill;
      a.fills[mrank] = FillEntry{src, a.staging_buf + (size_t)b * a.stride};
      s_slot[u] = -1 - b;
    }
  }
  if (u < n && !valid) s_slot[u] = INT_MIN;
  __syncthreads();
  for (int p = tid; p < C; p += nt) a.order[p] = a.order_tmp[p];
  if (tid == 0) {
    DevCache* dc = a.cache;
    dc->clock = clock0 + (uint64_t)n_hit + (uint64_t)n_fill;
    dc->lookups += (uint64_t)(n_hit + n_miss);
    dc->hits += (uint64_t)n_hit;
    dc->fills += (uint64_t)n_fill;
    dc->bypasses += (uint64_t)(n_miss - n_fill);
    dc->evictions += (uint64_t)*s_evict;
    a.meta->n_fill = n_miss;
    a.meta->n_hit = n_hit;
    a.meta->n_bypass = n_miss - n_fill;
  }
  __syncthreads();
}

struct FinalizeArgs {
  int T, H, E, k, renorm, n_chunks, has_shared;
  const double* partials;
  const float* bias;
  float* logits;
  int32_t* ids;
  float* gates;
  int32_t* user_ids;
  float* user_gates;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted;
  int32_t* inv;
  int32_t* unique;
  int32_t* slotcode;
  int32_t* tok;
  WorkItem* items;
  const uint8_t* shared_w;
  LookupArgs la;
};

__global__ __launch_bounds__(kFinalizeThreads) void route_finalize_kernel(FinalizeArgs a) {
  __shared__ int s_counts[1024];
  __shared__ unsigned long long s_mask[1024];
  __shared__ int s_offsets[1025];
  __shared__ int s_ids[1024];
  __shared__ int s_U[1024];
  __shared__ int s_slot[1024];
  __shared__ int s_tmp[16];
  __shared__ int s_evict;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int lane = tid & 63, w = tid >> 6, nw = nt >> 6;
  const int T = a.T, E = a.E, k = a.k;

  // 1. logits = fp32(sum of chunk partials in order + bias), fp64 inside
  for (int i = tid; i < T * E; i += nt) {
    const int t = i / E, e = i % E;
    double s = 0.0;
    for (int c = 0; c < a.n_chunks; c++) s += a.partials[((size_t)c * T + t) * E + e];
    if (a.bias) s += (double)a.bias[i];
    a.logits[i] = (float)s;
  }
  for (int e = tid; e < 1024; e += nt) {
    s_counts[e] = 0;
    s_mask[e] = 0ull;
  }
  __syncthreads();

  // 2. top-k per token (one wave per token): key = (ordered logit, ~expert)
  for (int t = w; t < T; t += nw) {
    uint64_t keys[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int e = lane + 64 * i;
      keys[i] = e < E ? ((uint64_t)ordered_bits(a.logits[(size_t)t * E + e]) << 32) |
                            (uint64_t)(0xFFFFFFFFu - (uint32_t)e)
                      : 0ull;
    }
    float my_l = 0.f;
    float l0 = 0.f;
    for (int j = 0; j < k; j++) {
      uint64_t best = 0;
#pragma unroll
      for (int i = 0; i < 16; i++) best = keys[i] > best ? keys[i] : best;
      best = wave_max_u64(best);
      const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
      const float l = from_ordered_bits((uint32_t)(best >> 32));
#pragma unroll
      for (int i = 0; i < 16; i++)
        if (lane + 64 * i == e) keys[i] = 0ull;
      if (lane == j) my_l = l;
      if (j == 0) l0 = l;
      if (lane == 0) {
        a.ids[t * k + j] = e;
        s_ids[t * k + j] = e;
        if (a.user_ids) a.user_ids[t * k + j] = e;
      }
    }
    double z = 0.0, denom;
    if (a.renorm) {
      z = lane < k ? exp((double)my_l - (double)l0) : 0.0;
      denom = wave_sum_f64(z);
    } else {
      double part = 0.0;
      for (int i = 0; i < 16; i++) {
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
  __syncthreads();

  // 3. dispatch: counts, offsets, stable permutation, unique experts
  const int nk = T * k;
  int n_unique;
  for (int f = tid; f < nk; f += nt) {
    const int e = s_ids[f];
    atomicAdd(&s_counts[e], 1);
    atomicOr(&s_mask[e], 1ull << (f / k));
  }
  __syncthreads();
  {
    const int e = tid;
    const int cnt = e < E ? s_counts[e] : 0;
    int total;
    const int off = block_excl_scan(cnt, s_tmp, &total);
    const int ur = block_excl_scan(cnt > 0 ? 1 : 0, s_tmp, &n_unique);
    if (e < E) {
      s_offsets[e] = off;
      a.counts[e] = cnt;
      a.offsets[e] = off;
      if (cnt > 0) {
        s_U[ur] = e;
        a.unique[ur] = e;
      }
    }
    if (tid == 0) {
      s_offsets[E] = total;
      a.offsets[E] = total;
      a.la.meta->n_unique = n_unique;
      a.la.meta->T = T;
    }
  }
  __syncthreads();
  for (int f = tid; f < nk; f += nt) {
    const int t = f / k, e = s_ids[f];
    const int rank = __popcll(s_mask[e] & ((1ull << t) - 1ull));
    const int pos = s_offsets[e] + rank;
    a.sorted[pos] = f;
    a.inv[f] = pos;
    a.tok[pos] = t;
  }
  __syncthreads();

  // 4. cache lookup of the unique experts
  block_lookup(a.la, s_U, n_unique, s_slot, s_tmp, &s_evict);

  // 5. work list for the expert kernels
  for (int u = tid; u < n_unique; u += nt) {
    const int code = s_slot[u];
    const uint8_t* wptr = code >= 0 ? a.la.slots + (size_t)code * a.la.stride
                                    : a.la.staging_buf + (size_t)(-1 - code) * a.la.stride;
    const int e = s_U[u];
    a.items[u] = WorkItem{wptr, s_offsets[e], s_counts[e]};
    a.slotcode[u] = code;
  }
  if (a.has_shared) {
    for (int t = tid; t < T; t += nt) a.tok[nk + t] = t;
    if (tid == 0) a.items[n_unique] = WorkItem{a.shared_w, nk, T};
  }
  if (tid == 0) a.la.meta->n_items = n_unique + a.has_shared;
}

// Standalone lookup for expert_cache_lookup / expert_cache_fill.
__global__ __launch_bounds__(kFinalizeThreads) void cache_lookup_kernel(
    LookupArgs la, const int32_t* experts, const int32_t* d_n, int n_max, int32_t* out_slot) {
  __shared__ int s_U[1024];
  __shared__ int s_slot[1024];
  __shared__ int s_tmp[16];
  __shared__ int s_evict;
  int n = *d_n;
  n = n < 0 ? 0 : (n > n_max ? n_max : n);
  for (int u = threadIdx.x; u < n; u += blockDim.x) s_U[u] = experts[u];
  __syncthreads();
  block_lookup(la, s_U, n, s_slot, s_tmp, &s_evict);
  for (int u = threadIdx.x; u < n; u += blockDim.x) out_slot[u] = s_slot[u];
}

LookupArgs make_lookup_args(Ctx* c, int layer) {
  LookupArgs la;
  la.layer = layer;
  la.E = c->cfg.n_experts;
  la.C = c->C;
  la.staging = c->cfg.staging_slots;
  la.key = c->d_key;
  la.stamp = c->d_stamp;
  la.order = c->d_order;
  la.order_tmp = c->d_order_tmp;
  la.map = c->d_map;
  la.hitflag = c->d_hitflag;
  la.victim = c->d_victim;
  la.cache = c->d_cache;
  la.pool = c->pool;
  la.slots = c->d_slots;
  la.staging_buf = c->d_staging;
  la.stride = c->stride;
  la.fills = c->d_fills;
  la.meta = c->d_meta;
  return la;
}

}  // namespace

int router_chunk_rows(int) { return kRouterRows; }

hipError_t launch_router_partial(const uint16_t* x, int T, int H, int E, const float* wr,
                                 double* partials, hipStream_t st) {
  const int chunks = (H + kRouterRows - 1) / kRouterRows;
  if (T <= 1)
    router_partial_kernel<1><<<chunks, 256, 0, st>>>(x, T, H, E, wr, partials);
  else if (T <= 4)
    router_partial_kernel<4><<<chunks, 256, 0, st>>>(x, T, H, E, wr, partials);
  else
    router_partial_kernel<16><<<chunks, 256, 0, st>>>(x, T, H, E, wr, partials);
  return hipGetLastError();
}

hipError_t launch_route_finalize(Ctx* c, int layer, int T, const float* bias,
                                 int32_t* user_ids, float* user_gates, hipStream_t st) {
  FinalizeArgs a;
  a.T = T;
  a.H = c->cfg.hidden;
  a.E = c->cfg.n_experts;
  a.k = c->cfg.top_k;
  a.renorm = c->cfg.renormalize;
  a.n_chunks = (a.H + kRouterRows - 1) / kRouterRows;
  a.has_shared = c->cfg.has_shared;
  a.partials = c->d_partials;
  a.bias = bias;
  a.logits = c->d_logits;
  a.ids = c->d_ids;
  a.gates = c->d_gates;
  a.user_ids = user_ids;
  a.user_gates = user_gates;
  a.counts = c->d_counts;
  a.offsets = c->d_offsets;
  a.sorted = c->d_sorted;
  a.inv = c->d_inv;
  a.unique = c->d_unique;
  a.slotcode = c->d_slotcode;
  a.tok = c->d_tok;
  a.items = c->d_items;
  a.shared_w = c->cfg.has_shared ? c->d_shared + (size_t)layer * c->stride : nullptr;
  a.la = make_lookup_args(c, layer);
  route_finalize_kernel<<<1, kFinalizeThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_cache_lookup(Ctx* c, int layer, const int32_t* d_experts, const int32_t* d_n,
                               int n_max, int32_t* d_slot, hipStream_t st) {
  cache_lookup_kernel<<<1, kFinalizeThreads, 0, st>>>(make_lookup_args(c, layer), d_experts, d_n,
                                                      n_max, d_slot);
  return hipGetLastError();
}

}  // namespace moe
