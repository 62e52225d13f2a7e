// C-ABI entry points of libmoe: validation, memory ownership, cache state,
// and the launch sequence of the decode forward.
#include <algorithm>
#include <cstring>
#include <new>
#include <numeric>
#include <string>
#include <thread>
#include <vector>

#include "moe_internal.h"

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIPCHK(expr)                                                        \
  do {                                                                      \
    hipError_t _e = (expr);                                                 \
    if (_e != hipSuccess)                                                   \
      return fail(MOE_ERR_HIP, std::string(#expr) + ": " +                  \
                                   hipGetErrorString(_e));                  \
  } while (0)

#define ALLOC(ptr, bytes)                                                   \
  do {                                                                      \
    size_t _b = (bytes);                                                    \
    if (_b) {                                                               \
      hipError_t _e = hipMalloc((void**)&(ptr), _b);                        \
      if (_e != hipSuccess) {                                               \
        destroy_all(c);                                                     \
        return fail(MOE_ERR_OOM, std::string("hipMalloc ") + #ptr + " (" +  \
                                     std::to_string(_b) + " bytes): " +     \
                                     hipGetErrorString(_e));                \
      }                                                                     \
    }                                                                       \
  } while (0)

template <class T>
void dfree(T*& p) {
  if (p) (void)hipFree((void*)p);
  p = nullptr;
}

void destroy_all(Ctx* c) {
  if (!c) return;
  prefill_free(c);
  if (c->pool) (void)hipHostFree(c->pool);
  c->pool = nullptr;
  dfree(c->d_router); dfree(c->d_shared); dfree(c->d_slots); dfree(c->d_staging);
  dfree(c->d_key); dfree(c->d_stamp); dfree(c->d_order); dfree(c->d_order_tmp);
  dfree(c->d_hitflag); dfree(c->d_map); dfree(c->d_victim); dfree(c->d_cache);
  dfree(c->d_logits); dfree(c->d_ids); dfree(c->d_gates);
  dfree(c->d_counts); dfree(c->d_offsets); dfree(c->d_sorted); dfree(c->d_inv);
  dfree(c->d_unique); dfree(c->d_slotcode); dfree(c->d_tok); dfree(c->d_items);
  dfree(c->d_fills); dfree(c->d_meta); dfree(c->d_h); dfree(c->d_yperm);
  dfree(c->d_lookup_ids);
  for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
  c->ev_pool.clear();
}

// Run fn(i) for i in [0, n) on up to `threads` host threads.
template <class F>
void parallel_for(int n, int threads, F fn) {
  threads = std::max(1, std::min(threads, n));
  if (threads == 1) {
    for (int i = 0; i < n; i++) fn(i);
    return;
  }
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; t++)
    pool.emplace_back([=, &fn] {
      for (int i = t; i < n; i += threads) fn(i);
    });
  for (auto& th : pool) th.join();
}

int host_threads() {
  unsigned n = std::thread::hardware_concurrency();
  return (int)std::max(1u, std::min(n, 16u));
}

bool scales_valid(const uint8_t* s, size_t n) {
  for (size_t i = 0; i < n; i++)
    if (s[i] == 255) return false;
  return true;
}

// Upload a host vector to a device array (sync).
template <class T>
hipError_t upload(T* dst, const std::vector<T>& v) {
  if (v.empty()) return hipSuccess;
  return hipMemcpy(dst, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice);
}

moe_status check_ctx(moe_ctx* ctx) {
  if (!ctx) return fail(MOE_ERR_INVALID_ARG, "ctx is NULL");
  return MOE_OK;
}

Ctx* C_(moe_ctx* ctx) { return reinterpret_cast<Ctx*>(ctx); }


constexpr size_t kMaxTimingPairs = 65536;

}  // namespace

namespace moe {

int fillable_slots(const Ctx* c, int layer, bool insert, int* slot0) {
  int first = 0, n = c->C;
  if (c->cfg.cache_policy == MOE_CACHE_PER_LAYER) {
    const int64_t L = c->cfg.n_layers;
    first = (int)(layer * (int64_t)c->C / L);
    n = (int)((layer + 1) * (int64_t)c->C / L) - first;
  } else if (c->cfg.cache_policy == MOE_CACHE_STATIC && !insert) {
    n = 0;
  }
  if (slot0) *slot0 = first;
  return n;
}

hipEvent_t timing_event(Ctx* c) {
  if (c->ev_next == c->ev_pool.size()) {
    hipEvent_t e;
    // Timing only: no system-scope fences (they flush caches and add
    // microseconds between the event and the kernel it brackets).
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    c->ev_pool.push_back(e);
  }
  return c->ev_pool[c->ev_next++];
}

// --------------------------------------------------------------- repacking
// Canonical row r of a [N][K] MXFP4 matrix: codes q[r][K/2], scales s[r][K/32].
// Lane l of the atom takes row row0 + l % 16, MX block 4 c + l / 16.
static void write_atom(const uint8_t* q, const uint8_t* s, int K, int row0, int c,
                       uint8_t* atom) {
  const int kc = K / 2, sc = K / 32;
  for (int l = 0; l < 64; l++) {
    const int r = row0 + (l % 16), blk = c * 4 + l / 16;
    std::memcpy(atom + l * 16, q + (size_t)r * kc + (size_t)blk * 16, 16);
    atom[kAtomData + l] = s[(size_t)r * sc + blk];
  }
}

void repack_gateup(const uint8_t* qg, const uint8_t* sg, const uint8_t* qu,
                   const uint8_t* su, int I, int H, uint8_t* out) {
  const int KC = H / kAtomK, groups = 2 * I / kAtomRows;
  parallel_for(groups, (size_t)I * H > (1 << 22) ? host_threads() : 1, [&](int rg) {
    const bool up = rg & 1;
    const int row0 = (rg / 2) * kAtomRows;
    for (int c = 0; c < KC; c++)
      write_atom(up ? qu : qg, up ? su : sg, H, row0, c,
                 out + ((size_t)rg * KC + c) * kAtomBytes);
  });
}

void repack_down(const uint8_t* qd, const uint8_t* sd, int H, int I, uint8_t* out) {
  const int KC = I / kAtomK, groups = H / kAtomRows;
  parallel_for(groups, (size_t)I * H > (1 << 22) ? host_threads() : 1, [&](int rg) {
    for (int c = 0; c < KC; c++)
      write_atom(qd, sd, I, rg * kAtomRows, c, out + ((size_t)rg * KC + c) * kAtomBytes);
  });
}

// bf16 [N][K] matrix: lane l of the atom takes row row0 + l % 16, values
// K = 32 (4 c + l / 16) .. +31, as 4 pieces of 8 at 1024 p + 16 l (piece p is
// what the lane feeds the MFMA at K step p).
static void write_atom_bf16(const uint16_t* w, int K, int row0, int c, uint8_t* atom) {
  for (int l = 0; l < 64; l++) {
    const uint16_t* src = w + (size_t)(row0 + l % 16) * K + (size_t)(c * 4 + l / 16) * 32;
    for (int p = 0; p < 4; p++) std::memcpy(atom + 1024 * p + 16 * l, src + 8 * p, 16);
  }
}

void repack_gateup_bf16(const uint16_t* wg, const uint16_t* wu, int I, int H, uint8_t* out) {
  const int KC = H / kAtomK, groups = 2 * I / kAtomRows;
  parallel_for(groups, (size_t)I * H > (1 << 22) ? host_threads() : 1, [&](int rg) {
    for (int c = 0; c < KC; c++)
      write_atom_bf16((rg & 1) ? wu : wg, H, (rg / 2) * kAtomRows, c,
                      out + ((size_t)rg * KC + c) * kAtomBytesBF16);
  });
}

void repack_down_bf16(const uint16_t* wd, int H, int I, uint8_t* out) {
  const int KC = I / kAtomK, groups = H / kAtomRows;
  parallel_for(groups, (size_t)I * H > (1 << 22) ? host_threads() : 1, [&](int rg) {
    for (int c = 0; c < KC; c++)
      write_atom_bf16(wd, I, rg * kAtomRows, c, out + ((size_t)rg * KC + c) * kAtomBytesBF16);
  });
}

// Repack one expert into `rec` in the context's format.
static void repack_expert(const Ctx* c, const uint8_t* qg, const uint8_t* qu, const uint8_t* qd,
                          const uint8_t* sg, const uint8_t* su, const uint8_t* sd, uint8_t* rec) {
  const int H = c->cfg.hidden, I = c->cfg.inter, fmt = c->cfg.weight_format;
  if (fmt == MOE_WEIGHTS_BF16) {
    repack_gateup_bf16((const uint16_t*)qg, (const uint16_t*)qu, I, H, rec);
    repack_down_bf16((const uint16_t*)qd, H, I, rec + gateup_section_bytes(H, I, fmt));
  } else {
    repack_gateup(qg, sg, qu, su, I, H, rec);
    repack_down(qd, sd, H, I, rec + gateup_section_bytes(H, I, fmt));
  }
}

}  // namespace moe

// =========================================================================
extern "C" {

const char* moe_last_error(void) { return g_err.c_str(); }

size_t moe_expert_bytes(int32_t hidden, int32_t inter) {
  if (hidden <= 0 || inter <= 0) return 0;
  return expert_record_bytes(hidden, inter);
}

moe_status moe_create(const moe_config* cfg, moe_ctx** out) {
  if (!cfg || !out) return fail(MOE_ERR_INVALID_ARG, "cfg and out must not be NULL");
  const moe_config& f = *cfg;
  if (f.hidden <= 0 || f.inter <= 0 || f.n_layers < 1 || f.top_k < 1 || f.top_k > 16 ||
      f.n_experts < f.top_k || f.n_experts > 1024 || f.max_tokens < 1 ||
      f.max_tokens > 64 || f.cache_slots < 0 || f.staging_slots < 0 ||
      f.max_prefill_tokens < 0 || (f.has_shared != 0 && f.has_shared != 1) ||
      f.cache_policy < MOE_CACHE_GLOBAL || f.cache_policy > MOE_CACHE_STATIC ||
      f.weight_format < MOE_WEIGHTS_MXFP4 || f.weight_format > MOE_WEIGHTS_BF16 ||
      (f.renormalize != 0 && f.renormalize != 1))
    return fail(MOE_ERR_INVALID_ARG, "moe_config field out of range");
  if ((int64_t)f.cache_slots > (int64_t)f.n_layers * f.n_experts)
    return fail(MOE_ERR_INVALID_ARG, "cache_slots exceeds n_layers*n_experts");
  if ((int64_t)f.n_layers * f.n_experts >= (1 << (31 - kOrderKeyShift)))
    return fail(MOE_ERR_UNSUPPORTED, "n_layers*n_experts too large");
  if (f.hidden % 128 || f.inter % 128 || f.hidden > kMaxH || f.inter > kMaxH)
    return fail(MOE_ERR_UNSUPPORTED, "hidden and inter must be multiples of 128, at most 6144");
  if (f.weight_format == MOE_WEIGHTS_BF16 && (f.max_tokens > 16 || f.max_prefill_tokens > 0))
    return fail(MOE_ERR_UNSUPPORTED,
                "bf16 experts run the decode path for at most 16 tokens per call (no prefill)");
  if (f.cache_slots > kMaxCacheSlots)
    return fail(MOE_ERR_UNSUPPORTED, "cache_slots above 4096");
  if (f.max_prefill_tokens > (1 << 20))
    return fail(MOE_ERR_INVALID_ARG, "max_prefill_tokens too large");
  // The prefill kernels address x (T x H bf16), h (a bf16 plane of
  // T*(k+1) x I) and h's low-order records through 32-bit buffer offsets.
  if ((int64_t)f.max_prefill_tokens * f.hidden * 2 >= (int64_t(1) << 31) ||
      (int64_t)f.max_prefill_tokens * (f.top_k + 1) * f.inter * 2 >= (int64_t(1) << 31) ||
      (int64_t)prefill_lo_bytes(f.max_prefill_tokens, f.top_k, f.n_experts, f.inter) >=
          (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED,
                "max_prefill_tokens too large for this shape (x or h reach 2 GiB)");

  Ctx* c = new (std::nothrow) Ctx();
  if (!c) return fail(MOE_ERR_OOM, "context allocation");
  c->cfg = f;
  {
    const hipError_t e0 = hipGetDevice(&c->device);
    if (e0 != hipSuccess) {
      delete c;
      return fail(MOE_ERR_HIP, std::string("device query: ") + hipGetErrorString(e0));
    }
  }
  const int H = f.hidden, I = f.inter, E = f.n_experts, k = f.top_k, L = f.n_layers;
  const int Tm = f.max_tokens;
  c->rec_bytes = expert_record_bytes(H, I, f.weight_format);
  c->stride = (c->rec_bytes + 255) / 256 * 256;
  c->max_unique = std::min(Tm * k, E);
  c->max_items = c->max_unique + f.has_shared;
  c->rows_max = Tm * k + Tm;
  c->C = f.cache_slots;
  c->router_set.assign(L, 0);
  c->shared_set.assign(L, 0);

  const size_t pool_bytes = (size_t)L * E * c->stride;
  hipError_t e = hipHostMalloc((void**)&c->pool, pool_bytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    c->pool = nullptr;
    destroy_all(c);
    delete c;
    return fail(MOE_ERR_OOM, "pinned host pool of " + std::to_string(pool_bytes) +
                                 " bytes: " + hipGetErrorString(e));
  }
  ALLOC(c->d_router, (size_t)L * H * E * sizeof(float));
  if (f.has_shared) ALLOC(c->d_shared, (size_t)L * c->stride);
  ALLOC(c->d_slots, (size_t)c->C * c->stride);
  ALLOC(c->d_staging, (size_t)f.staging_slots * c->stride);
  ALLOC(c->d_key, (size_t)std::max(c->C, 1) * 4);
  ALLOC(c->d_stamp, (size_t)std::max(c->C, 1) * 8);
  ALLOC(c->d_order, (size_t)std::max(c->C, 1) * 4);
  ALLOC(c->d_order_tmp, (size_t)std::max(c->C, 1) * 4);
  ALLOC(c->d_hitflag, (size_t)std::max(c->C, 1));
  ALLOC(c->d_map, (size_t)L * E * 4);
  ALLOC(c->d_victim, (size_t)c->max_unique * 4);
  ALLOC(c->d_cache, sizeof(DevCache));
  ALLOC(c->d_logits, (size_t)Tm * E * 4);
  ALLOC(c->d_ids, (size_t)Tm * k * 4);
  ALLOC(c->d_gates, (size_t)Tm * k * 4);
  ALLOC(c->d_counts, (size_t)E * 4);
  ALLOC(c->d_offsets, (size_t)(E + 1) * 4);
  ALLOC(c->d_sorted, (size_t)Tm * k * 4);
  ALLOC(c->d_inv, (size_t)Tm * k * 4);
  ALLOC(c->d_unique, (size_t)E * 4);
  ALLOC(c->d_slotcode, (size_t)E * 4);
  ALLOC(c->d_tok, (size_t)c->rows_max * 4);
  ALLOC(c->d_items, (size_t)c->max_items * sizeof(WorkItem));
  ALLOC(c->d_fills, (size_t)c->max_unique * sizeof(FillEntry));
  ALLOC(c->d_meta, sizeof(DevMeta));
  ALLOC(c->d_h, (size_t)c->rows_max * I * 2 * 2);  // hi and lo bf16 planes
  ALLOC(c->d_yperm, (size_t)c->rows_max * H * 4);
  ALLOC(c->d_lookup_ids, (size_t)(E + 1) * 4);

  std::vector<int32_t> key(std::max(c->C, 1), -1), order(std::max(c->C, 1)), map((size_t)L * E, -1);
  std::iota(order.begin(), order.end(), 0);  // all empty: slot | (0 << kOrderKeyShift)
  std::vector<uint64_t> stamp(std::max(c->C, 1), 0);
  std::vector<uint8_t> zero(sizeof(DevCache) > sizeof(DevMeta) ? sizeof(DevCache) : sizeof(DevMeta), 0);
  if (upload(c->d_key, key) != hipSuccess || upload(c->d_order, order) != hipSuccess ||
      upload(c->d_stamp, stamp) != hipSuccess || upload(c->d_map, map) != hipSuccess ||
      hipMemcpy(c->d_cache, zero.data(), sizeof(DevCache), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(c->d_meta, zero.data(), sizeof(DevMeta), hipMemcpyHostToDevice) != hipSuccess) {
    destroy_all(c);
    delete c;
    return fail(MOE_ERR_HIP, "initialising cache state");
  }
  *out = reinterpret_cast<moe_ctx*>(c);
  g_err.clear();
  return MOE_OK;
}

moe_status moe_destroy(moe_ctx* ctx) {
  if (!ctx) return MOE_OK;
  Ctx* c = C_(ctx);
  (void)hipDeviceSynchronize();
  destroy_all(c);
  delete c;
  return MOE_OK;
}

moe_status moe_set_router(moe_ctx* ctx, int32_t layer, const float* h_router) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (layer < 0 || layer >= c->cfg.n_layers || !h_router)
    return fail(MOE_ERR_INVALID_ARG, "bad layer or NULL router");
  const size_t H = c->cfg.hidden, E = c->cfg.n_experts;
  std::vector<float> t(H * E);  // [E][H]: one expert's column contiguous
  for (size_t h = 0; h < H; h++)
    for (size_t e = 0; e < E; e++) t[e * H + h] = h_router[h * E + e];
  HIPCHK(hipMemcpy(c->d_router + (size_t)layer * H * E, t.data(), H * E * 4,
                   hipMemcpyHostToDevice));
  c->router_set[layer] = 1;
  return MOE_OK;
}

moe_status moe_set_expert(moe_ctx* ctx, int32_t layer, int32_t expert,
                          const uint8_t* qg, const uint8_t* qu, const uint8_t* qd,
                          const uint8_t* sg, const uint8_t* su, const uint8_t* sd) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  const int H = c->cfg.hidden, I = c->cfg.inter;
  if (layer < 0 || layer >= c->cfg.n_layers || expert < -1 || expert >= c->cfg.n_experts)
    return fail(MOE_ERR_INVALID_ARG, "bad layer or expert index");
  const bool bf16 = c->cfg.weight_format == MOE_WEIGHTS_BF16;
  if (!qg || !qu || !qd || (!bf16 && (!sg || !su || !sd)))
    return fail(MOE_ERR_INVALID_ARG, "NULL weight pointer");
  if (bf16 && (sg || su || sd))
    return fail(MOE_ERR_INVALID_ARG, "bf16 experts take no scale arrays");
  if (expert == -1 && !c->cfg.has_shared)
    return fail(MOE_ERR_STATE, "context has no shared expert");
  const size_t ns = (size_t)H * I / 32;
  if (!bf16 && (!scales_valid(sg, ns) || !scales_valid(su, ns) || !scales_valid(sd, ns)))
    return fail(MOE_ERR_INVALID_ARG, "E8M0 scale byte 255 (NaN)");
  if (expert >= 0) {
    uint8_t* rec = c->pool + ((size_t)layer * c->cfg.n_experts + expert) * c->stride;
    repack_expert(c, qg, qu, qd, sg, su, sd, rec);
    return MOE_OK;
  }
  std::vector<uint8_t> rec(c->stride, 0);
  repack_expert(c, qg, qu, qd, sg, su, sd, rec.data());
  HIPCHK(hipMemcpy(c->d_shared + (size_t)layer * c->stride, rec.data(), c->stride,
                   hipMemcpyHostToDevice));
  c->shared_set[layer] = 1;
  return MOE_OK;
}

moe_status moe_set_layer(moe_ctx* ctx, int32_t layer, const float* h_router,
                         const uint8_t* h_q, const uint8_t* h_s,
                         const uint8_t* h_shared_q, const uint8_t* h_shared_s) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  const bool bf16 = c->cfg.weight_format == MOE_WEIGHTS_BF16;
  if (layer < 0 || layer >= c->cfg.n_layers || !h_router || !h_q || (!bf16 && !h_s))
    return fail(MOE_ERR_INVALID_ARG, "bad layer or NULL pointer");
  if (bf16 && (h_s || h_shared_s)) return fail(MOE_ERR_INVALID_ARG, "bf16 experts take no scales");
  if (c->cfg.has_shared && (!h_shared_q || (!bf16 && !h_shared_s)))
    return fail(MOE_ERR_INVALID_ARG, "shared expert weights required");
  const size_t H = c->cfg.hidden, I = c->cfg.inter;
  const size_t q1 = bf16 ? H * I * 2 : H * I / 2, s1 = bf16 ? 0 : H * I / 32;
  auto sp = [&](const uint8_t* base, size_t off) { return base ? base + off : nullptr; };
  if (moe_status s = moe_set_router(ctx, layer, h_router)) return s;
  for (int e = 0; e < c->cfg.n_experts; e++) {
    const uint8_t* q = h_q + (size_t)e * 3 * q1;
    const uint8_t* s = sp(h_s, (size_t)e * 3 * s1);
    if (moe_status st = moe_set_expert(ctx, layer, e, q, q + q1, q + 2 * q1, s, sp(s, s1),
                                       sp(s, 2 * s1)))
      return st;
  }
  if (c->cfg.has_shared)
    return moe_set_expert(ctx, layer, -1, h_shared_q, h_shared_q + q1, h_shared_q + 2 * q1,
                          h_shared_s, sp(h_shared_s, s1), sp(h_shared_s, 2 * s1));
  return MOE_OK;
}

moe_status moe_layer_forward(moe_ctx* ctx, int32_t layer, const void* d_x, int32_t T,
                             const float* d_bias, void* d_y, float* d_y32, int32_t* d_ids,
                             float* d_gates, void* stream) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  const moe_config& f = c->cfg;
  if (layer < 0 || layer >= f.n_layers) return fail(MOE_ERR_INVALID_ARG, "bad layer");
  if (T < 0 || T > f.max_tokens) return fail(MOE_ERR_INVALID_ARG, "T outside [0, max_tokens]");
  if (T == 0) return MOE_OK;
  if (!d_x || !d_y) return fail(MOE_ERR_INVALID_ARG, "NULL x or y");
  if (!c->router_set[layer]) return fail(MOE_ERR_STATE, "router of this layer not set");
  if (f.has_shared && !c->shared_set[layer])
    return fail(MOE_ERR_STATE, "shared expert of this layer not set");
  const int worst_bypass =
      std::max(0, std::min(T * f.top_k, f.n_experts) - fillable_slots(c, layer, false, nullptr));
  if (worst_bypass > f.staging_slots)
    return fail(MOE_ERR_CAPACITY, "staging_slots (" + std::to_string(f.staging_slots) +
                                      ") below worst-case bypass count " +
                                      std::to_string(worst_bypass));
  hipStream_t st = (hipStream_t)stream;
  const float* wr = c->d_router + (size_t)layer * f.hidden * f.n_experts;
  HIPCHK(launch_router((const uint16_t*)d_x, T, f.hidden, f.n_experts, wr, d_bias, c->d_logits,
                       st));
  HIPCHK(launch_route_finalize(c, layer, T, d_ids, d_gates, st));
  HIPCHK(launch_fill(c->d_fills, c->d_meta, c->max_unique, c->rec_bytes, st));
  Ctx::TimingRec tr{nullptr, nullptr, nullptr, nullptr};
  if (c->timing && c->t_decode.size() < kMaxTimingPairs) {
    tr = {timing_event(c), timing_event(c), timing_event(c), timing_event(c)};
    if (!(tr.gu0 && tr.gu1 && tr.dn0 && tr.dn1)) tr = {nullptr, nullptr, nullptr, nullptr};
  }
  HIPCHK(launch_expert_gateup(c, (const uint16_t*)d_x, T, st, tr.gu0, tr.gu1));
  HIPCHK(launch_expert_down(c, T, st, tr.dn0, tr.dn1));
  if (tr.gu0) c->t_decode.push_back(tr);
  HIPCHK(launch_combine(c, T, (uint16_t*)d_y, d_y32, st));
  c->host_stats.forward_calls++;
  return MOE_OK;
}

moe_status moe_prefill_forward(moe_ctx* ctx, int32_t n_layers, const void* const* h_x,
                               int32_t T, const float* const* h_bias, void* const* h_y,
                               float* const* h_y32, void* stream) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  const moe_config& f = c->cfg;
  if (f.max_prefill_tokens == 0) return fail(MOE_ERR_STATE, "prefill disabled (max_prefill_tokens = 0)");
  if (n_layers < 1 || n_layers > f.n_layers || !h_x || !h_y)
    return fail(MOE_ERR_INVALID_ARG, "bad n_layers or NULL pointer arrays");
  if (T < 1 || T > f.max_prefill_tokens) return fail(MOE_ERR_INVALID_ARG, "T outside [1, max_prefill_tokens]");
  for (int l = 0; l < n_layers; l++) {
    if (!h_x[l] || !h_y[l]) return fail(MOE_ERR_INVALID_ARG, "NULL x or y pointer");
    if (!c->router_set[l]) return fail(MOE_ERR_STATE, "router not set");
    if (f.has_shared && !c->shared_set[l]) return fail(MOE_ERR_STATE, "shared expert not set");
  }
  hipError_t e = prefill_forward(c, n_layers, h_x, T, h_bias, h_y, h_y32, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return fail(MOE_ERR_UNSUPPORTED, "prefill path not available");
  if (e == hipErrorOutOfMemory) return fail(MOE_ERR_OOM, "prefill buffers");
  HIPCHK(e);
  c->host_stats.prefill_layers += n_layers;
  return MOE_OK;
}

moe_status expert_cache_lookup(moe_ctx* ctx, int32_t layer, const int32_t* d_experts,
                               const int32_t* d_n, int32_t* d_slot, void* stream) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (layer < 0 || layer >= c->cfg.n_layers || !d_experts || !d_n || !d_slot)
    return fail(MOE_ERR_INVALID_ARG, "bad layer or NULL pointer");
  const int worst_bypass = std::max(0, c->max_unique - fillable_slots(c, layer, false, nullptr));
  if (worst_bypass > c->cfg.staging_slots)
    return fail(MOE_ERR_CAPACITY, "staging_slots below worst-case bypass count");
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(launch_cache_lookup(c, layer, d_experts, d_n, c->max_unique, d_slot, false, st));
  HIPCHK(launch_fill(c->d_fills, c->d_meta, c->max_unique, c->rec_bytes, st));
  return MOE_OK;
}

moe_status expert_cache_fill(moe_ctx* ctx, int32_t layer, const int32_t* h_experts,
                             int32_t n, void* stream) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (layer < 0 || layer >= c->cfg.n_layers || n < 0 || n > c->max_unique ||
      (n > 0 && !h_experts))
    return fail(MOE_ERR_INVALID_ARG, "bad layer, count or NULL list");
  for (int i = 0; i < n; i++) {
    if (h_experts[i] < 0 || h_experts[i] >= c->cfg.n_experts)
      return fail(MOE_ERR_INVALID_ARG, "expert id out of range");
    if (i && h_experts[i] <= h_experts[i - 1])
      return fail(MOE_ERR_INVALID_ARG, "expert ids must be ascending and unique");
  }
  if (n == 0) return MOE_OK;
  if (std::max(0, n - fillable_slots(c, layer, true, nullptr)) > c->cfg.staging_slots)
    return fail(MOE_ERR_CAPACITY, "fill would bypass more experts than staging_slots");
  hipStream_t st = (hipStream_t)stream;
  std::vector<int32_t> buf(h_experts, h_experts + n);
  buf.push_back(n);
  HIPCHK(hipStreamSynchronize(st));
  HIPCHK(hipMemcpy(c->d_lookup_ids, buf.data(), buf.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(launch_cache_lookup(c, layer, c->d_lookup_ids, c->d_lookup_ids + n, n, c->d_slotcode, true,
                             st));
  HIPCHK(launch_fill(c->d_fills, c->d_meta, n, c->rec_bytes, st));
  HIPCHK(hipStreamSynchronize(st));
  return MOE_OK;
}

moe_status expert_cache_resize(moe_ctx* ctx, int32_t new_slots, void* stream) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  const int L = c->cfg.n_layers, E = c->cfg.n_experts;
  if (new_slots < 0 || (int64_t)new_slots > (int64_t)L * E)
    return fail(MOE_ERR_INVALID_ARG, "new_slots outside [0, n_layers*n_experts]");
  if (new_slots > kMaxCacheSlots) return fail(MOE_ERR_UNSUPPORTED, "cache_slots above 4096");
  if (c->cfg.cache_policy != MOE_CACHE_GLOBAL)
    return fail(MOE_ERR_UNSUPPORTED, "resize is supported for the global cache policy only");
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(hipStreamSynchronize(st));
  HIPCHK(hipDeviceSynchronize());
  const int C = c->C, C2 = new_slots;
  std::vector<int32_t> key(C);
  std::vector<uint64_t> stamp(C);
  DevCache dc;
  if (C) {
    HIPCHK(hipMemcpy(key.data(), c->d_key, (size_t)C * 4, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(stamp.data(), c->d_stamp, (size_t)C * 8, hipMemcpyDeviceToHost));
  }
  HIPCHK(hipMemcpy(&dc, c->d_cache, sizeof dc, hipMemcpyDeviceToHost));

  // New state: src_of[d] = old slot copied into new slot d (or -1).
  std::vector<int32_t> key2(C2, -1), src_of(C2, -1);
  std::vector<uint64_t> stamp2(C2, 0);
  uint64_t evicted = 0, moved = 0;
  if (C2 >= C) {
    for (int s = 0; s < C; s++)
      if (key[s] >= 0) { key2[s] = key[s]; stamp2[s] = stamp[s]; src_of[s] = s; }
  } else {
    std::vector<int> occ;
    for (int s = 0; s < C; s++) if (key[s] >= 0) occ.push_back(s);
    std::sort(occ.begin(), occ.end(), [&](int a, int b) { return stamp[a] < stamp[b]; });
    std::vector<char> alive(C, 0);
    size_t drop = occ.size() > (size_t)C2 ? occ.size() - C2 : 0;
    for (size_t i = drop; i < occ.size(); i++) alive[occ[i]] = 1;
    evicted = drop;
    std::vector<int> free_low;
    for (int s = 0; s < C2; s++) {
      if (alive[s]) { key2[s] = key[s]; stamp2[s] = stamp[s]; src_of[s] = s; }
      else free_low.push_back(s);
    }
    size_t fi = 0;
    for (int s = C2; s < C; s++)
      if (alive[s]) {
        const int d = free_low[fi++];
        key2[d] = key[s]; stamp2[d] = stamp[s]; src_of[d] = s;
        moved++;
      }
  }
  // Move the surviving records into a slot buffer of the new size.
  uint8_t* slots2 = nullptr;
  if (C2 && hipMalloc((void**)&slots2, (size_t)C2 * c->stride) != hipSuccess)
    return fail(MOE_ERR_OOM, "resized slot buffer");
  std::vector<FillEntry> pairs;
  for (int d = 0; d < C2; d++)
    if (src_of[d] >= 0)
      pairs.push_back({c->d_slots + (size_t)src_of[d] * c->stride, slots2 + (size_t)d * c->stride});
  if (!pairs.empty()) {
    FillEntry* dp = nullptr;
    HIPCHK(hipMalloc((void**)&dp, pairs.size() * sizeof(FillEntry)));
    HIPCHK(hipMemcpy(dp, pairs.data(), pairs.size() * sizeof(FillEntry), hipMemcpyHostToDevice));
    HIPCHK(launch_copy_pairs(dp, (int)pairs.size(), c->rec_bytes, st));
    HIPCHK(hipStreamSynchronize(st));
    HIPCHK(hipFree(dp));
  }
  dfree(c->d_slots);
  c->d_slots = slots2;
  // Recency order: empty slots by index, then occupied by stamp.
  std::vector<int32_t> order(C2);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return (key2[a] < 0 ? 0 : stamp2[a]) < (key2[b] < 0 ? 0 : stamp2[b]);
  });
  for (auto& o : order) o |= (key2[o] + 1) << kOrderKeyShift;
  std::vector<int32_t> map((size_t)L * E, -1);
  for (int s = 0; s < C2; s++) if (key2[s] >= 0) map[key2[s]] = s;
  dfree(c->d_key); dfree(c->d_stamp); dfree(c->d_order); dfree(c->d_order_tmp); dfree(c->d_hitflag);
  const size_t n1 = std::max(C2, 1);
  if (hipMalloc((void**)&c->d_key, n1 * 4) != hipSuccess ||
      hipMalloc((void**)&c->d_stamp, n1 * 8) != hipSuccess ||
      hipMalloc((void**)&c->d_order, n1 * 4) != hipSuccess ||
      hipMalloc((void**)&c->d_order_tmp, n1 * 4) != hipSuccess ||
      hipMalloc((void**)&c->d_hitflag, n1) != hipSuccess)
    return fail(MOE_ERR_OOM, "resized cache state");
  HIPCHK(upload(c->d_key, key2));
  HIPCHK(upload(c->d_stamp, stamp2));
  HIPCHK(upload(c->d_order, order));
  HIPCHK(upload(c->d_map, map));
  dc.evictions += evicted;
  HIPCHK(hipMemcpy(c->d_cache, &dc, sizeof dc, hipMemcpyHostToDevice));
  c->C = C2;
  c->host_stats.resizes++;
  c->host_stats.bytes_d2d += moved * c->rec_bytes;
  return MOE_OK;
}

moe_status expert_cache_snapshot(moe_ctx* ctx, int32_t capacity, int32_t* h_key,
                                 uint64_t* h_stamp, uint64_t* h_clock, int32_t* h_slots) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  if (!h_slots) return fail(MOE_ERR_INVALID_ARG, "h_slots is NULL");
  *h_slots = c->C;
  if (capacity < c->C) return fail(MOE_ERR_CAPACITY, "snapshot capacity below cache size");
  if ((c->C && (!h_key || !h_stamp)) || !h_clock)
    return fail(MOE_ERR_INVALID_ARG, "NULL snapshot array");
  HIPCHK(hipDeviceSynchronize());
  if (c->C) {
    HIPCHK(hipMemcpy(h_key, c->d_key, (size_t)c->C * 4, hipMemcpyDeviceToHost));
    HIPCHK(hipMemcpy(h_stamp, c->d_stamp, (size_t)c->C * 8, hipMemcpyDeviceToHost));
  }
  DevCache dc;
  HIPCHK(hipMemcpy(&dc, c->d_cache, sizeof dc, hipMemcpyDeviceToHost));
  *h_clock = dc.clock;
  return MOE_OK;
}

moe_status moe_inspect_dispatch(moe_ctx* ctx, int32_t* h_T, int32_t* h_counts,
                                int32_t* h_offsets, int32_t* h_sorted, int32_t* h_inv,
                                int32_t* h_unique, int32_t* h_n_unique, int32_t* h_slot) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  HIPCHK(hipDeviceSynchronize());
  DevMeta m;
  HIPCHK(hipMemcpy(&m, c->d_meta, sizeof m, hipMemcpyDeviceToHost));
  const int E = c->cfg.n_experts, nk = m.T * c->cfg.top_k;
  if (h_T) *h_T = m.T;
  if (h_n_unique) *h_n_unique = m.n_unique;
  if (h_counts) HIPCHK(hipMemcpy(h_counts, c->d_counts, (size_t)E * 4, hipMemcpyDeviceToHost));
  if (h_offsets) HIPCHK(hipMemcpy(h_offsets, c->d_offsets, (size_t)(E + 1) * 4, hipMemcpyDeviceToHost));
  if (h_sorted && nk) HIPCHK(hipMemcpy(h_sorted, c->d_sorted, (size_t)nk * 4, hipMemcpyDeviceToHost));
  if (h_inv && nk) HIPCHK(hipMemcpy(h_inv, c->d_inv, (size_t)nk * 4, hipMemcpyDeviceToHost));
  if (h_unique && m.n_unique)
    HIPCHK(hipMemcpy(h_unique, c->d_unique, (size_t)m.n_unique * 4, hipMemcpyDeviceToHost));
  if (h_slot && m.n_unique)
    HIPCHK(hipMemcpy(h_slot, c->d_slotcode, (size_t)m.n_unique * 4, hipMemcpyDeviceToHost));
  return MOE_OK;
}

moe_status moe_inspect_prefill(moe_ctx* ctx, int32_t* h_T, int32_t* h_ids, float* h_gates) {
  if (moe_status s = check_ctx(ctx)) return s;
  if (!h_T) return fail(MOE_ERR_INVALID_ARG, "h_T is NULL");
  HIPCHK(prefill_inspect(C_(ctx), h_T, h_ids, h_gates));
  return MOE_OK;
}

moe_status moe_get_stats(moe_ctx* ctx, moe_stats* out) {
  if (moe_status s = check_ctx(ctx)) return s;
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  Ctx* c = C_(ctx);
  HIPCHK(hipDeviceSynchronize());
  DevCache dc;
  HIPCHK(hipMemcpy(&dc, c->d_cache, sizeof dc, hipMemcpyDeviceToHost));
  *out = c->host_stats;
  out->lookups = dc.lookups;
  out->hits = dc.hits;
  out->fills = dc.fills;
  out->bypasses = dc.bypasses;
  out->evictions = dc.evictions;
  out->bytes_h2d = (dc.fills + dc.bypasses) * c->rec_bytes;
  return MOE_OK;
}

moe_status moe_reset_stats(moe_ctx* ctx) {
  if (moe_status s = check_ctx(ctx)) return s;
  Ctx* c = C_(ctx);
  HIPCHK(hipDeviceSynchronize());
  DevCache dc;
  HIPCHK(hipMemcpy(&dc, c->d_cache, sizeof dc, hipMemcpyDeviceToHost));
  const uint64_t clock = dc.clock;
  dc = DevCache{};
  dc.clock = clock;
  HIPCHK(hipMemcpy(c->d_cache, &dc, sizeof dc, hipMemcpyHostToDevice));
  c->host_stats = moe_stats{};
  return MOE_OK;
}

moe_status moe_set_timing(moe_ctx* ctx, int32_t enable) {
  if (moe_status s = check_ctx(ctx)) return s;
  C_(ctx)->timing = enable != 0;
  return MOE_OK;
}

static hipError_t sum_timing(const std::vector<Ctx::TimingRec>& v, double* ms3) {
  double s[3] = {0, 0, 0};
  for (const auto& r : v) {
    float a = 0, b = 0;
    hipError_t e = hipEventElapsedTime(&a, r.gu0, r.gu1);
    if (e == hipSuccess) e = hipEventElapsedTime(&b, r.dn0, r.dn1);
    if (e != hipSuccess) return e;
    s[0] += (double)a + b;
    s[1] += a;
    s[2] += b;
  }
  for (int i = 0; i < 3; i++) ms3[i] = s[i];
  return hipSuccess;
}

static moe_status take_timing(Ctx* c, int32_t* n2, double* ms6) {
  HIPCHK(hipDeviceSynchronize());
  n2[0] = (int32_t)c->t_decode.size();
  n2[1] = (int32_t)c->t_prefill.size();
  HIPCHK(sum_timing(c->t_decode, ms6));
  HIPCHK(sum_timing(c->t_prefill, ms6 + 3));
  c->t_decode.clear();
  c->t_prefill.clear();
  c->ev_next = 0;
  return MOE_OK;
}

moe_status moe_get_timing(moe_ctx* ctx, int32_t* h_n_decode, double* h_ms_decode,
                          int32_t* h_n_prefill, double* h_ms_prefill) {
  if (moe_status s = check_ctx(ctx)) return s;
  int32_t n[2];
  double ms[6];
  if (moe_status s = take_timing(C_(ctx), n, ms)) return s;
  if (h_n_decode) *h_n_decode = n[0];
  if (h_n_prefill) *h_n_prefill = n[1];
  if (h_ms_decode) *h_ms_decode = ms[0];
  if (h_ms_prefill) *h_ms_prefill = ms[3];
  return MOE_OK;
}

moe_status moe_get_timing_split(moe_ctx* ctx, int32_t* h_n, double* h_ms) {
  if (moe_status s = check_ctx(ctx)) return s;
  if (!h_n || !h_ms) return fail(MOE_ERR_INVALID_ARG, "NULL output array");
  return take_timing(C_(ctx), h_n, h_ms);
}

moe_status moe_probe_copy(const void* d_src, void* d_dst, size_t n_bytes, void* stream) {
  if (!d_src || !d_dst || n_bytes % 16) return fail(MOE_ERR_INVALID_ARG, "bad copy arguments");
  if (!n_bytes) return MOE_OK;
  HIPCHK(launch_probe_copy(d_src, d_dst, n_bytes, (hipStream_t)stream));
  return MOE_OK;
}

}  // extern "C"
