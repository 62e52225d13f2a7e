// Decode expert FFN: grouped skinny GEMMs over the experts of one call.
//
// Each expert of the call has 1..T tokens.  Its weights are streamed once
// from HBM in 1088-byte MXFP4 atoms (one 16-byte load per lane, one lane per
// MX block), dequantised in registers with the gfx950 scaled FP4 -> bf16
// convert, and multiplied on v_mfma_f32_16x16x32_bf16 with up to 16 tokens as
// the A operand.  The kernels are HBM-bound, so the design is about bytes in
// flight: a workgroup owns one output tile (a 16-row gate/up pair, or two
// 16-row down row groups) of one expert and splits K over up to 16 waves,
// and the waves' partial tiles are summed through LDS in a fixed order
// (results do not depend on where an expert's weights live).  Calls of up
// to 16 tokens use the streaming kernels (a wave walks its K range in steps
// of two chunks with two steps of loads in flight; chunks per wave set per
// shape by the launcher); larger calls use the kernels that issue all of a
// wave's loads before its first MFMA and loop over 16-token M tiles.  MFMA
// replaces the per-lane dot products and wave reductions of a VALU GEMV,
// keeping VALU work per weight byte flat in the token count.
//
// FFN: o = W_d (silu(W_g x) * (W_u x)); the pages name MXFP4 experts
// (jansverre.net FreeToken article, section "Hvor raskt kjører modellene?")
// but not the FFN form, which is SwiGLU here.  h passes between the two
// kernels as a hi/lo pair of bf16 values (two MFMAs per weight fragment in
// the down kernel, free while HBM-bound), so it keeps ~16 significant bits.
#include <algorithm>

#include "moe_internal.h"
#include "nvfp4_dequant.h"

namespace moe {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxWaves = 16;

__device__ __forceinline__ float scale_of(uint32_t sbyte) { return __uint_as_float(sbyte << 23); }

// 8 E2M1 codes (one dword, low nibble first) times 2^(sbyte-127) -> 8 bf16.
// The convert reads only the exponent field of its fp32 scale operand.
__device__ __forceinline__ bf16x8 dequant8(uint32_t q, uint32_t sbyte) {
  const float s = scale_of(sbyte);
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 3));
  return __builtin_bit_cast(bf16x8, r);
}

using nvfp4::dequant8_nv;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float silu(float a) { return a / (1.0f + expf(-a)); }

// Workgroup barrier for the LDS reduction: waits for LDS operations only, so
// the output stores of one M tile stay in flight across it (__syncthreads()
// would drain them first).  No thread reads another's global stores.
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}


// Global-address-space loads (global_load rather than flat_load) of the
// weights.  NT: nontemporal, so that the atoms, which a call streams once,
// are not allocated in L2 or the Infinity Cache (the launchers choose it
// where the cache slots cannot stay in the Infinity Cache anyway).
template <bool NT, class V>
__device__ __forceinline__ V load_weights(const uint8_t* p) {
  typedef __attribute__((address_space(1))) const V gv;
  if constexpr (NT)
    return __builtin_nontemporal_load((gv*)p);
  else
    return *(gv*)p;
}
template <bool NT>
__device__ __forceinline__ u32x4 load_atom_data(const uint8_t* atom, int lane) {
  return load_weights<NT, u32x4>(atom + lane * 16);
}
template <bool NT>
__device__ __forceinline__ uint32_t load_scale(const uint8_t* atom, int lane) {
  return load_weights<NT, uint8_t>(atom + kAtomData + lane);
}

// Activation loads go through a bounds-checked buffer resource: a lane whose
// row does not exist passes an out-of-range offset and reads zeros without
// touching memory (no branch, no wait at a branch join).
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8 bload8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Epilogues shared by the kernels below: the waves' partial 16x16 tiles in
// red[wave][tile][lane] are summed in wave order (a fixed order, so results
// do not depend on scheduling).
//
// Gate/up: h for tokens m0 .. m0+15 of the item, columns 16p .. 16p+15, as
// hi = RNE(h) and lo = RNE(h - hi).
__device__ __forceinline__ void gateup_epilogue(const f32x4* red, int nw, const WorkItem& it,
                                                int m0, int p, int I, uint16_t* __restrict__ h,
                                                size_t lo_plane) {
  for (int v0 = threadIdx.x; v0 < 256; v0 += blockDim.x) {  // 64 lanes x 4 values
    const int L = v0 >> 2, i = v0 & 3;
    float gs = 0.f, us = 0.f;
    for (int v = 0; v < nw; v++) {
      gs += red[(2 * v) * 64 + L][i];
      us += red[(2 * v + 1) * 64 + L][i];
    }
    const int mm = m0 + 4 * (L >> 4) + i;
    if (mm < it.cnt) {
      const float hv = silu(gs) * us;
      const uint16_t hi = f32_to_bf16_rne(hv);
      const size_t o = (size_t)(it.pos0 + mm) * I + p * 16 + (L & 15);
      h[o] = hi;
      h[lo_plane + o] = f32_to_bf16_rne(hv - bf16_to_f32(hi));
    }
  }
}
// Down: rows 32q .. 32q+31 of H (tiles g = 0, 1) for tokens m0 .. m0+15.
__device__ __forceinline__ void down_epilogue(const f32x4* red, int nw, const WorkItem& it, int m0,
                                              int q, int H, float* __restrict__ yperm) {
  for (int v0 = threadIdx.x; v0 < 512; v0 += blockDim.x) {  // 2 tiles x 64 lanes x 4 values
    const int g = v0 >> 8, L = (v0 >> 2) & 63, i = v0 & 3;
    float s = 0.f;
    for (int v = 0; v < nw; v++) s += red[(2 * v + g) * 64 + L][i];
    const int mm = m0 + 4 * (L >> 4) + i;
    if (mm < it.cnt) yperm[(size_t)(it.pos0 + mm) * H + (2 * q + g) * 16 + (L & 15)] = s;
  }
}

// Weight-format policies of the expert kernels: how a lane loads its part of
// an atom and forms the bf16x8 operand of K step j (4 steps per atom).  NT:
// the weight loads are nontemporal.
template <bool NT>
struct WMxfp4 {
  static constexpr int kAtom = kAtomBytes;
  static constexpr int kStep = 2;
  static constexpr int kMaxThreads = 1024;
  static constexpr bool kMatrixScale = false;
  struct Reg {
    u32x4 q;
    uint32_t s;
  };
  __device__ static void load_data(Reg& r, const uint8_t* atom, int lane) {
    r.q = load_atom_data<NT>(atom, lane);
  }
  __device__ static void load_aux(Reg& r, const uint8_t* atom, int lane) {
    r.s = load_scale<NT>(atom, lane);
  }
  __device__ static bf16x8 op(const Reg& r, int j) { return dequant8(r.q[j], r.s); }
  __device__ static void hide(Reg& r) { asm volatile("" : "+v"(r.q), "+v"(r.s)); }
};
template <bool NT>
struct WBf16 {
  static constexpr int kAtom = kAtomBytesBF16;
  static constexpr int kStep = 1;
  static constexpr int kMaxThreads = 512;
  static constexpr bool kMatrixScale = false;
  struct Reg {
    u32x4 v[4];
  };
  __device__ static void load_data(Reg& r, const uint8_t* atom, int lane) {
#pragma unroll
    for (int p = 0; p < 4; p++) r.v[p] = load_weights<NT, u32x4>(atom + 1024 * p + lane * 16);
  }
  __device__ static void load_aux(Reg&, const uint8_t*, int) {}
  __device__ static bf16x8 op(const Reg& r, int j) { return __builtin_bit_cast(bf16x8, r.v[j]); }
  __device__ static void hide(Reg& r) {
    asm volatile("" : "+v"(r.v[0]), "+v"(r.v[1]), "+v"(r.v[2]), "+v"(r.v[3]));
  }
};
// NVFP4: the MXFP4 code layout; the lane's two E4M3 block scales (K steps 0-1
// and 2-3 of its 32 elements) in one 16-bit load; the matrix's fp32 scale
// multiplies the accumulators.
template <bool NT>
struct WNvfp4 {
  static constexpr int kAtom = kAtomBytesNV;
  static constexpr int kStep = 2;
  static constexpr int kMaxThreads = 1024;
  static constexpr bool kMatrixScale = true;
  struct Reg {
    u32x4 q;
    uint32_t s;
  };
  __device__ static void load_data(Reg& r, const uint8_t* atom, int lane) {
    r.q = load_atom_data<NT>(atom, lane);
  }
  __device__ static void load_aux(Reg& r, const uint8_t* atom, int lane) {
    r.s = load_weights<NT, uint16_t>(atom + kAtomData + 2 * lane);
  }
  __device__ static bf16x8 op(const Reg& r, int j) {
    return dequant8_nv(r.q[j], (r.s >> (8 * (j >> 1))) & 0xFFu);
  }
  __device__ static void hide(Reg& r) { asm volatile("" : "+v"(r.q), "+v"(r.s)); }
};

// Gate/up + SwiGLU for calls of more than 16 tokens.  Block (pair p, item):
// 16 gate and 16 up rows of one expert; wave w takes K chunks
// [w*CPW, w*CPW+CPW), all loaded before its first MFMA.  M tiles of 16
// tokens are processed one after another with the weights held in
// registers.
template <int CPW, class W>
__global__ __launch_bounds__(W::kMaxThreads) void gateup_decode_kernel(
    const WorkItem* __restrict__ items, int items_cap, const int32_t* __restrict__ lo_p,
    const int32_t* __restrict__ hi_p,
    const int32_t* __restrict__ tok, const uint16_t* __restrict__ x, uint32_t x_bytes, int H,
    int I, uint16_t* __restrict__ h, size_t lo_plane, size_t ms_off) {
  // the launch covers items [*lo_p, *hi_p) of the work list (items_cap
  // entries; hi <= items_cap)
  const int item = *lo_p + blockIdx.y;
  // The item load is issued with the bound loads (clamped into the array,
  // so that it needs no bound first): one memory latency before the weight
  // loads instead of two.  The exit
  // test reads the whole item (a real item has cnt >= 1 and a weight
  // pointer) so the compiler cannot sink the item load below it.
  const int n_items = *hi_p;
  const WorkItem it = items[item < items_cap ? item : items_cap - 1];
  if ((item >= n_items) | (it.cnt < 1) | (it.w == nullptr)) return;
  const int p = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int KC = H / kAtomK;
  const uint8_t* gbase = it.w + (size_t)(2 * p) * KC * W::kAtom;
  const uint8_t* ubase = gbase + (size_t)KC * W::kAtom;
  extern __shared__ f32x4 red[];  // [waves][2][64], sized by the launch
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, x_bytes);
  // the gate and up matrices' fp32 scales (at ms_off of the record)
  float msg = 1.0f, msu = 1.0f;
  if constexpr (W::kMatrixScale) {
    const float* ms = reinterpret_cast<const float*>(it.w + ms_off);
    msg = ms[0];
    msu = ms[1];
  }

  // Token row of this lane in the first M tile.
  const int trow = (lane & 15) < it.cnt ? tok[it.pos0 + (lane & 15)] : 0;
  // Weight loads are unconditional: a chunk past K (only when waves do not
  // divide K) reads chunk 0, whose finite values meet zero activations.
  // A guarded load would wait at its branch instead of staying in flight.
  typename W::Reg wg[CPW], wu[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; cc++) {
    const int c = w * CPW + cc;
    const uint8_t* ga = gbase + (size_t)(c < KC ? c : 0) * W::kAtom;
    const uint8_t* ua = ubase + (size_t)(c < KC ? c : 0) * W::kAtom;
    W::load_data(wg[cc], ga, lane);
    W::load_data(wu[cc], ua, lane);
    W::load_aux(wg[cc], ga, lane);
    W::load_aux(wu[cc], ua, lane);
  }

  // One M tile of 16 tokens.  The first tile is peeled out of the loop so
  // that its loads are scheduled against the weight loads precisely.
  auto tile = [&](int m0, int trow) {
    const int m = m0 + (lane & 15);
    const bool mok = m < it.cnt;
    // byte offset of this lane's 32 activations in chunk c, or out of range
    const uint32_t xrow = (uint32_t)(trow * H + 32 * (lane >> 4)) * 2u;
    auto xoff = [&](int c) { return (mok && c < KC) ? xrow + (uint32_t)c * kAtomK * 2u : kOutOfRange; };
    // activation fragments (L2-resident) are fetched one chunk ahead
    bf16x8 xa[2][4];
    {
      const uint32_t o = xoff(w * CPW);
#pragma unroll
      for (int j = 0; j < 4; j++) xa[0][j] = bload8(rx, o + 16u * j);
    }
    f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < CPW; cc++) {
      const int c = w * CPW + cc;
      if (cc + 1 < CPW) {
        const uint32_t o = xoff(c + 1);
#pragma unroll
        for (int j = 0; j < 4; j++) xa[(cc + 1) & 1][j] = bload8(rx, o + 16u * j);
      }
      if (cc == 0) {
        // The packed weights stay in registers across M tiles; hiding them
        // from loop-invariant motion keeps the (4x larger) dequantised
        // fragments from being hoisted out of the tile loop and held live.
#pragma unroll
        for (int q = 0; q < CPW; q++) {
          W::hide(wg[q]);
          W::hide(wu[q]);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[cc & 1][j], W::op(wg[cc], j), ag, 0, 0, 0);
        au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[cc & 1][j], W::op(wu[cc], j), au, 0, 0, 0);
        // keep each fragment's dequant next to its MFMAs (bounds live registers)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (W::kMatrixScale) {
      ag *= msg;
      au *= msu;
    }
    red[(2 * w) * 64 + lane] = ag;
    red[(2 * w + 1) * 64 + lane] = au;
    lds_sync();
    gateup_epilogue(red, nw, it, m0, p, I, h, lo_plane);
    lds_sync();
  };
  tile(0, trow);
  for (int m0 = 16; m0 < it.cnt; m0 += 16) {
    const int m = m0 + (lane & 15);
    tile(m0, m < it.cnt ? tok[it.pos0 + m] : 0);
  }
}

// Down projection for calls of more than 16 tokens.  Block (row-group pair
// q, item): rows [32q, 32q+32) of H of one expert, as two 16-row groups that
// share every h fragment; waves split K = I; each weight fragment meets both
// h planes.
template <int CPW, class W>
__global__ __launch_bounds__(W::kMaxThreads) void down_decode_kernel(
    const WorkItem* __restrict__ items, int items_cap, const int32_t* __restrict__ lo_p,
    const int32_t* __restrict__ hi_p,
    const uint16_t* __restrict__ h, size_t lo_plane, int H, int I, size_t gateup_bytes,
    float* __restrict__ yperm, size_t ms_off) {
  // the launch covers items [*lo_p, *hi_p) of the work list (items_cap
  // entries; hi <= items_cap)
  const int item = *lo_p + blockIdx.y;
  // The item load is issued with the bound loads (clamped into the array,
  // so that it needs no bound first): one memory latency before the weight
  // loads instead of two.  The exit
  // test reads the whole item (a real item has cnt >= 1 and a weight
  // pointer) so the compiler cannot sink the item load below it.
  const int n_items = *hi_p;
  const WorkItem it = items[item < items_cap ? item : items_cap - 1];
  if ((item >= n_items) | (it.cnt < 1) | (it.w == nullptr)) return;
  const int q = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int KC = I / kAtomK;
  const uint8_t* abase = it.w + gateup_bytes + (size_t)(2 * q) * KC * W::kAtom;
  const uint8_t* bbase = abase + (size_t)KC * W::kAtom;
  extern __shared__ f32x4 red[];  // [waves][2][64], sized by the launch
  const uint32_t lo_bytes = (uint32_t)(lo_plane * 2);
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(h, 2 * lo_bytes);
  // the down matrix's fp32 scale (at ms_off of the record)
  float msd = 1.0f;
  if constexpr (W::kMatrixScale) msd = reinterpret_cast<const float*>(it.w + ms_off)[2];

  // Unconditional weight loads, as in the gate/up kernel.
  typename W::Reg wa[CPW], wb[CPW];
#pragma unroll
  for (int cc = 0; cc < CPW; cc++) {
    const int c = w * CPW + cc;
    const size_t o = (size_t)(c < KC ? c : 0) * W::kAtom;
    W::load_data(wa[cc], abase + o, lane);
    W::load_data(wb[cc], bbase + o, lane);
    W::load_aux(wa[cc], abase + o, lane);
    W::load_aux(wb[cc], bbase + o, lane);
  }

  // One M tile of 16 tokens (first tile peeled, as in the gate/up kernel).
  auto tile = [&](int m0) {
    const int m = m0 + (lane & 15);
    const bool mok = m < it.cnt;
    const uint32_t hrow = (uint32_t)((it.pos0 + m) * I + 32 * (lane >> 4)) * 2u;
    auto hoff = [&](int c) { return (mok && c < KC) ? hrow + (uint32_t)c * kAtomK * 2u : kOutOfRange; };
    // h fragments (L2-resident, hi and lo planes) are fetched one chunk ahead
    bf16x8 ahi[2][4], alo[2][4];
    {
      const uint32_t o = hoff(w * CPW);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        ahi[0][j] = bload8(rh, o + 16u * j);
        alo[0][j] = bload8(rh, o == kOutOfRange ? o : o + lo_bytes + 16u * j);
      }
    }
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < CPW; cc++) {
      const int c = w * CPW + cc;
      if (cc + 1 < CPW) {
        const uint32_t o = hoff(c + 1);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          ahi[(cc + 1) & 1][j] = bload8(rh, o + 16u * j);
          alo[(cc + 1) & 1][j] = bload8(rh, o == kOutOfRange ? o : o + lo_bytes + 16u * j);
        }
      }
      if (cc == 0) {
#pragma unroll
        for (int r = 0; r < CPW; r++) {
          W::hide(wa[r]);
          W::hide(wb[r]);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const bf16x8 b0 = W::op(wa[cc], j);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[cc & 1][j], b0, acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[cc & 1][j], b0, acc0, 0, 0, 0);
        const bf16x8 b1 = W::op(wb[cc], j);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[cc & 1][j], b1, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[cc & 1][j], b1, acc1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (W::kMatrixScale) {
      acc0 *= msd;
      acc1 *= msd;
    }
    red[(2 * w) * 64 + lane] = acc0;
    red[(2 * w + 1) * 64 + lane] = acc1;
    lds_sync();
    down_epilogue(red, nw, it, m0, q, H, yperm);
    lds_sync();
  };
  tile(0);
  for (int m0 = 16; m0 < it.cnt; m0 += 16) tile(m0);
}

// Weight formats of the streaming kernels.  A lane holds its part of an atom
// (row l % 16, K block l / 16 of a 16-row x 128-K tile) in registers and
// turns K step j into the MFMA's bf16x8 operand: MXFP4 as one 16-byte load
// of codes plus the scale byte, dequantised per step; bf16 as four 16-byte
// pieces used as they are.  kStep: chunks per load step (a bf16 chunk holds
// four times the bytes); kMaxThreads: workgroup size limit (bf16 keeps 8
// waves, which leaves its larger operands 256 registers a lane).
// Streaming variants for calls of at most 16 tokens (one M tile).  A wave
// covers CPW consecutive K chunks in steps of two chunks with two steps of
// weight loads in flight (double-buffered registers), so a wave can cover
// more of K than it can hold.  The launch then needs fewer waves, and with
// CPW chosen from the kernels' occupancy every workgroup of the call is
// resident at once: a second round of workgroups would wait out the memory
// latency a second time.  Same data layout, reduction order and epilogues
// as above.
template <int CPW, class W>
__global__ __launch_bounds__(W::kMaxThreads) void gateup_stream_kernel(
    const WorkItem* __restrict__ items, int items_cap, const int32_t* __restrict__ lo_p,
    const int32_t* __restrict__ hi_p,
    const int32_t* __restrict__ tok, const uint16_t* __restrict__ x, uint32_t x_bytes, int H,
    int I, uint16_t* __restrict__ h, size_t lo_plane, size_t ms_off) {
  constexpr int S = CPW < W::kStep ? CPW : W::kStep;  // chunks per step
  constexpr int NS = CPW / S;           // steps
  // the launch covers items [*lo_p, *hi_p) of the work list (items_cap
  // entries; hi <= items_cap)
  const int item = *lo_p + blockIdx.y;
  // The item load is issued with the bound loads (clamped into the array,
  // so that it needs no bound first): one memory latency before the weight
  // loads instead of two.  The exit
  // test reads the whole item (a real item has cnt >= 1 and a weight
  // pointer) so the compiler cannot sink the item load below it.
  const int n_items = *hi_p;
  const WorkItem it = items[item < items_cap ? item : items_cap - 1];
  if ((item >= n_items) | (it.cnt < 1) | (it.w == nullptr)) return;
  const int p = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int KC = H / kAtomK;
  const int c0 = w * CPW;
  const uint8_t* gbase = it.w + (size_t)(2 * p) * KC * W::kAtom;
  const uint8_t* ubase = gbase + (size_t)KC * W::kAtom;
  extern __shared__ f32x4 red[];  // [waves][2][64], sized by the launch
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, x_bytes);
  // the gate and up matrices' fp32 scales (at ms_off of the record)
  float msg = 1.0f, msu = 1.0f;
  if constexpr (W::kMatrixScale) {
    const float* ms = reinterpret_cast<const float*>(it.w + ms_off);
    msg = ms[0];
    msu = ms[1];
  }

  // The token row first: loads return in order, so a token index loaded
  // after the weights would hold the activation loads back until every
  // weight load had landed.
  const int m = lane & 15;
  const bool mok = m < it.cnt;
  const int trow = mok ? tok[it.pos0 + m] : 0;

  // Weight loads of step st into buffer b; a chunk past K reads chunk 0
  // (finite values that meet zero activations), as in the kernels above.
  typename W::Reg wg[2][S], wu[2][S];
  auto load_step = [&](int st, int b) {
#pragma unroll
    for (int cc = 0; cc < S; cc++) {
      const int c = c0 + st * S + cc;
      const size_t o = (size_t)(c < KC ? c : 0) * W::kAtom;
      W::load_data(wg[b][cc], gbase + o, lane);
      W::load_data(wu[b][cc], ubase + o, lane);
      W::load_aux(wg[b][cc], gbase + o, lane);
      W::load_aux(wu[b][cc], ubase + o, lane);
    }
  };
  load_step(0, 0);
  if (NS > 1) load_step(1, 1);

  const uint32_t xrow = (uint32_t)(trow * H + 32 * (lane >> 4)) * 2u;
  auto xoff = [&](int c) { return (mok && c < KC) ? xrow + (uint32_t)c * kAtomK * 2u : kOutOfRange; };
  bf16x8 xa[2][4];  // activation fragments, fetched one chunk ahead
  {
    const uint32_t o = xoff(c0);
#pragma unroll
    for (int j = 0; j < 4; j++) xa[0][j] = bload8(rx, o + 16u * j);
  }
  f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < NS; st++) {
    const int b = st & 1;
#pragma unroll
    for (int cc = 0; cc < S; cc++) {
      const int q = st * S + cc;
      if (q + 1 < CPW) {
        const uint32_t o = xoff(c0 + q + 1);
#pragma unroll
        for (int j = 0; j < 4; j++) xa[(q + 1) & 1][j] = bload8(rx, o + 16u * j);
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        ag = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[q & 1][j], W::op(wg[b][cc], j), ag, 0, 0, 0);
        au = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[q & 1][j], W::op(wu[b][cc], j), au, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // refill the buffer this step consumed
    if (st + 2 < NS) load_step(st + 2, b);
  }
  if constexpr (W::kMatrixScale) {
    ag *= msg;
    au *= msu;
  }
  red[(2 * w) * 64 + lane] = ag;
  red[(2 * w + 1) * 64 + lane] = au;
  lds_sync();
  gateup_epilogue(red, nw, it, 0, p, I, h, lo_plane);
}

template <int CPW, class W>
__global__ __launch_bounds__(W::kMaxThreads) void down_stream_kernel(
    const WorkItem* __restrict__ items, int items_cap, const int32_t* __restrict__ lo_p,
    const int32_t* __restrict__ hi_p,
    const uint16_t* __restrict__ h, size_t lo_plane, int H, int I, size_t gateup_bytes,
    float* __restrict__ yperm, size_t ms_off) {
  constexpr int S = CPW < W::kStep ? CPW : W::kStep;
  constexpr int NS = CPW / S;
  // the launch covers items [*lo_p, *hi_p) of the work list (items_cap
  // entries; hi <= items_cap)
  const int item = *lo_p + blockIdx.y;
  // The item load is issued with the bound loads (clamped into the array,
  // so that it needs no bound first): one memory latency before the weight
  // loads instead of two.  The exit
  // test reads the whole item (a real item has cnt >= 1 and a weight
  // pointer) so the compiler cannot sink the item load below it.
  const int n_items = *hi_p;
  const WorkItem it = items[item < items_cap ? item : items_cap - 1];
  if ((item >= n_items) | (it.cnt < 1) | (it.w == nullptr)) return;
  const int q = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int KC = I / kAtomK;
  const int c0 = w * CPW;
  const uint8_t* abase = it.w + gateup_bytes + (size_t)(2 * q) * KC * W::kAtom;
  const uint8_t* bbase = abase + (size_t)KC * W::kAtom;
  extern __shared__ f32x4 red[];  // [waves][2][64], sized by the launch
  const uint32_t lo_bytes = (uint32_t)(lo_plane * 2);
  // the down matrix's fp32 scale (at ms_off of the record)
  float msd = 1.0f;
  if constexpr (W::kMatrixScale) msd = reinterpret_cast<const float*>(it.w + ms_off)[2];
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(h, 2 * lo_bytes);

  typename W::Reg wa[2][S], wb[2][S];
  auto load_step = [&](int st, int b) {
#pragma unroll
    for (int cc = 0; cc < S; cc++) {
      const int c = c0 + st * S + cc;
      const size_t o = (size_t)(c < KC ? c : 0) * W::kAtom;
      W::load_data(wa[b][cc], abase + o, lane);
      W::load_data(wb[b][cc], bbase + o, lane);
      W::load_aux(wa[b][cc], abase + o, lane);
      W::load_aux(wb[b][cc], bbase + o, lane);
    }
  };
  load_step(0, 0);
  if (NS > 1) load_step(1, 1);

  const int m = lane & 15;
  const bool mok = m < it.cnt;
  const uint32_t hrow = (uint32_t)((it.pos0 + m) * I + 32 * (lane >> 4)) * 2u;
  auto hoff = [&](int c) { return (mok && c < KC) ? hrow + (uint32_t)c * kAtomK * 2u : kOutOfRange; };
  bf16x8 ahi[2][4], alo[2][4];  // h fragments (both planes), fetched one chunk ahead
  {
    const uint32_t o = hoff(c0);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      ahi[0][j] = bload8(rh, o + 16u * j);
      alo[0][j] = bload8(rh, o == kOutOfRange ? o : o + lo_bytes + 16u * j);
    }
  }
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < NS; st++) {
    const int b = st & 1;
#pragma unroll
    for (int cc = 0; cc < S; cc++) {
      const int k = st * S + cc;
      if (k + 1 < CPW) {
        const uint32_t o = hoff(c0 + k + 1);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          ahi[(k + 1) & 1][j] = bload8(rh, o + 16u * j);
          alo[(k + 1) & 1][j] = bload8(rh, o == kOutOfRange ? o : o + lo_bytes + 16u * j);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const bf16x8 b0 = W::op(wa[b][cc], j);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[k & 1][j], b0, acc0, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[k & 1][j], b0, acc0, 0, 0, 0);
        const bf16x8 b1 = W::op(wb[b][cc], j);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[k & 1][j], b1, acc1, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[k & 1][j], b1, acc1, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (st + 2 < NS) load_step(st + 2, b);
  }
  if constexpr (W::kMatrixScale) {
    acc0 *= msd;
    acc1 *= msd;
  }
  red[(2 * w) * 64 + lane] = acc0;
  red[(2 * w + 1) * 64 + lane] = acc1;
  lds_sync();
  down_epilogue(red, nw, it, 0, q, H, yperm);
}

// y[t] = sum_j g[t,j] * o[inv(t,j)] (+ shared row), fp32 in rank order, bf16 out.
// A thread takes 4 consecutive columns (H is a multiple of 128); the k rows
// (at most 16) are all loaded before the fmas, which keep rank order.
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ yperm, const int32_t* __restrict__ inv,
    const float* __restrict__ gates, int T, int k, int H, int has_shared,
    uint16_t* __restrict__ y, float* __restrict__ y32) {
  const int t = blockIdx.y;
  const int col = 4 * (blockIdx.x * 256 + threadIdx.x);
  if (col >= H) return;
  f32x4 v[17];
#pragma unroll
  for (int j = 0; j < 16; j++)
    if (j < k) v[j] = *reinterpret_cast<const f32x4*>(yperm + (size_t)inv[t * k + j] * H + col);
  if (has_shared) v[16] = *reinterpret_cast<const f32x4*>(yperm + (size_t)(T * k + t) * H + col);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 16; j++)
    if (j < k) {
      const float g = gates[t * k + j];
#pragma unroll
      for (int c = 0; c < 4; c++) acc[c] = fmaf(g, v[j][c], acc[c]);
    }
  if (has_shared) {
#pragma unroll
    for (int c = 0; c < 4; c++) acc[c] += v[16][c];
  }
  const uint32_t lo = (uint32_t)f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  *reinterpret_cast<u32x2_t*>(y + (size_t)t * H + col) = u32x2_t{lo, hi};
  if (y32) *reinterpret_cast<f32x4*>(y32 + (size_t)t * H + col) = acc;
}

// Waves per workgroup (the split of K) and chunks per wave.
struct Split {
  int waves, cpw;
};

// Chunks per wave of the streaming launches (1, 2, 4, 8 or 16), from timings
// of every variant on the 35B-A3B, DSV4 and GLM decode shapes (K of 16, 32
// and 48 chunks for gate/up, 4 and 16 for down):
//  - gate/up: two chunks per wave while K needs at most 16 such waves (the
//    whole K of a workgroup in flight at once), else 16 chunks per wave;
//  - down: the fewest chunks per wave that keep a workgroup at <= 8 waves.
constexpr int kMaxStreamTokens = 16;

int stream_waves(int KC, int cpw) { return (KC + cpw - 1) / cpw; }

int gateup_stream_cpw(int KC) {
  if (KC <= 1) return 1;
  return stream_waves(KC, 2) <= kMaxWaves ? 2 : 16;
}
// bf16 streaming launches: the MXFP4 choice `cpw`, with fewer, longer waves
// where it would need more than the 8 a bf16 workgroup may have.  Where the
// two formats launch alike, their partial sums meet in the same order.
int bf16_stream_cpw(int KC, int cpw) {
  while (cpw < 16 && stream_waves(KC, cpw) > 8) cpw *= 2;
  return cpw;
}
int down_stream_cpw(int KC) {
  int cpw = 1;
  while (cpw < 16 && (cpw < KC ? stream_waves(KC, cpw) : 1) > 8) cpw *= 2;
  return cpw;
}

}  // namespace

// Work-list rows of the launch grid: the most items a call of T tokens has
// in the given part (every unique expert may be resident, or copied), and
// the device counters that bound the part.
static int items_for(const Ctx* c, int T, ItemRange part) {
  const int u = std::min(T * c->cfg.top_k, c->cfg.n_experts);
  return part == kItemsCopied ? u : u + c->cfg.has_shared;
}
static ExpertList decode_list(const Ctx* c, const DecodeScratch& s, int T, ItemRange part) {
  ExpertList L;
  L.items = s.items;
  L.items_cap = s.max_items;
  L.lo_p = part == kItemsCopied ? &s.meta->n_items_a : &s.meta->zero;
  L.hi_p = part == kItemsResident ? &s.meta->n_items_a : &s.meta->n_items;
  L.grid_items = items_for(c, T, part);
  L.split_items = items_for(c, T, kItemsAll);
  L.tok = s.tok;
  L.h = s.h;
  L.lo_plane = s.lo_plane;
  L.yperm = s.yperm;
  L.stream = T <= kMaxStreamTokens;
  return L;
}

// The K split of the kernels for more than 16 rows per item: within the
// format's workgroup size, for the whole list whichever part a launch
// covers (so that an expert's partial sums meet in the same order resident
// or copied).
static Split list_split(const Ctx* c, const ExpertList& L, int KC, int row_groups) {
  const int max_waves = c->cfg.weight_format == MOE_WEIGHTS_BF16 ? WBf16<false>::kMaxThreads / 64 : kMaxWaves;
  int s = 1;
  while (s < max_waves && s * row_groups * L.split_items < 4096) s *= 2;
  s = std::max(s, (KC + 3) / 4);
  s = std::min(s, std::min(max_waves, KC));
  return {s, (KC + s - 1) / s};
}

// Whether the kernels for more than 16 rows per item can split a K of this
// length (bf16 weights take at most 8 waves of 4 chunks).
static bool list_split_fits(const Ctx* c, int K) {
  const int max_waves = c->cfg.weight_format == MOE_WEIGHTS_BF16 ? WBf16<false>::kMaxThreads / 64 : kMaxWaves;
  return K / kAtomK <= 4 * max_waves;
}

// Weights are loaded nontemporal where the cache slots hold more than the
// 256 MB Infinity Cache could keep: every call streams its experts' atoms
// once, and allocating them would only evict the token rows, h and the
// shared experts, which later calls read again.  A smaller cache (the
// 35B-A3B-shaped one, 107 MB) stays in the Infinity Cache from call to call
// when loaded normally, and nontemporal loads would forfeit that.  Measured
// per launch: GLM-5.2 shape gate/up 15.2 -> 14.6 us and down 10.6 -> 10.3
// us, DSV4 shape 9.9 -> 9.7 and 7.8 -> 7.7 us; the 35B-A3B shape at T = 16
// would go from 13.2 to 15.4 us.
constexpr size_t kInfinityCacheBytes = size_t(256) << 20;
static bool weights_nontemporal(const Ctx* c) {
  return (size_t)c->C * c->stride > kInfinityCacheBytes;
}

hipError_t launch_gateup_list(const Ctx* c, const ExpertList& L, const uint16_t* x,
                              uint32_t x_bytes, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  dim3 grid(c->cfg.inter / kAtomRows, L.grid_items);
  const size_t lo = L.lo_plane;
  const int H = c->cfg.hidden, I = c->cfg.inter;
  const int KC = H / kAtomK;
  const bool bf16 = c->cfg.weight_format == MOE_WEIGHTS_BF16;
  const bool nv = c->cfg.weight_format == MOE_WEIGHTS_NVFP4;
  const bool nt = weights_nontemporal(c);
  const size_t ms_off = nv ? nv_trailer_offset(H, I) : 0;
  if (L.stream) {
    const int cpw = bf16 ? bf16_stream_cpw(KC, gateup_stream_cpw(KC)) : gateup_stream_cpw(KC);
    const int waves = stream_waves(KC, cpw);
#define GATEUP_S(N, F)                                                                     \
  MOE_LAUNCH((gateup_stream_kernel<N, F>), grid, waves * 64, waves * 2 * 64 * 16, st, ev0, \
             ev1, L.items, L.items_cap, L.lo_p, L.hi_p, L.tok, x, x_bytes, H, I, L.h, lo, ms_off)
#define GATEUP_F(N) \
  if (bf16) { if (nt) GATEUP_S(N, WBf16<true>); else GATEUP_S(N, WBf16<false>); }      \
  else if (nv) { if (nt) GATEUP_S(N, WNvfp4<true>); else GATEUP_S(N, WNvfp4<false>); } \
  else { if (nt) GATEUP_S(N, WMxfp4<true>); else GATEUP_S(N, WMxfp4<false>); }
    switch (cpw) {
      case 1: GATEUP_F(1); break;
      case 2: GATEUP_F(2); break;
      case 4: GATEUP_F(4); break;
      case 8: GATEUP_F(8); break;
      default: GATEUP_F(16); break;
    }
#undef GATEUP_F
#undef GATEUP_S
    return hipGetLastError();
  }
  if (!list_split_fits(c, H)) return hipErrorNotSupported;
  const Split sp = list_split(c, L, KC, grid.x);
#define GATEUP_L(N, F)                                                                          \
  MOE_LAUNCH((gateup_decode_kernel<N, F>), grid, sp.waves * 64, sp.waves * 2 * 64 * 16, st, ev0, \
             ev1, L.items, L.items_cap, L.lo_p, L.hi_p, L.tok, x, x_bytes, H, I, L.h, lo, ms_off)
#define GATEUP(N) \
  if (bf16) { if (nt) GATEUP_L(N, WBf16<true>); else GATEUP_L(N, WBf16<false>); }      \
  else if (nv) { if (nt) GATEUP_L(N, WNvfp4<true>); else GATEUP_L(N, WNvfp4<false>); } \
  else { if (nt) GATEUP_L(N, WMxfp4<true>); else GATEUP_L(N, WMxfp4<false>); }
  switch (sp.cpw) {
    case 1: GATEUP(1); break;
    case 2: GATEUP(2); break;
    case 3: GATEUP(3); break;
    default: GATEUP(4); break;
  }
#undef GATEUP
#undef GATEUP_L
  return hipGetLastError();
}

hipError_t launch_down_list(const Ctx* c, const ExpertList& L, hipStream_t st, hipEvent_t ev0,
                            hipEvent_t ev1) {
  dim3 grid(c->cfg.hidden / (2 * kAtomRows), L.grid_items);
  const size_t lo = L.lo_plane;
  const int H = c->cfg.hidden, I = c->cfg.inter;
  const bool bf16 = c->cfg.weight_format == MOE_WEIGHTS_BF16;
  const bool nv = c->cfg.weight_format == MOE_WEIGHTS_NVFP4;
  const bool nt = weights_nontemporal(c);
  const size_t ms_off = nv ? nv_trailer_offset(H, I) : 0;
  const size_t gub = gateup_section_bytes(H, I, c->cfg.weight_format);
  const int KC = I / kAtomK;
  if (L.stream) {
    const int cpw = bf16 ? bf16_stream_cpw(KC, down_stream_cpw(KC)) : down_stream_cpw(KC);
    const int waves = stream_waves(KC, cpw);
#define DOWN_S(N, F)                                                                         \
  MOE_LAUNCH((down_stream_kernel<N, F>), grid, waves * 64, waves * 2 * 64 * 16, st, ev0, ev1, \
             L.items, L.items_cap, L.lo_p, L.hi_p, L.h, lo, H, I, gub, L.yperm, ms_off)
#define DOWN_F(N) \
  if (bf16) { if (nt) DOWN_S(N, WBf16<true>); else DOWN_S(N, WBf16<false>); }      \
  else if (nv) { if (nt) DOWN_S(N, WNvfp4<true>); else DOWN_S(N, WNvfp4<false>); } \
  else { if (nt) DOWN_S(N, WMxfp4<true>); else DOWN_S(N, WMxfp4<false>); }
    switch (cpw) {
      case 1: DOWN_F(1); break;
      case 2: DOWN_F(2); break;
      case 4: DOWN_F(4); break;
      case 8: DOWN_F(8); break;
      default: DOWN_F(16); break;
    }
#undef DOWN_F
#undef DOWN_S
    return hipGetLastError();
  }
  if (!list_split_fits(c, I)) return hipErrorNotSupported;
  const Split sp = list_split(c, L, KC, grid.x);
#define DOWN_L(N, F)                                                                          \
  MOE_LAUNCH((down_decode_kernel<N, F>), grid, sp.waves * 64, sp.waves * 2 * 64 * 16, st, ev0, \
             ev1, L.items, L.items_cap, L.lo_p, L.hi_p, L.h, lo, H, I, gub, L.yperm, ms_off)
#define DOWN(N) \
  if (bf16) { if (nt) DOWN_L(N, WBf16<true>); else DOWN_L(N, WBf16<false>); }      \
  else if (nv) { if (nt) DOWN_L(N, WNvfp4<true>); else DOWN_L(N, WNvfp4<false>); } \
  else { if (nt) DOWN_L(N, WMxfp4<true>); else DOWN_L(N, WMxfp4<false>); }
  switch (sp.cpw) {
    case 1: DOWN(1); break;
    case 2: DOWN(2); break;
    case 3: DOWN(3); break;
    default: DOWN(4); break;
  }
#undef DOWN
#undef DOWN_L
  return hipGetLastError();
}

hipError_t launch_expert_gateup(const Ctx* c, const DecodeScratch& s, const uint16_t* x, int T,
                                ItemRange part, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  return launch_gateup_list(c, decode_list(c, s, T, part), x, (uint32_t)T * c->cfg.hidden * 2, st,
                            ev0, ev1);
}

hipError_t launch_expert_down(const Ctx* c, const DecodeScratch& s, int T, ItemRange part,
                              hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  return launch_down_list(c, decode_list(c, s, T, part), st, ev0, ev1);
}

hipError_t launch_combine_rows(const float* yperm, const int32_t* inv, const float* gates, int T,
                               int k, int H, int has_shared, uint16_t* y, float* y32,
                               hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  dim3 grid((H / 4 + 255) / 256, T);
  MOE_LAUNCH(combine_kernel, grid, 256, 0, st, ev0, ev1, yperm, inv, gates, T, k, H, has_shared,
             y, y32);
  return hipGetLastError();
}

}  // namespace moe
