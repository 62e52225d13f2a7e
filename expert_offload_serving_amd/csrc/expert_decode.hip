// Decode expert FFN: grouped skinny GEMMs over the experts of one call.
//
// Each expert of the call has 1..T tokens.  Its weights are streamed once
// from HBM in 1088-byte MXFP4 atoms (one 16-byte load per lane), dequantised
// in registers with the gfx950 scaled FP4 -> bf16 convert, and multiplied on
// v_mfma_f32_16x16x32_bf16 with the tokens as the 16-row A operand.  The
// kernels are HBM-bound: MFMA replaces the per-lane dot products and wave
// reductions a VALU GEMV would need, keeping VALU work per weight byte flat
// in the token count.  FFN: o = W_d (silu(W_g x) * (W_u x)); the pages name
// MXFP4 experts (jansverre.net FreeToken article, section "Hvor raskt kjører
// modellene?") but not the FFN form, which is SwiGLU here.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMT = 4;  // 16-token M tiles per pass

// 8 E2M1 codes (one dword, low nibble first) times 2^(s-127) -> 8 bf16.
// The convert reads only the exponent field of its fp32 scale operand.
__device__ __forceinline__ bf16x8 dequant8(uint32_t q, uint32_t sbyte) {
  const float s = __uint_as_float(sbyte << 23);
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 3));
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu(float a) { return a / (1.0f + expf(-a)); }

__device__ __forceinline__ bf16x8 load_a(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Gate/up + SwiGLU.  Block (p, item): row pair p (16 gate + 16 up rows) of
// one expert; the 4 waves split K and are reduced through LDS in fixed order.
__global__ __launch_bounds__(256) void gateup_decode_kernel(
    const WorkItem* __restrict__ items, const DevMeta* __restrict__ meta,
    const int32_t* __restrict__ tok, const uint16_t* __restrict__ x, int H, int I,
    uint16_t* __restrict__ h) {
  const int item = blockIdx.y;
  if (item >= meta->n_items) return;
  const WorkItem it = items[item];
  const int p = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int KC = H / kAtomK;
  const uint8_t* gbase = it.w + (size_t)(2 * p) * KC * kAtomBytes;
  const uint8_t* ubase = gbase + (size_t)KC * kAtomBytes;
  __shared__ f32x4 red[4][2][kMT][64];
  const bf16x8 zero = {};

  for (int m0 = 0; m0 < it.cnt; m0 += 16 * kMT) {
    const int mt_n = min(kMT, (it.cnt - m0 + 15) / 16);
    const uint16_t* xrow[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; mt++) {
      const int m = m0 + mt * 16 + (lane & 15);
      xrow[mt] = (mt < mt_n && m < it.cnt)
                     ? x + (size_t)tok[it.pos0 + m] * H + 8 * (lane >> 4)
                     : nullptr;
    }
    f32x4 accg[kMT], accu[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; mt++) accg[mt] = accu[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int c = w; c < KC; c += 4) {
      const uint8_t* ga = gbase + (size_t)c * kAtomBytes;
      const uint8_t* ua = ubase + (size_t)c * kAtomBytes;
      const u32x4 dg = *reinterpret_cast<const u32x4*>(ga + lane * 16);
      const u32x4 du = *reinterpret_cast<const u32x4*>(ua + lane * 16);
      const uint32_t sg = *reinterpret_cast<const uint32_t*>(ga + kAtomData + (lane & 15) * 4);
      const uint32_t su = *reinterpret_cast<const uint32_t*>(ua + kAtomData + (lane & 15) * 4);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const bf16x8 bg = dequant8(dg[j], (sg >> (8 * j)) & 0xFFu);
        const bf16x8 bu = dequant8(du[j], (su >> (8 * j)) & 0xFFu);
#pragma unroll
        for (int mt = 0; mt < kMT; mt++) {
          if (mt < mt_n) {
            const bf16x8 a = xrow[mt] ? load_a(xrow[mt] + c * kAtomK + 32 * j) : zero;
            accg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bg, accg[mt], 0, 0, 0);
            accu[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bu, accu[mt], 0, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < kMT; mt++) {
      if (mt < mt_n) {
        red[w][0][mt][lane] = accg[mt];
        red[w][1][mt][lane] = accu[mt];
      }
    }
    __syncthreads();
    if (w < mt_n) {
      const int mt = w;
      const f32x4 g = ((red[0][0][mt][lane] + red[1][0][mt][lane]) + red[2][0][mt][lane]) +
                      red[3][0][mt][lane];
      const f32x4 u = ((red[0][1][mt][lane] + red[1][1][mt][lane]) + red[2][1][mt][lane]) +
                      red[3][1][mt][lane];
      const int col = p * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int m = m0 + mt * 16 + 4 * (lane >> 4) + i;
        if (m < it.cnt)
          h[(size_t)(it.pos0 + m) * I + col] = f32_to_bf16_rne(silu(g[i]) * u[i]);
      }
    }
    __syncthreads();
  }
}

// Down projection.  Block (rb, item): 4 row groups (64 rows of H), one per
// wave, over the full K = I.
__global__ __launch_bounds__(256) void down_decode_kernel(
    const WorkItem* __restrict__ items, const DevMeta* __restrict__ meta,
    const uint16_t* __restrict__ h, int H, int I, size_t gateup_bytes,
    float* __restrict__ yperm) {
  const int item = blockIdx.y;
  if (item >= meta->n_items) return;
  const WorkItem it = items[item];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rg = blockIdx.x * 4 + w;
  if (rg >= H / kAtomRows) return;
  const int KC = I / kAtomK;
  const uint8_t* dbase = it.w + gateup_bytes + (size_t)rg * KC * kAtomBytes;
  const bf16x8 zero = {};

  for (int m0 = 0; m0 < it.cnt; m0 += 16 * kMT) {
    const int mt_n = min(kMT, (it.cnt - m0 + 15) / 16);
    const uint16_t* hrow[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; mt++) {
      const int m = m0 + mt * 16 + (lane & 15);
      hrow[mt] = (mt < mt_n && m < it.cnt) ? h + (size_t)(it.pos0 + m) * I + 8 * (lane >> 4)
                                           : nullptr;
    }
    f32x4 acc[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; mt++) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < KC; c++) {
      const uint8_t* da = dbase + (size_t)c * kAtomBytes;
      const u32x4 d = *reinterpret_cast<const u32x4*>(da + lane * 16);
      const uint32_t s = *reinterpret_cast<const uint32_t*>(da + kAtomData + (lane & 15) * 4);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const bf16x8 b = dequant8(d[j], (s >> (8 * j)) & 0xFFu);
#pragma unroll
        for (int mt = 0; mt < kMT; mt++) {
          if (mt < mt_n) {
            const bf16x8 a = hrow[mt] ? load_a(hrow[mt] + c * kAtomK + 32 * j) : zero;
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[mt], 0, 0, 0);
          }
        }
      }
    }
    const int col = rg * 16 + (lane & 15);
#pragma unroll
    for (int mt = 0; mt < kMT; mt++) {
      if (mt < mt_n) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int m = m0 + mt * 16 + 4 * (lane >> 4) + i;
          if (m < it.cnt) yperm[(size_t)(it.pos0 + m) * H + col] = acc[mt][i];
        }
      }
    }
  }
}

// y[t] = sum_j g[t,j] * o[inv(t,j)] (+ shared row), fp32 in rank order, bf16 out.
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ yperm, const int32_t* __restrict__ inv,
    const float* __restrict__ gates, int T, int k, int H, int has_shared,
    uint16_t* __restrict__ y, float* __restrict__ y32) {
  const int t = blockIdx.y;
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= H) return;
  float acc = 0.f;
  for (int j = 0; j < k; j++)
    acc = fmaf(gates[t * k + j], yperm[(size_t)inv[t * k + j] * H + col], acc);
  if (has_shared) acc += yperm[(size_t)(T * k + t) * H + col];
  y[(size_t)t * H + col] = f32_to_bf16_rne(acc);
  if (y32) y32[(size_t)t * H + col] = acc;
}

}  // namespace

static int items_for(const Ctx* c, int T) {
  return std::min(T * c->cfg.top_k, c->cfg.n_experts) + c->cfg.has_shared;
}

hipError_t launch_expert_gateup(const Ctx* c, const uint16_t* x, int T, hipStream_t st) {
  dim3 grid(c->cfg.inter / kAtomRows, items_for(c, T));
  gateup_decode_kernel<<<grid, 256, 0, st>>>(c->d_items, c->d_meta, c->d_tok, x, c->cfg.hidden,
                                             c->cfg.inter, c->d_h);
  return hipGetLastError();
}

hipError_t launch_expert_down(const Ctx* c, int T, hipStream_t st) {
  dim3 grid((c->cfg.hidden / kAtomRows + 3) / 4, items_for(c, T));
  down_decode_kernel<<<grid, 256, 0, st>>>(c->d_items, c->d_meta, c->d_h, c->cfg.hidden,
                                           c->cfg.inter,
                                           gateup_section_bytes(c->cfg.hidden, c->cfg.inter),
                                           c->d_yperm);
  return hipGetLastError();
}

hipError_t launch_combine(const Ctx* c, int T, uint16_t* y, float* y32, hipStream_t st) {
  dim3 grid((c->cfg.hidden + 255) / 256, T);
  combine_kernel<<<grid, 256, 0, st>>>(c->d_yperm, c->d_inv, c->d_gates, T, c->cfg.top_k,
                                       c->cfg.hidden, c->cfg.has_shared, y, y32);
  return hipGetLastError();
}

}  // namespace moe
