// Prefill forward: whole layers of experts streamed from the pinned pool into
// two HBM layer buffers (layer l+1 uploads on a copy stream while layer l
// computes: aipolix.com FreeToken article, fourth paragraph; jansverre.net
// FreeToken article, section "Hvorfor er båndbredden viktigere enn antall
// kjerner?"), an fp64 router GEMM on MFMA, multi-workgroup top-k and
// counting-sort dispatch, and the expert FFN as grouped MFMA GEMMs over every
// expert: bf16 MFMAs on MXFP4 weights dequantised in registers (the default),
// on bf16 weights as stored and on NVFP4 weights dequantised exactly, or the
// opt-in MXFP8 mode on the scaled fp8 x fp4 MFMA.
#include <algorithm>

#include "moe_internal.h"
#include "nvfp4_dequant.h"
#include "route_common.h"

namespace moe {

// Routing arrays are kept per layer ([L][...]) so that every layer of the
// last call can be inspected; the GEMM scratch is shared by the layers.
struct Prefill {
  int Tmax = 0;
  int last_T = 0;
  int last_layers = 0;
  int last_mx = 0;             // the last call ran in the MXFP8 mode
  int nchunk_max = 0;
  int max_tiles = 0;
  int resident_wgs = 8;        // GEMM workgroups resident at once: one per CU, a multiple of 8
  float* logits = nullptr;     // [Tmax][E]
  int32_t* ids = nullptr;      // [L][Tmax*k]
  float* gates = nullptr;      // [L][Tmax*k]
  int32_t* chunk_cnt = nullptr;  // [nchunk][E]
  int32_t* counts = nullptr;   // [L][E+1]: rows per group (group E: shared expert)
  int32_t* offsets = nullptr;  // [L][E+1]: first permuted row per group
  int32_t* sorted = nullptr;   // [L][Tmax*k]
  int32_t* inv = nullptr;      // [L][Tmax*k]
  int32_t* tok = nullptr;      // [Tmax*k + Tmax]
  int2* tiles = nullptr;       // [max_tiles]: (group, first row)
  int32_t* n_tiles = nullptr;  // [1]
  uint16_t* h = nullptr;       // bf16 [rows][I]: h rounded to bf16; in the MXFP8
                               // mode the same memory holds h's codes
                               // [rows][I] then its scales [rows][I/32]
  uint8_t* xq = nullptr;       // MXFP8 mode: x codes [Tmax][H], then scales
                               // [Tmax][H/32] (allocated on first use)
  uint8_t* hlo = nullptr;      // low-order records of h: [max_tiles][I/128][8][1664]
  float* yperm = nullptr;      // [rows][H]
};

// Tiles of 128 rows: every group's partial tile plus the whole rows, rounded
// up to a multiple of 8 (the launch deals tiles to the 8 XCDs).
int prefill_max_tiles(int T, int k, int E) {
  return ((T * k + T + 127) / 128 + E + 1 + 7) / 8 * 8;
}
// Bytes of the low-order records of h: 13 KB per tile and K chunk of 128.
size_t prefill_lo_bytes(int T, int k, int E, int I) {
  return (size_t)prefill_max_tiles(T, k, E) * (size_t)(I / 128) * (8 * 1664);
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kChunkTokens = 64;   // tokens per dispatch chunk (one wave)
constexpr int kBM = 128;           // tokens per GEMM tile
constexpr int kFragsPerWave = 8;   // weight atoms (16 columns each) per wave
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8 dequant8(uint32_t q, uint32_t sbyte) {
  const float s = __uint_as_float(sbyte << 23);
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, s, 3));
  return __builtin_bit_cast(bf16x8, r);
}
// silu(a) = a / (1 + e^-a) on the hardware exp2 and reciprocal (about 1 ulp
// each; the GEMM epilogue evaluates it for every h element, and the IEEE
// divide and library exp cost about 30 instructions per value).  Very
// negative a gives e^-a = inf and a * rcp(inf) = -0; the inputs are finite.
__device__ __forceinline__ float silu(float a) {
  const float e = __builtin_amdgcn_exp2f(-a * 1.4426950408889634f);
  return a * __builtin_amdgcn_rcpf(1.0f + e);
}

// ---------------------------------------------------------------- router
// logits[t][e] = fp32(sum_h x[t][h] W_r[h][e] + bias), fp64 products and
// sums on v_mfma_f64_16x16x4_f64.  Block: 64 tokens x 64 experts, K staged
// through LDS in chunks of 64 as fp32 (bf16 x and fp32 W_r are exact in
// fp64); each wave owns a 32 x 32 sub-tile (2 x 2 fragments).  Operands:
// lane l holds A[l % 16][l / 16] and B[l / 16][l % 16] of a K=4 step.  The
// LDS is double-buffered: a chunk's global loads go to registers before the
// MFMAs of the previous chunk and into the other buffer after them, one
// barrier per chunk (a DSV4 layer has exactly one block per CU, one wave per
// SIMD, so nothing else would hide the loads).
__global__ __launch_bounds__(256) void router_prefill_kernel(
    const uint16_t* __restrict__ x, int T, int H, int E, const float* __restrict__ wrt,
    const float* __restrict__ bias, float* __restrict__ logits) {
  __shared__ float xs[2][64][65];
  __shared__ float ws[2][64][65];
  const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w & 1, wn = w >> 1;
  f64x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
  // thread's two pieces per chunk: row r = i >> 3, 8 columns from 8 (i & 7)
  u32x4 xv[2];
  f32x4 wv[2][2];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int i = threadIdx.x + 256 * u, r = i >> 3, q = i & 7;
      const int t = t0 + r, e = e0 + r;
      xv[u] = u32x4{0u, 0u, 0u, 0u};
      wv[u][0] = wv[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (t < T) xv[u] = *reinterpret_cast<const u32x4*>(x + (size_t)t * H + k0 + 8 * q);
      if (e < E) {
        wv[u][0] = *reinterpret_cast<const f32x4*>(wrt + (size_t)e * H + k0 + 8 * q);
        wv[u][1] = *reinterpret_cast<const f32x4*>(wrt + (size_t)e * H + k0 + 8 * q + 4);
      }
    }
  };
  auto store = [&](int b) {
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int i = threadIdx.x + 256 * u, r = i >> 3, q = i & 7;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        xs[b][r][8 * q + 2 * j] = __uint_as_float(xv[u][j] << 16);
        xs[b][r][8 * q + 2 * j + 1] = __uint_as_float(xv[u][j] & 0xFFFF0000u);
        ws[b][r][8 * q + j] = wv[u][0][j];
        ws[b][r][8 * q + 4 + j] = wv[u][1][j];
      }
    }
  };
  load(0);
  store(0);
  __syncthreads();
  for (int k0 = 0, b = 0; k0 < H; k0 += 64, b ^= 1) {
    const bool more = k0 + 64 < H;
    if (more) load(k0 + 64);
#pragma unroll 4
    for (int kk = 0; kk < 64; kk += 4) {
      double a[2], bb[2];
#pragma unroll
      for (int f = 0; f < 2; f++) {
        a[f] = (double)xs[b][wm * 32 + f * 16 + (lane & 15)][kk + (lane >> 4)];
        bb[f] = (double)ws[b][wn * 32 + f * 16 + (lane & 15)][kk + (lane >> 4)];
      }
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], bb[j], acc[i][j], 0, 0, 0);
    }
    // buffer b^1 was last read before the previous barrier
    if (more) store(b ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        // f64 16x16x4 output: lane l, register r holds row (l / 16) + 4 r
        const int t = t0 + wm * 32 + i * 16 + (lane >> 4) + 4 * r;
        const int e = e0 + wn * 32 + j * 16 + (lane & 15);
        if (t < T && e < E) {
          const size_t o = (size_t)t * E + e;
          const double s = acc[i][j][r];
          logits[o] = (float)(bias ? s + (double)bias[o] : s);
        }
      }
}

// ------------------------------------------------------------------ top-k
template <int NK>
__global__ __launch_bounds__(1024) void topk_prefill_kernel(TopkArgs a, int T) {
  const int t = blockIdx.x * 16 + (threadIdx.x >> 6);
  if (t < T) topk_token<NK>(a, t, nullptr);
}

// --------------------------------------------------------------- dispatch
// Per chunk of 64 tokens: a bit matrix [token][expert] in LDS, then for each
// expert a ballot over the chunk's tokens gives the count (and, in the place
// kernel, each token's rank among the chunk's tokens of that expert).
__device__ void chunk_bits(const int32_t* ids, int T, int k, int chunk, uint32_t (*bits)[33]) {
  for (int i = threadIdx.x; i < kChunkTokens * 32; i += blockDim.x) bits[i >> 5][i & 31] = 0u;
  __syncthreads();
  for (int i = threadIdx.x; i < kChunkTokens * k; i += blockDim.x) {
    const int r = i / k, t = chunk * kChunkTokens + r;
    if (t < T) {
      const int e = ids[t * k + i % k];
      atomicOr(&bits[r][e >> 5], 1u << (e & 31));
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ ids,
                                                             int T, int k, int E,
                                                             int32_t* __restrict__ chunk_cnt) {
  __shared__ uint32_t bits[kChunkTokens][33];
  const int c = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  chunk_bits(ids, T, k, c, bits);
  for (int e = w; e < E; e += blockDim.x >> 6) {
    const bool has = (bits[lane][e >> 5] >> (e & 31)) & 1u;
    const uint64_t b = __ballot(has);
    if (lane == 0) chunk_cnt[(size_t)c * E + e] = __popcll(b);
  }
}

__global__ __launch_bounds__(1024) void dispatch_place_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int has_shared, int nchunk,
    const int32_t* __restrict__ chunk_cnt, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ inv,
    int32_t* __restrict__ tok, int2* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  __shared__ uint32_t bits[kChunkTokens][33];
  __shared__ int s_base[1024];
  __shared__ __attribute__((aligned(16))) int s_rem[1024];
  __shared__ int s_tmp[16];
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  chunk_bits(ids, T, k, c, bits);
  const int e = tid;
  int tot = 0, pre = 0;
  if (e < E) {
    for (int cc = 0; cc < nchunk; cc++) {
      const int v = chunk_cnt[(size_t)cc * E + e];
      tot += v;
      if (cc < c) pre += v;
    }
  }
  int total;
  const int off = block_excl_scan(tot, s_tmp, &total);
  if (e < E) s_base[e] = off + pre;
  if (c == 0) {
    if (e < E) {
      counts[e] = tot;
      offsets[e] = off;
    }
    if (tid == 0) {
      counts[E] = has_shared ? T : 0;
      offsets[E] = T * k;
    }
    // GEMM tiles of kBM rows.  Every full tile first (routed groups 0..E-1,
    // then the shared group E), then each group's partial tile by descending
    // row count (ties: lower group first).  Workgroups start in tile order,
    // so the last round of the GEMM launches holds the smallest tiles, which
    // issue the fewest loads and MFMAs, instead of full ones.
    const int nfull = e < E ? tot / kBM : 0;
    const int nfs = has_shared ? T / kBM : 0;
    int nfull_tot;
    const int ffirst = block_excl_scan(nfull, s_tmp, &nfull_tot);
    for (int i = 0; i < nfull; i++) tiles[ffirst + i] = int2{e, i * kBM};
    for (int i = tid; i < nfs; i += blockDim.x) tiles[nfull_tot + i] = int2{E, i * kBM};
    const int full_end = nfull_tot + nfs;
    // Partial tiles: group g has s_rem[g] rows left over (0: none; entries
    // past E stay 0).  One scan counts the routed partial tiles (low 16
    // bits) and the routed groups that rank before the shared group's
    // partial tile, s_rem >= rs (high 16 bits).
    const int rs = has_shared ? T % kBM : 0;
    const int mine = e < E ? tot % kBM : 0;
    s_rem[tid] = mine;
    int counts2;
    block_excl_scan((mine > 0 ? 1 : 0) | (rs > 0 && mine >= rs ? 1 << 16 : 0), s_tmp,
                    &counts2);  // its barriers also publish s_rem
    if (mine > 0) {
      int rank = rs > mine ? 1 : 0;  // the shared group ranks after equal routed ones
      const int4* r4 = reinterpret_cast<const int4*>(s_rem);
      for (int g4 = 0; g4 < (E + 3) / 4; g4++) {
        const int4 r = r4[g4];
        const int g = 4 * g4;
        rank += (r.x > mine) | ((r.x == mine) & (g < e));
        rank += (r.y > mine) | ((r.y == mine) & (g + 1 < e));
        rank += (r.z > mine) | ((r.z == mine) & (g + 2 < e));
        rank += (r.w > mine) | ((r.w == mine) & (g + 3 < e));
      }
      tiles[full_end + rank] = int2{e, nfull * kBM};
    }
    if (tid == 0) {
      const int npart = (counts2 & 0xFFFF) + (rs > 0 ? 1 : 0);
      if (rs > 0) tiles[full_end + (counts2 >> 16)] = int2{E, nfs * kBM};
      *n_tiles = full_end + npart;
    }
    if (has_shared)
      for (int t = tid; t < T; t += blockDim.x) tok[T * k + t] = t;
  }
  __syncthreads();
  const int t = c * kChunkTokens + lane;
  for (int ee = w; ee < E; ee += blockDim.x >> 6) {
    const bool has = (bits[lane][ee >> 5] >> (ee & 31)) & 1u;
    const uint64_t b = __ballot(has);
    if (has) {
      const int pos = s_base[ee] + __popcll(b & ((1ull << lane) - 1ull));
      int j = 0;
      while (ids[t * k + j] != ee) j++;
      const int f = t * k + j;
      sorted[pos] = f;
      inv[f] = pos;
      tok[pos] = t;
    }
  }
}

// -------------------------------------------------------------- grouped GEMM
// Tile t of the tile list and n-block nb, with the workgroups of one tile
// kept on one XCD (workgroup ids are dealt round-robin over the 8 XCDs), so
// that the tile's gathered token rows stay in that XCD's L2.
__device__ __forceinline__ void tile_of_index(int L, int nbn, int* ti, int* nb) {
  const int xcd = L & 7, j = L >> 3;
  *ti = (j / nbn) * 8 + xcd;
  *nb = j % nbn;
}
__device__ __forceinline__ void tile_of_block(int nbn, int* ti, int* nb) {
  tile_of_index(blockIdx.x, nbn, ti, nb);
}

// Grouped GEMM tile: C[128 token rows][512 columns] over K in chunks of 128,
// on 8 waves (two per SIMD): wave w owns columns 128(w%4).. and the 16-row
// fragments 2i + w/4 (i < 4) -- interleaved, so that the two waves sharing
// a SIMD hold nearly equal row counts in a partly filled tile -- as 4 x 8
// fragments of the 16x16x32 bf16 MFMA.  512 columns read each gathered
// token row once per 512 output columns: the token rows are the larger
// operand (bf16 against 4-bit weights) and, re-read from L2 by every column
// block, dominate what the loads move.  Both operands go straight from
// global memory into LDS with buffer-to-LDS loads, so nothing but the
// accumulators lives across chunks:
//  - A (bf16 token rows, gathered): fragment mf is 4 KB, one 256-byte chunk
//    row per token row, its sixteen 16-byte pieces stored XOR-swizzled by
//    the row (piece p of row r at slot p ^ r).  Each load instruction fills
//    1 KB, four whole rows (so every 128-byte line it touches is read in
//    full: half-line reads measured at half the rate).  At K step j a lane
//    needs the elements its weight fragment covers, 32(l/16) + 8j (MX block
//    l/16, sub-block j), i.e. piece 4(l/16) + j of row l%16; the swizzle
//    puts the 16 rows' pieces in 16 different bank groups;
//  - B (the tile's 32 MXFP4 weight atoms of the chunk, 8 per column
//    quarter): the 1 KB of codes of atom t at block t (lane order, as
//    stored), then every atom's 64 scale bytes packed at 64t (one 4-byte
//    load per lane fetches the scales of four atoms); dequantised in
//    registers right before its MFMAs;
//  - in the down GEMM, the low-order piece of h (see below): the tile's 13 KB
//    record of the chunk, contracted once per chunk with the scaled
//    fp6 x fp4 MFMA on the weight codes as they are stored.
// The loads are split by source.  Waves 0-3 fetch A (rows 32w .. 32w+31:
// 8 loads per step, plus 3-4 loads of the low-order record in the down
// GEMM), mostly L2 hits since the column blocks of a token tile run together
// on one XCD; waves 4-7 fetch B (atoms 8(w-4) .. +7: 10 loads per chunk),
// which streams from HBM.  Both are fetched one step ahead.  The address
// unit takes a 1 KB buffer-to-LDS load about every 25 cycles and a wave
// that issues while it is busy stalls, so the two kinds are issued apart:
// the A waves right after the step's barrier, the B waves after the MFMAs of
// their first K step (their loads then no longer queue behind the A loads,
// and the A wave on the same SIMD computes meanwhile).  Per step every wave
// waits for its own loads of the step, one barrier makes them visible and
// frees the stages the previous step read.  Loads past the end go to an
// out-of-range offset (zeros, no memory traffic) into a stage no one reads
// any more, so the wait counts never change.  The barrier is a bare
// s_barrier with a compiler memory clobber: a workgroup fence there would
// make the compiler drain every buffer-to-LDS load in flight, including the
// prefetched ones.
//
// h between the two GEMMs: hi = RNE_bf16(h) as a bf16 plane [rows][I], and
// the remainder h - hi (at most 2^-9 |h|) as a block-scaled fp6 (E2M3)
// piece: per row and block of 32 columns one power-of-two scale 2^E with
// the block's largest remainder at most 7.5 * 2^E, each element RNE to the
// E2M3 grid.  The remainder piece errs by at most 2^-5 of its block's
// largest remainder, so h is carried to about 2^-14 of its block's largest
// value; the scaled MFMA contracts it at a quarter of the cost of a second
// bf16 plane.  Records: per (tile, K chunk of the down GEMM, 16-row
// fragment) 1664 bytes laid out as the MFMA operand wants them: lane L
// (row L%16, block L/16 of the chunk) has its 24 code bytes (element i at
// bits 6i) at 16L (bytes 0-15) and 1024 + 8L (bytes 16-23), its scale byte
// (E + 127) at 1536 + L; 64 bytes of padding.
constexpr int kGemmWaves = 8;
constexpr int kStagesA = 2;
constexpr int kStagesB = 2;
constexpr int kAtomsPerTile = 32;                                   // 512 columns
constexpr int kLdsA = kBM * kAtomK * 2;                             // 32 KB per A stage
constexpr int kLdsBc = kAtomsPerTile * kAtomData;                   // 32 KB of codes
constexpr int kLdsBStage = kLdsBc + kAtomsPerTile * 64;             // + 2 KB of scales
constexpr int kLoFrag = 1664;                                       // one 16-row fragment
constexpr int kLoChunk = 8 * kLoFrag;                               // 13 KB per tile and chunk
constexpr int kLdsMain = kStagesA * kLdsA + kStagesB * kLdsBStage;  // 132 KB
constexpr int kEpiStride = 68;  // floats per row in the epilogue's transpose: rows 4 apart
                                // land 16 banks apart
constexpr int kEpiWave = 4 * 16 * kEpiStride * 4;                   // 17 KB per wave
constexpr int kLdsGateUp = kLdsMain > 8 * kEpiWave ? kLdsMain : 8 * kEpiWave;  // 136 KB
constexpr int kLdsDown = kLdsMain + kStagesA * kLoChunk;            // 158 KB
static_assert(kLdsGateUp <= 160 * 1024 && kLdsDown <= 160 * 1024, "LDS per CU");
static_assert(kStagesA == 2 && kStagesB == 2, "the waits below assume one step in flight");
static_assert(kLoChunk % 1024 == 0, "low-order records load in whole kilobytes");

typedef __attribute__((address_space(3))) void lds_void;
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct GemmTile {
  const uint8_t* wbase;  // expert section start (gate/up or down)
  uint32_t wbytes;       // section bytes
  int KC;                // K chunks of the weights
  int k0;                // first K chunk: the walk is k0 .. KC-1, 0 .. k0-1
  int rows;              // valid rows in this tile (<= kBM)
  uint32_t lo0;          // down: byte offset of this tile's low-order records
  uint32_t aoff[8];      // A waves: this lane's piece of row 32w + 4i + l/16 for
                         // load i (row start + swizzled piece), or kOOB past
                         // the valid rows
  uint32_t woff[8];      // B waves: atom 8(w-4) + t, chunk 0
  uint32_t soff[2];      // B waves: this lane's scale dwords (atoms
                         // 8(w-4) + 4h + l/16, bytes 4(l%16) ..), chunk 0
};

// Buffer-to-LDS loads: `bytes` per lane from rsrc + voffset into LDS at
// lds + lane * slot (16 bytes for the 16-byte form, a 4-byte slot for one
// dword).  Written as asm so that the compiler, which cannot tell the stage
// buffers apart, adds no waits of its own before the LDS reads: every wait
// on these loads is an explicit one.  No output registers: the data goes to
// LDS.  The s_nop is the wait state an M0 write needs before a load that
// reads M0 (the compiler emits M0 right before).
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset, void* lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset), "s"(r),
               "{m0}"((uint32_t)(uintptr_t)(lds_void*)lds)
               : "memory");
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, uint32_t voffset, void* lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voffset), "s"(r),
               "{m0}"((uint32_t)(uintptr_t)(lds_void*)lds)
               : "memory");
}

// The same loads with the nontemporal hint, for the weights of the GEMMs
// that HBM bounds (the MXFP8 mode's, and those on bf16 and NVFP4 experts),
// which stream them once: without it they are allocated in L2 and the
// Infinity Cache for nothing.  Measured per layer: MXFP8 mode at the DSV4
// shape, T = 4096, gate/up 567 -> 553 us and down 372 -> 357 us (the
// combine after them 103 -> 121 us: its reads of the fp32 outputs now meet
// their write-backs); bf16 experts at the 35B-A3B shape gate/up 352 -> 328
// us, down 403 -> 393 us, combine 58 -> 45 us; NVFP4 experts gate/up 409 ->
// 392 us, down 265 -> 260 us.  The default mode's GEMMs on MXFP4 weights,
// bound by the matrix cores, run the same either way and keep normal loads.
__device__ __forceinline__ void lds_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voffset, void* lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voffset), "s"(r),
               "{m0}"((uint32_t)(uintptr_t)(lds_void*)lds)
               : "memory");
}
__device__ __forceinline__ void lds_load4_nt(__amdgpu_buffer_rsrc_t r, uint32_t voffset, void* lds) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, 0 offen nt lds" ::"v"(voffset), "s"(r),
               "{m0}"((uint32_t)(uintptr_t)(lds_void*)lds)
               : "memory");
}

// Wait until none of this wave's vector-memory instructions is outstanding.
__device__ __forceinline__ void wait_vmem_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most the last N vector-memory instructions of this wave are
// outstanding (loads complete in issue order): with weights three stages
// deep, a B wave's N loads of the next step.
template <int N>
__device__ __forceinline__ void wait_vmem_keep() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// MF: this wave's 16-row fragments that hold rows (0..4).  LO: the down GEMM,
// which also contracts the low-order piece of h (records through rl).
template <int MF, bool LO>
__device__ __forceinline__ void gemm_tile_mf(const GemmTile& gt, __amdgpu_buffer_rsrc_t ra,
                                             __amdgpu_buffer_rsrc_t rl, uint8_t* lds,
                                             f32x4 (&acc)[MF > 0 ? MF : 1][kFragsPerWave]) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int mh = w >> 2, nq = w & 3;
  const bool a_wave = w < 4;
  const int KC = gt.KC;
  const __amdgpu_buffer_rsrc_t rw = rsrc(gt.wbase, gt.wbytes);
  uint8_t* const lostages = lds + kStagesA * kLdsA;
  uint8_t* const bstages = lostages + (LO ? kStagesA * kLoChunk : 0);
  // Chunk of the weights (and of A) that walk position c covers.
  auto chunk = [&](int c) { return c + gt.k0 < KC ? c + gt.k0 : c + gt.k0 - KC; };
  // A waves: step s into stage s % 2; in the down GEMM also kilobytes
  // q0 .. q0+n-1 of the step's low-order record (4, 3, 3, 3 of its 13).
  // Loads that would fetch only rows at or past gt.rows are not issued: the
  // LDS rows they would fill feed only output rows that are never stored
  // (an MFMA output row depends on its own A row alone), so stale values
  // there are harmless.  The same holds for the kilobytes of a low-order
  // record past the tile's last 16-row fragment.
  auto issue_a = [&](int s) {
    const int st = s % kStagesA;
    uint8_t* buf = lds + st * kLdsA;
    const bool in = s < KC;
    const uint32_t k = (uint32_t)chunk(s) * (kAtomK * 2);
#pragma unroll
    for (int i = 0; i < 8; i++)
      if (32 * w + 4 * i < gt.rows)
        lds_load16(ra, in ? gt.aoff[i] + k : kOOB, buf + (8 * w + i) * 1024);
    if constexpr (LO) {
      const int q0 = w == 0 ? 0 : 1 + 3 * w, n = w == 0 ? 4 : 3;
      const int lo_end = ((gt.rows + 15) >> 4) * kLoFrag;  // bytes of the valid fragments
      const uint32_t lk = gt.lo0 + (uint32_t)chunk(s) * kLoChunk + 16u * (uint32_t)lane;
#pragma unroll
      for (int t = 0; t < 4; t++)
        if (t < n && (q0 + t) * 1024 < lo_end)
          lds_load16(rl, in ? lk + (uint32_t)(q0 + t) * 1024u : kOOB,
                     lostages + st * kLoChunk + (q0 + t) * 1024);
    }
  };
  // B waves: chunk c into stage c % 2.
  auto issue_b = [&](int c) {
    uint8_t* buf = bstages + (c % kStagesB) * kLdsBStage;
    const int u = w - 4;
    const bool in = c < KC;
    const uint32_t k = (uint32_t)chunk(c) * kAtomBytes;
#pragma unroll
    for (int t = 0; t < 8; t++)
      lds_load16(rw, in ? gt.woff[t] + k + 16u * lane : kOOB, buf + (8 * u + t) * kAtomData);
#pragma unroll
    for (int hh = 0; hh < 2; hh++)
      lds_load4(rw, in ? gt.soff[hh] + k : kOOB, buf + kLdsBc + (8 * u + 4 * hh) * 64);
  };
  // One step: the A fragments and dequantised weights of K step j+1 are
  // fetched while the MFMAs of step j run.
  auto compute = [&](int s) {
    if constexpr (MF == 0) {
      if (!a_wave) issue_b(s + 1);
    } else {
      const uint8_t* abuf = lds + (s % kStagesA) * kLdsA;
      const uint8_t* bbuf = bstages + (s % kStagesB) * kLdsBStage;
      u32x4 wd[kFragsPerWave];
      uint32_t sd[kFragsPerWave];
#pragma unroll
      for (int f = 0; f < kFragsPerWave; f++) {
        const int atom = nq * kFragsPerWave + f;
        wd[f] = *reinterpret_cast<const u32x4*>(bbuf + atom * kAtomData + 16 * lane);
        sd[f] = bbuf[kLdsBc + atom * 64 + lane];
      }
      bf16x8 a[2][MF];
      auto fetch = [&](int j, int q) {
        const int r = lane & 15;
        const int slot = ((4 * (lane >> 4) + j) ^ r) & 15;
#pragma unroll
        for (int i = 0; i < MF; i++)
          a[q][i] = *reinterpret_cast<const bf16x8*>(abuf + (2 * i + mh) * 4096 + 256 * r + 16 * slot);
      };
      // low-order operand: 24 code bytes and the scale of (row l%16, block l/16)
      u32x4 lq[MF];
      u32x2 lr[MF];
      uint32_t ls[MF];
      fetch(0, 0);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (j + 1 < 4) fetch(j + 1, (j + 1) & 1);
        if (LO && j == 3) {
          const uint8_t* lbuf = lostages + (s % kStagesA) * kLoChunk;
#pragma unroll
          for (int i = 0; i < MF; i++) {
            const uint8_t* fr = lbuf + (2 * i + mh) * kLoFrag;
            lq[i] = *reinterpret_cast<const u32x4*>(fr + 16 * lane);
            lr[i] = *reinterpret_cast<const u32x2*>(fr + 1024 + 8 * lane);
            ls[i] = fr[1536 + lane];
          }
        }
        // each atom's weights are dequantised right before its MFMAs
        // two operand registers in turn: the convert for atom f+1 never
        // waits for the MFMAs still reading atom f's operand
        bf16x8 bb[2];
        bb[0] = dequant8(wd[0][j], sd[0]);
#pragma unroll
        for (int f = 0; f < kFragsPerWave; f++) {
          if (f + 1 < kFragsPerWave) bb[(f + 1) & 1] = dequant8(wd[f + 1][j], sd[f + 1]);
#pragma unroll
          for (int i = 0; i < MF; i++)
            acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j & 1][i], bb[f & 1], acc[i][f], 0, 0, 0);
        }
        if (j == 0 && !a_wave) {
          __builtin_amdgcn_sched_barrier(0);
          issue_b(s + 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if constexpr (LO) {
        // fp6 (E2M3) remainder x fp4 (E2M1) weights, both block-scaled:
        // one MFMA covers the chunk's 128 K for a fragment and an atom
#pragma unroll
        for (int f = 0; f < kFragsPerWave; f++) {
          const i32x8 b8 = {(int)wd[f][0], (int)wd[f][1], (int)wd[f][2], (int)wd[f][3], 0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < MF; i++) {
            const i32x8 a8 = {(int)lq[i][0], (int)lq[i][1], (int)lq[i][2], (int)lq[i][3],
                              (int)lr[i][0], (int)lr[i][1], 0,            0};
            acc[i][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                a8, b8, acc[i][f], 2 /* A: fp6 E2M3 */, 4 /* B: fp4 E2M1 */, 0, (int)ls[i], 0,
                (int)sd[f]);
          }
        }
      }
    }
  };
  if (a_wave)
    issue_a(0);
  else
    issue_b(0);
  __builtin_amdgcn_sched_barrier(0);
  for (int s = 0; s < KC; s++) {
    wait_vmem_all();
    lds_barrier();
    if (a_wave) issue_a(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(s);  // the B waves issue step s+1 inside
  }
  // No buffer-to-LDS write may land after the workgroup has ended.
  wait_vmem_all();
}

// A wave w loads rows 32w .. 32w+31 (offsets set by the kernel); B wave
// w loads tile atoms 8(w-4) .. +7, which are weight row groups rg0 .. rg0+7.
// Row groups at or past ngroups (the last, partial column block) read group
// 0 instead: their columns are never stored.
__device__ __forceinline__ void clear_loads(GemmTile& gt) {
#pragma unroll
  for (int i = 0; i < 8; i++) gt.aoff[i] = kOOB;
#pragma unroll
  for (int t = 0; t < 8; t++) gt.woff[t] = 0;
  gt.soff[0] = gt.soff[1] = 0;
  gt.lo0 = 0;
}
// Byte offset, within a 256-byte chunk row, of the piece that lane l loads
// for tile row r: it lands in LDS slot l % 16 of that row, which holds
// piece (l % 16) ^ (r % 16).
__device__ __forceinline__ uint32_t a_piece(int r, int lane) {
  return 16u * (uint32_t)(((lane & 15) ^ r) & 15);
}
__device__ __forceinline__ void set_weight_loads(GemmTile& gt, int rg0, int lane, int ngroups) {
  const uint32_t group_bytes = (uint32_t)gt.KC * kAtomBytes;
#pragma unroll
  for (int t = 0; t < 8; t++) gt.woff[t] = (uint32_t)(rg0 + t < ngroups ? rg0 + t : 0) * group_bytes;
#pragma unroll
  for (int hh = 0; hh < 2; hh++) {
    const int rl = rg0 + 4 * hh + (lane >> 4);
    gt.soff[hh] = (uint32_t)(rl < ngroups ? rl : 0) * group_bytes + kAtomData + 4u * (lane & 15);
  }
}

struct GroupArgs {
  const int2* tiles;
  const int32_t* n_tiles;
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* tok;
  const uint8_t* layerbuf;
  size_t stride;
  const uint8_t* shared_w;
  int E;
};

// This wave's fragment count: of the tile's ceil(rows/16) fragments, those
// with index parity w/4.
#define MOE_MF_SWITCH(mf, CALL)  \
  switch (mf) {                  \
    case 0: CALL(0); break;      \
    case 1: CALL(1); break;      \
    case 2: CALL(2); break;      \
    case 3: CALL(3); break;      \
    default: CALL(4); break;     \
  }

__device__ __forceinline__ int wave_mfrags(int rows) {
  const int mh = wave_id() >> 2;
  return (((rows + 15) >> 4) - mh + 1) >> 1;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x6 __attribute__((ext_vector_type(6)));

template <int MF>
__device__ __forceinline__ void gateup_tile(const GemmTile& gt, __amdgpu_buffer_rsrc_t ra,
                                            uint8_t* lds, uint16_t* __restrict__ hhi,
                                            uint8_t* __restrict__ hlo, int I, size_t row0,
                                            int p0) {
  const int npairs = I / kAtomRows;
  const int lane = threadIdx.x & 63, w = wave_id(), mh = w >> 2;
  f32x4 acc[MF > 0 ? MF : 1][kFragsPerWave];
#pragma unroll
  for (int i = 0; i < (MF > 0 ? MF : 1); i++)
#pragma unroll
    for (int f = 0; f < kFragsPerWave; f++) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_tile_mf<MF, false>(gt, ra, ra, lds, acc);
  // Every wave's loads have landed (each ended with vmcnt(0)); after this
  // barrier no wave reads a stage any more and the LDS holds the transpose:
  // wave w's h at w * kEpiWave as [fragment i][row][64 columns] floats.
  lds_barrier();
  float* ep = reinterpret_cast<float*>(lds + w * kEpiWave);
#pragma unroll
  for (int i = 0; i < MF; i++)
#pragma unroll
    for (int q = 0; q < kFragsPerWave / 2; q++)
#pragma unroll
      for (int r = 0; r < 4; r++)
        ep[(i * 16 + 4 * (lane >> 4) + r) * kEpiStride + 16 * q + (lane & 15)] =
            silu(acc[i][2 * q][r]) * acc[i][2 * q + 1][r];
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave reads its own writes
  // Lane L: row L%16 of fragment 2it + L/32, block (L/16)%2 of the wave's
  // 64 columns (h columns 16 p0 + 32 b ..), i.e. block kb = (p0/2 + b) % 4 of
  // the down GEMM's chunk p0/8.
  const int row = lane & 15, b = (lane >> 4) & 1;
  const bool col_ok = p0 + 2 * b < npairs;
  const int kb = ((p0 >> 1) + b) & 3, LL = row + 16 * kb;
  uint8_t* const rec_chunk = hlo + (size_t)(p0 >> 3) * kLoChunk;
#pragma unroll
  for (int it = 0; it < (MF + 1) / 2; it++) {
    const int i = 2 * it + (lane >> 5);
    if (i < MF && col_ok) {
      const float* src = ep + (i * 16 + row) * kEpiStride + 32 * b;
      float v[32];
#pragma unroll
      for (int t = 0; t < 8; t++) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(src + 4 * t);
        v[4 * t] = x4[0], v[4 * t + 1] = x4[1], v[4 * t + 2] = x4[2], v[4 * t + 3] = x4[3];
      }
      // bf16 of each value (v_cvt_pk_bf16_f32: nearest, ties to even) and
      // the remainder, exact in fp32
      uint32_t hp[16];
      float mx = 0.0f;
#pragma unroll
      for (int t = 0; t < 32; t++) {
        const uint32_t hb = __builtin_bit_cast(uint16_t, (__bf16)v[t]);
        hp[t >> 1] = (t & 1) ? (hp[t >> 1] | (hb << 16)) : hb;
        v[t] -= __uint_as_float(hb << 16);
        mx = fmaxf(mx, fabsf(v[t]));
      }
      // block exponent: the largest remainder at most 7.5 * 2^E
      int E = -127;
      if (mx > 0.0f) {
        E = (int)((__float_as_uint(mx) >> 23) & 0xffu) - 127 - 2;
        E = E < -126 ? -126 : E;  // 2^E stays a normal float
        if (mx > 7.5f * __uint_as_float((uint32_t)(E + 127) << 23)) E += 1;
      }
      // E2M3 codes of remainder / 2^E, nearest with ties to even (|.| <= 7.5 by
      // the choice of E), packed 6 bits each: v_cvt_scalef32_2xpk16_fp6_f32
      // writes its first operand's element j at position 2j and its second's
      // at 2j + 1, so it takes the even and the odd elements.  An all-zero
      // block gives zero codes with any scale.
      f32x16 ev, od;
#pragma unroll
      for (int j = 0; j < 16; j++) ev[j] = v[2 * j], od[j] = v[2 * j + 1];
      const float scale = mx > 0.0f ? __uint_as_float((uint32_t)(E + 127) << 23) : 1.0f;
      const i32x6 d6 = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, scale);
      uint32_t d[6];
#pragma unroll
      for (int j = 0; j < 6; j++) d[j] = (uint32_t)d6[j];
      const int g = 2 * i + mh, m = g * 16 + row;
      if (m < gt.rows) {
        u32x4* dst = reinterpret_cast<u32x4*>(hhi + (row0 + m) * I + 16 * p0 + 32 * b);
#pragma unroll
        for (int t = 0; t < 4; t++) dst[t] = u32x4{hp[4 * t], hp[4 * t + 1], hp[4 * t + 2], hp[4 * t + 3]};
      }
      uint8_t* rec = rec_chunk + g * kLoFrag;
      *reinterpret_cast<u32x4*>(rec + 16 * LL) = u32x4{d[0], d[1], d[2], d[3]};
      *reinterpret_cast<u32x2*>(rec + 1024 + 8 * LL) = u32x2{d[4], d[5]};
      rec[1536 + LL] = (uint8_t)(E + 127);
    }
  }
}

template <int MF>
__device__ __forceinline__ void down_tile(const GemmTile& gt, __amdgpu_buffer_rsrc_t ra,
                                          __amdgpu_buffer_rsrc_t rl, uint8_t* lds,
                                          float* __restrict__ yperm, int H, size_t row0, int rg0,
                                          int ngroups) {
  const int lane = threadIdx.x & 63, mh = wave_id() >> 2;
  f32x4 acc[MF > 0 ? MF : 1][kFragsPerWave];
#pragma unroll
  for (int i = 0; i < (MF > 0 ? MF : 1); i++)
#pragma unroll
    for (int f = 0; f < kFragsPerWave; f++) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_tile_mf<MF, true>(gt, ra, rl, lds, acc);
#pragma unroll
  for (int i = 0; i < MF; i++)
#pragma unroll
    for (int f = 0; f < kFragsPerWave; f++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = (2 * i + mh) * 16 + 4 * (lane >> 4) + r;
        if (m < gt.rows && rg0 + f < ngroups)
          yperm[(row0 + m) * H + (rg0 + f) * 16 + (lane & 15)] = acc[i][f][r];
      }
}

// Gate/up + SwiGLU.  N-block nb covers row pairs nb*16 .. nb*16+15 (gate,
// up; pairs past I/16 in the last block are computed on group 0 and not
// stored); column quarter nq takes pairs nb*16 + 4nq .. +3 (atoms g0, u0,
// g1, u1, ...).  h leaves as the bf16 plane hi and the tile's low-order
// records (their layout is described above the GEMM constants).
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void gateup_prefill_kernel(
    GroupArgs g, const uint16_t* x, uint32_t x_bytes, int H, int I, int nbn,
    uint16_t* __restrict__ hhi, uint8_t* __restrict__ hlo) {
  int ti, nb;
  tile_of_block(nbn, &ti, &nb);
  if (ti >= *g.n_tiles) return;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsGateUp];
  const int2 td = g.tiles[ti];
  const int grp = td.x, m0 = td.y;
  const int cnt = g.counts[grp], pos0 = g.offsets[grp];
  const int lane = threadIdx.x & 63, w = wave_id(), nq = w & 3;
  GemmTile gt;
  gt.wbase = grp < g.E ? g.layerbuf + (size_t)grp * g.stride : g.shared_w;
  gt.KC = H / kAtomK;
  gt.wbytes = (uint32_t)(2 * I / kAtomRows) * (uint32_t)gt.KC * kAtomBytes;
  gt.k0 = nb * gt.KC / nbn;
  gt.rows = min(kBM, cnt - m0);
  clear_loads(gt);
  if (w < 4) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int r = 32 * w + 4 * i + (lane >> 4);
      if (r < gt.rows) gt.aoff[i] = (uint32_t)g.tok[pos0 + m0 + r] * (uint32_t)H * 2u + a_piece(r, lane);
    }
  } else {
    // Tile atom a (column quarter a/8, atom a%8 of it) is row group 32nb + a:
    // pair 16nb + a/2, gate if a is even, up if odd.
    set_weight_loads(gt, nb * 32 + 8 * (w - 4), lane, 2 * I / kAtomRows);
  }
  const __amdgpu_buffer_rsrc_t ra = rsrc(x, x_bytes);
  const size_t row0 = (size_t)(pos0 + m0);
  const int p0 = nb * 16 + 4 * nq;
  uint8_t* const tile_lo = hlo + (size_t)ti * (size_t)(I / kAtomK) * kLoChunk;
#define GU(N) gateup_tile<N>(gt, ra, lds, hhi, tile_lo, I, row0, p0)
  MOE_MF_SWITCH(wave_mfrags(gt.rows), GU)
#undef GU
}

// Down.  N-block nb covers row groups nb*32 .. nb*32+31 of H (512 columns;
// the last block may be partial); column quarter nq takes row groups
// nb*32 + 8nq .. +7.  A is the bf16 plane hi; the low-order records of h
// come through their own stage.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void down_prefill_kernel(
    GroupArgs g, const uint16_t* hhi, uint32_t hhi_bytes, const uint8_t* hlo, uint32_t hlo_bytes,
    int H, int I, int nbn, size_t gateup_bytes, float* __restrict__ yperm) {
  int ti, nb;
  tile_of_block(nbn, &ti, &nb);
  if (ti >= *g.n_tiles) return;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsDown];
  const int2 td = g.tiles[ti];
  const int grp = td.x, m0 = td.y;
  const int cnt = g.counts[grp], pos0 = g.offsets[grp];
  const int lane = threadIdx.x & 63, w = wave_id(), nq = w & 3;
  const int ngroups = H / kAtomRows;  // a multiple of 8; the last n-block may be partial
  GemmTile gt;
  gt.wbase = (grp < g.E ? g.layerbuf + (size_t)grp * g.stride : g.shared_w) + gateup_bytes;
  gt.KC = I / kAtomK;
  gt.wbytes = (uint32_t)ngroups * (uint32_t)gt.KC * kAtomBytes;
  gt.k0 = nb * gt.KC / nbn;
  gt.rows = min(kBM, cnt - m0);
  clear_loads(gt);
  gt.lo0 = (uint32_t)ti * (uint32_t)gt.KC * (uint32_t)kLoChunk;
  if (w < 4) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int r = 32 * w + 4 * i + (lane >> 4);
      if (r < gt.rows) gt.aoff[i] = (uint32_t)(pos0 + m0 + r) * (uint32_t)I * 2u + a_piece(r, lane);
    }
  } else {
    set_weight_loads(gt, nb * 32 + 8 * (w - 4), lane, ngroups);  // tile atom a: row group 32nb + a
  }
  const __amdgpu_buffer_rsrc_t ra = rsrc(hhi, hhi_bytes), rl = rsrc(hlo, hlo_bytes);
  const size_t row0 = (size_t)(pos0 + m0);
  const int rg0 = nb * 32 + 8 * nq;
#define DN(N) down_tile<N>(gt, ra, rl, lds, yperm, H, row0, rg0, ngroups)
  MOE_MF_SWITCH(wave_mfrags(gt.rows), DN)
#undef DN
}

// ------------------------------------------------ gate/up on bf16 weights
// Grouped GEMM tile for bf16 experts: C[128 token rows][128 columns] over K
// in chunks of 128, on the loads, stages and waits of gemm_tile_mf (A waves
// 0-3 fetch the token rows, B waves 4-7 the weights, one step ahead).  A
// tile holds 8 weight atoms of 4 KB (4 pairs of 16 gate and 16 up rows), the
// stage the same 32 KB of LDS an MXFP4 stage of 32 atoms takes; wave w owns
// pair w % 4 (atoms 2(w%4), 2(w%4)+1) and the fragments 2i + w/4, and feeds
// the stored bf16 pieces to the MFMA as they are.  Each wave then holds the
// gate and up sums of its own pair, so h = silu(g) * u is formed in
// registers and leaves as two bf16 planes (hi = RNE(h), lo = RNE(h - hi)).
constexpr int kBwAtoms = 8;                                          // 128 columns
constexpr int kLdsBwB = kBwAtoms * kAtomBytesBF16;                   // 32 KB per B stage
constexpr int kStagesBw = 3;                                         // weights two steps ahead
constexpr int kBwLoads = 8;                                          // per B wave and step
constexpr int kLdsBw = kStagesA * kLdsA + kStagesBw * kLdsBwB;       // 160 KB
static_assert(kLdsBw <= 160 * 1024, "LDS per CU");


template <int MF>
__device__ __forceinline__ void gemm_tile_bw(const GemmTile& gt, __amdgpu_buffer_rsrc_t ra,
                                             uint8_t* lds, f32x4 (&acc)[MF > 0 ? MF : 1][2]) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int mh = w >> 2, nq = w & 3;
  const bool a_wave = w < 4;
  const int KC = gt.KC;
  const __amdgpu_buffer_rsrc_t rw = rsrc(gt.wbase, gt.wbytes);
  uint8_t* const bstages = lds + kStagesA * kLdsA;
  auto chunk = [&](int c) { return c + gt.k0 < KC ? c + gt.k0 : c + gt.k0 - KC; };
  // A waves: as in gemm_tile_mf (rows past gt.rows are not fetched).
  auto issue_a = [&](int s) {
    uint8_t* buf = lds + (s % kStagesA) * kLdsA;
    const bool in = s < KC;
    const uint32_t k = (uint32_t)chunk(s) * (kAtomK * 2);
#pragma unroll
    for (int i = 0; i < 8; i++)
      if (32 * w + 4 * i < gt.rows)
        lds_load16(ra, in ? gt.aoff[i] + k : kOOB, buf + (8 * w + i) * 1024);
  };
  // B waves: wave 4 + u loads atoms 2u, 2u+1 of the chunk (8 KB), always
  // kBwLoads instructions (chunks past the end go to the out-of-range offset).
  auto issue_b = [&](int c) {
    uint8_t* buf = bstages + (c % kStagesBw) * kLdsBwB;
    const int u = w - 4;
    const bool in = c < KC;
    const uint32_t k = (uint32_t)chunk(c) * kAtomBytesBF16;
#pragma unroll
    for (int t = 0; t < 8; t++) {
      const int a = 2 * u + (t >> 2), piece = t & 3;
      lds_load16_nt(rw, in ? gt.woff[t >> 2] + k + 1024u * piece + 16u * lane : kOOB,
                 buf + a * kAtomBytesBF16 + piece * 1024);
    }
  };
  auto compute = [&](int s) {
    if constexpr (MF == 0) {
      if (!a_wave) issue_b(s + 2);
    } else {
      const uint8_t* abuf = lds + (s % kStagesA) * kLdsA;
      const uint8_t* bbuf = bstages + (s % kStagesBw) * kLdsBwB;
      const int r = lane & 15;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int slot = ((4 * (lane >> 4) + j) ^ r) & 15;
        bf16x8 a[MF];
#pragma unroll
        for (int i = 0; i < MF; i++)
          a[i] = *reinterpret_cast<const bf16x8*>(abuf + (2 * i + mh) * 4096 + 256 * r + 16 * slot);
        const bf16x8 bg = *reinterpret_cast<const bf16x8*>(bbuf + (2 * nq) * kAtomBytesBF16 + 1024 * j + 16 * lane);
        const bf16x8 bu = *reinterpret_cast<const bf16x8*>(bbuf + (2 * nq + 1) * kAtomBytesBF16 + 1024 * j + 16 * lane);
#pragma unroll
        for (int i = 0; i < MF; i++) {
          acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bg, acc[i][0], 0, 0, 0);
          acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], bu, acc[i][1], 0, 0, 0);
        }
        if (j == 0 && !a_wave) {
          __builtin_amdgcn_sched_barrier(0);
          issue_b(s + 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  // The weights stream from HBM, the token rows mostly from L2: the B waves
  // keep two steps of weights in flight (three stages), the A waves one.
  // Step s writes B stage (s+2) % 3, which step s-1 read: every wave has
  // passed step s's barrier, so none reads it any more.
  if (a_wave) {
    issue_a(0);
  } else {
    issue_b(0);
    issue_b(1);
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int s = 0; s < KC; s++) {
    if (a_wave)
      wait_vmem_all();
    else
      wait_vmem_keep<kBwLoads>();  // step s has landed; step s+1 may still be in flight
    lds_barrier();
    if (a_wave) issue_a(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(s);  // the B waves issue step s+2 inside
  }
  // No buffer-to-LDS write may land after the workgroup has ended.
  wait_vmem_all();
}

template <int MF>
__device__ __forceinline__ void gateup_tile_bw(const GemmTile& gt, __amdgpu_buffer_rsrc_t ra,
                                               uint8_t* lds, uint16_t* __restrict__ h,
                                               size_t lo_plane, int I, size_t row0, int pair) {
  const int lane = threadIdx.x & 63, mh = wave_id() >> 2;
  f32x4 acc[MF > 0 ? MF : 1][2];
#pragma unroll
  for (int i = 0; i < (MF > 0 ? MF : 1); i++) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_tile_bw<MF>(gt, ra, lds, acc);
  if (pair >= I / kAtomRows) return;  // columns past I (the last block's)
#pragma unroll
  for (int i = 0; i < MF; i++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int m = (2 * i + mh) * 16 + 4 * (lane >> 4) + r;
      if (m < gt.rows) {
        const float hv = silu(acc[i][0][r]) * acc[i][1][r];
        const uint16_t hi = __builtin_bit_cast(uint16_t, (__bf16)hv);
        const uint16_t lo = __builtin_bit_cast(uint16_t, (__bf16)(hv - __uint_as_float((uint32_t)hi << 16)));
        const size_t o = (row0 + m) * (size_t)I + (size_t)pair * 16 + (lane & 15);
        h[o] = hi;
        h[lo_plane + o] = lo;
      }
    }
}

// Gate/up + SwiGLU on bf16 experts.  N-block nb covers pairs 4nb .. 4nb+3
// (atoms: row groups 8nb .. 8nb+7, gate and up alternating); h leaves as two
// bf16 planes, lo_plane elements apart, for the down kernel.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void gateup_prefill_bw_kernel(
    GroupArgs g, const uint16_t* x, uint32_t x_bytes, int H, int I, int nbn,
    uint16_t* __restrict__ h, size_t lo_plane) {
  int ti, nb;
  tile_of_block(nbn, &ti, &nb);
  if (ti >= *g.n_tiles) return;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBw];
  const int2 td = g.tiles[ti];
  const int grp = td.x, m0 = td.y;
  const int cnt = g.counts[grp], pos0 = g.offsets[grp];
  const int lane = threadIdx.x & 63, w = wave_id(), nq = w & 3;
  const int ngroups = 2 * I / kAtomRows;
  GemmTile gt;
  gt.wbase = grp < g.E ? g.layerbuf + (size_t)grp * g.stride : g.shared_w;
  gt.KC = H / kAtomK;
  gt.wbytes = (uint32_t)ngroups * (uint32_t)gt.KC * kAtomBytesBF16;
  gt.k0 = nb * gt.KC / nbn;
  gt.rows = min(kBM, cnt - m0);
  clear_loads(gt);
  if (w < 4) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int r = 32 * w + 4 * i + (lane >> 4);
      if (r < gt.rows) gt.aoff[i] = (uint32_t)g.tok[pos0 + m0 + r] * (uint32_t)H * 2u + a_piece(r, lane);
    }
  } else {
    // B wave 4 + u: atoms 2u, 2u+1 = row groups 8nb + 2u, +1 (one pair)
    const uint32_t group_bytes = (uint32_t)gt.KC * kAtomBytesBF16;
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int rg = 8 * nb + 2 * (w - 4) + t;
      gt.woff[t] = (uint32_t)(rg < ngroups ? rg : 0) * group_bytes;
    }
  }
  const __amdgpu_buffer_rsrc_t ra = rsrc(x, x_bytes);
  const size_t row0 = (size_t)(pos0 + m0);
  const int pair = 4 * nb + nq;
#define GUB(N) gateup_tile_bw<N>(gt, ra, lds, h, lo_plane, I, row0, pair)
  MOE_MF_SWITCH(wave_mfrags(gt.rows), GUB)
#undef GUB
}

// ------------------------------------------------- gate/up on NVFP4 weights
// The MXFP4 grouped GEMM tile (gemm_tile_mf: 128 token rows x 512 columns,
// 32 atoms per stage) on NVFP4 atoms: 1024 code bytes as MXFP4, then lane
// l's two E4M3 block scales at 1024 + 2l.  A B stage holds the 32 atoms'
// codes and then their 128-byte scale blocks (36 KB); a B wave fetches its 8
// atoms' scales with one 16-byte load per lane (lane l: atom l/8, bytes
// 16 (l%8)).  The dequant is the exact one of the decode kernels.  Each wave
// holds gate and up of 4 pairs, so h = silu(t_g g) * (t_u u) (t: the
// matrix scales) is formed in registers and stored as two bf16 planes.
constexpr int kLdsNvB = kAtomsPerTile * kAtomData + kAtomsPerTile * 128;    // 36 KB
constexpr int kLdsNv = kStagesA * kLdsA + kStagesB * kLdsNvB;             // 136 KB
static_assert(kLdsNv <= 160 * 1024, "LDS per CU");

template <int MF>
__device__ __forceinline__ void gemm_tile_nv(const GemmTile& gt, __amdgpu_buffer_rsrc_t ra,
                                             uint8_t* lds,
                                             f32x4 (&acc)[MF > 0 ? MF : 1][kFragsPerWave]) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int mh = w >> 2, nq = w & 3;
  const bool a_wave = w < 4;
  const int KC = gt.KC;
  const __amdgpu_buffer_rsrc_t rw = rsrc(gt.wbase, gt.wbytes);
  uint8_t* const bstages = lds + kStagesA * kLdsA;
  constexpr int kScales = kAtomsPerTile * kAtomData;  // scale blocks within a B stage
  auto chunk = [&](int c) { return c + gt.k0 < KC ? c + gt.k0 : c + gt.k0 - KC; };
  auto issue_a = [&](int s) {
    uint8_t* buf = lds + (s % kStagesA) * kLdsA;
    const bool in = s < KC;
    const uint32_t k = (uint32_t)chunk(s) * (kAtomK * 2);
#pragma unroll
    for (int i = 0; i < 8; i++)
      if (32 * w + 4 * i < gt.rows)
        lds_load16(ra, in ? gt.aoff[i] + k : kOOB, buf + (8 * w + i) * 1024);
  };
  // B waves: chunk c into stage c % 2 (codes of atoms 8u .. 8u+7, then
  // their scale blocks).
  auto issue_b = [&](int c) {
    uint8_t* buf = bstages + (c % kStagesB) * kLdsNvB;
    const int u = w - 4;
    const bool in = c < KC;
    const uint32_t k = (uint32_t)chunk(c) * kAtomBytesNV;
#pragma unroll
    for (int t = 0; t < 8; t++)
      lds_load16_nt(rw, in ? gt.woff[t] + k + 16u * lane : kOOB, buf + (8 * u + t) * kAtomData);
    lds_load16_nt(rw, in ? gt.soff[0] + k : kOOB, buf + kScales + 8 * u * 128);
  };
  auto compute = [&](int s) {
    if constexpr (MF == 0) {
      if (!a_wave) issue_b(s + 1);
    } else {
      const uint8_t* abuf = lds + (s % kStagesA) * kLdsA;
      const uint8_t* bbuf = bstages + (s % kStagesB) * kLdsNvB;
      u32x4 wd[kFragsPerWave];
      uint32_t sd[kFragsPerWave];
#pragma unroll
      for (int f = 0; f < kFragsPerWave; f++) {
        const int atom = nq * kFragsPerWave + f;
        wd[f] = *reinterpret_cast<const u32x4*>(bbuf + atom * kAtomData + 16 * lane);
        sd[f] = *reinterpret_cast<const uint16_t*>(bbuf + kScales + atom * 128 + 2 * lane);
      }
      bf16x8 a[2][MF];
      auto fetch = [&](int j, int q) {
        const int r = lane & 15;
        const int slot = ((4 * (lane >> 4) + j) ^ r) & 15;
#pragma unroll
        for (int i = 0; i < MF; i++)
          a[q][i] = *reinterpret_cast<const bf16x8*>(abuf + (2 * i + mh) * 4096 + 256 * r + 16 * slot);
      };
      fetch(0, 0);
#pragma unroll
      for (int j = 0; j < 4; j++) {
        if (j + 1 < 4) fetch(j + 1, (j + 1) & 1);
        const int sh = 8 * (j >> 1);  // steps 0-1: the first block scale, 2-3: the second
        bf16x8 bb[2];
        bb[0] = nvfp4::dequant8_nv(wd[0][j], (sd[0] >> sh) & 0xFFu);
#pragma unroll
        for (int f = 0; f < kFragsPerWave; f++) {
          if (f + 1 < kFragsPerWave) bb[(f + 1) & 1] = nvfp4::dequant8_nv(wd[f + 1][j], (sd[f + 1] >> sh) & 0xFFu);
#pragma unroll
          for (int i = 0; i < MF; i++)
            acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j & 1][i], bb[f & 1], acc[i][f], 0, 0, 0);
        }
        if (j == 0 && !a_wave) {
          __builtin_amdgcn_sched_barrier(0);
          issue_b(s + 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  if (a_wave)
    issue_a(0);
  else
    issue_b(0);
  __builtin_amdgcn_sched_barrier(0);
  for (int s = 0; s < KC; s++) {
    wait_vmem_all();
    lds_barrier();
    if (a_wave) issue_a(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(s);  // the B waves issue step s+1 inside
  }
  wait_vmem_all();
}

template <int MF>
__device__ __forceinline__ void gateup_tile_nv(const GemmTile& gt, __amdgpu_buffer_rsrc_t ra,
                                               uint8_t* lds, uint16_t* __restrict__ h,
                                               size_t lo_plane, int I, size_t row0, int p0,
                                               float tg, float tu) {
  const int lane = threadIdx.x & 63, mh = wave_id() >> 2;
  f32x4 acc[MF > 0 ? MF : 1][kFragsPerWave];
#pragma unroll
  for (int i = 0; i < (MF > 0 ? MF : 1); i++)
#pragma unroll
    for (int f = 0; f < kFragsPerWave; f++) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_tile_nv<MF>(gt, ra, lds, acc);
#pragma unroll
  for (int q = 0; q < kFragsPerWave / 2; q++) {
    const int pair = p0 + q;
    if (pair >= I / kAtomRows) break;  // columns past I (the last block's)
#pragma unroll
    for (int i = 0; i < MF; i++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = (2 * i + mh) * 16 + 4 * (lane >> 4) + r;
        if (m < gt.rows) {
          const float hv = silu(tg * acc[i][2 * q][r]) * (tu * acc[i][2 * q + 1][r]);
          const uint16_t hi = __builtin_bit_cast(uint16_t, (__bf16)hv);
          const uint16_t lo =
              __builtin_bit_cast(uint16_t, (__bf16)(hv - __uint_as_float((uint32_t)hi << 16)));
          const size_t o = (row0 + m) * (size_t)I + (size_t)pair * 16 + (lane & 15);
          h[o] = hi;
          h[lo_plane + o] = lo;
        }
      }
  }
}

// Gate/up + SwiGLU on NVFP4 experts: n-block nb and column quarters as in
// gateup_prefill_kernel; h leaves as two bf16 planes for the down kernel.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void gateup_prefill_nv_kernel(
    GroupArgs g, const uint16_t* x, uint32_t x_bytes, int H, int I, int nbn, size_t ms_off,
    uint16_t* __restrict__ h, size_t lo_plane) {
  int ti, nb;
  tile_of_block(nbn, &ti, &nb);
  if (ti >= *g.n_tiles) return;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsNv];
  const int2 td = g.tiles[ti];
  const int grp = td.x, m0 = td.y;
  const int cnt = g.counts[grp], pos0 = g.offsets[grp];
  const int lane = threadIdx.x & 63, w = wave_id(), nq = w & 3;
  const int ngroups = 2 * I / kAtomRows;
  const uint8_t* rec = grp < g.E ? g.layerbuf + (size_t)grp * g.stride : g.shared_w;
  GemmTile gt;
  gt.wbase = rec;
  gt.KC = H / kAtomK;
  gt.wbytes = (uint32_t)ngroups * (uint32_t)gt.KC * kAtomBytesNV;
  gt.k0 = nb * gt.KC / nbn;
  gt.rows = min(kBM, cnt - m0);
  clear_loads(gt);
  if (w < 4) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int r = 32 * w + 4 * i + (lane >> 4);
      if (r < gt.rows) gt.aoff[i] = (uint32_t)g.tok[pos0 + m0 + r] * (uint32_t)H * 2u + a_piece(r, lane);
    }
  } else {
    // atoms 8(w-4) + t of the tile: row groups 32nb + 8(w-4) + t; groups
    // past the matrix (the last, partial block) read group 0
    const uint32_t group_bytes = (uint32_t)gt.KC * kAtomBytesNV;
    const int rg0 = nb * 32 + 8 * (w - 4);
#pragma unroll
    for (int t = 0; t < 8; t++)
      gt.woff[t] = (uint32_t)(rg0 + t < ngroups ? rg0 + t : 0) * group_bytes;
    const int rs = rg0 + (lane >> 3);
    gt.soff[0] = (uint32_t)(rs < ngroups ? rs : 0) * group_bytes + kAtomData + 16u * (lane & 7);
  }
  const float* ms = reinterpret_cast<const float*>(rec + ms_off);
  const float tg = ms[0], tu = ms[1];
  const __amdgpu_buffer_rsrc_t ra = rsrc(x, x_bytes);
  const size_t row0 = (size_t)(pos0 + m0);
  const int p0 = nb * 16 + 4 * nq;
#define GUN(N) gateup_tile_nv<N>(gt, ra, lds, h, lo_plane, I, row0, p0, tg, tu)
  MOE_MF_SWITCH(wave_mfrags(gt.rows), GUN)
#undef GUN
}

// --------------------------------------------------- down on NVFP4 weights
// Down GEMM tile for NVFP4 experts: C[128 rows][128 columns of H] over K = I
// in chunks of 128, A = h as its two bf16 planes (hi and lo, each swizzled
// as the A stage of gemm_tile_mf), B = 8 NVFP4 atoms (row groups of H) with
// their scale blocks.  Every weight fragment meets both planes, so h's
// 16 significant bits reach the sums, as in the decode kernels.  Wave w owns
// atoms 2(w%4), 2(w%4)+1 and fragments 2i + w/4.
constexpr int kNvdAtoms = 8;
constexpr int kLdsNvdA = 2 * kLdsA;                                     // hi, lo: 64 KB
constexpr int kLdsNvdB = kNvdAtoms * kAtomData + kNvdAtoms * 128;       // 9 KB
constexpr int kLdsNvd = kStagesA * kLdsNvdA + kStagesB * kLdsNvdB;      // 146 KB
static_assert(kLdsNvd <= 160 * 1024, "LDS per CU");

template <int MF>
__device__ __forceinline__ void gemm_tile_nvd(const GemmTile& gt, __amdgpu_buffer_rsrc_t ra,
                                              uint32_t lo_bytes, uint8_t* lds,
                                              f32x4 (&acc)[MF > 0 ? MF : 1][2]) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int mh = w >> 2, nq = w & 3;
  const bool a_wave = w < 4;
  const int KC = gt.KC;
  const __amdgpu_buffer_rsrc_t rw = rsrc(gt.wbase, gt.wbytes);
  uint8_t* const bstages = lds + kStagesA * kLdsNvdA;
  constexpr int kScales = kNvdAtoms * kAtomData;
  auto chunk = [&](int c) { return c + gt.k0 < KC ? c + gt.k0 : c + gt.k0 - KC; };
  // A waves: rows 32w .. 32w+31 of both planes (16 loads).
  auto issue_a = [&](int s) {
    uint8_t* buf = lds + (s % kStagesA) * kLdsNvdA;
    const bool in = s < KC;
    const uint32_t k = (uint32_t)chunk(s) * (kAtomK * 2);
#pragma unroll
    for (int pl = 0; pl < 2; pl++)
#pragma unroll
      for (int i = 0; i < 8; i++)
        if (32 * w + 4 * i < gt.rows)
          lds_load16(ra, in ? gt.aoff[i] + k + (pl ? lo_bytes : 0u) : kOOB,
                     buf + pl * kLdsA + (8 * w + i) * 1024);
  };
  // B waves: wave 4 + u loads atoms 2u, 2u+1 (codes) and their two scale
  // blocks (one 4-byte load a lane: 256 bytes).
  auto issue_b = [&](int c) {
    uint8_t* buf = bstages + (c % kStagesB) * kLdsNvdB;
    const int u = w - 4;
    const bool in = c < KC;
    const uint32_t k = (uint32_t)chunk(c) * kAtomBytesNV;
#pragma unroll
    for (int t = 0; t < 2; t++)
      lds_load16_nt(rw, in ? gt.woff[t] + k + 16u * lane : kOOB, buf + (2 * u + t) * kAtomData);
    lds_load4_nt(rw, in ? gt.soff[0] + k : kOOB, buf + kScales + 2 * u * 128);
  };
  auto compute = [&](int s) {
    if constexpr (MF == 0) {
      if (!a_wave) issue_b(s + 1);
    } else {
      const uint8_t* abuf = lds + (s % kStagesA) * kLdsNvdA;
      const uint8_t* bbuf = bstages + (s % kStagesB) * kLdsNvdB;
      u32x4 wd[2];
      uint32_t sd[2];
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int atom = 2 * nq + t;
        wd[t] = *reinterpret_cast<const u32x4*>(bbuf + atom * kAtomData + 16 * lane);
        sd[t] = *reinterpret_cast<const uint16_t*>(bbuf + kScales + atom * 128 + 2 * lane);
      }
      const int r = lane & 15;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int slot = ((4 * (lane >> 4) + j) ^ r) & 15;
        const int sh = 8 * (j >> 1);
        bf16x8 bb[2];
#pragma unroll
        for (int t = 0; t < 2; t++) bb[t] = nvfp4::dequant8_nv(wd[t][j], (sd[t] >> sh) & 0xFFu);
#pragma unroll
        for (int i = 0; i < MF; i++) {
          const uint8_t* row = abuf + (2 * i + mh) * 4096 + 256 * r + 16 * slot;
          const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(row);
          const bf16x8 alo = *reinterpret_cast<const bf16x8*>(row + kLdsA);
#pragma unroll
          for (int t = 0; t < 2; t++) {
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bb[t], acc[i][t], 0, 0, 0);
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bb[t], acc[i][t], 0, 0, 0);
          }
        }
        if (j == 0 && !a_wave) {
          __builtin_amdgcn_sched_barrier(0);
          issue_b(s + 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  if (a_wave)
    issue_a(0);
  else
    issue_b(0);
  __builtin_amdgcn_sched_barrier(0);
  for (int s = 0; s < KC; s++) {
    wait_vmem_all();
    lds_barrier();
    if (a_wave) issue_a(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(s);
  }
  wait_vmem_all();
}

template <int MF>
__device__ __forceinline__ void down_tile_nvd(const GemmTile& gt, __amdgpu_buffer_rsrc_t ra,
                                              uint32_t lo_bytes, uint8_t* lds,
                                              float* __restrict__ yperm, int H, size_t row0,
                                              int rg0, float td) {
  const int lane = threadIdx.x & 63, mh = wave_id() >> 2;
  f32x4 acc[MF > 0 ? MF : 1][2];
#pragma unroll
  for (int i = 0; i < (MF > 0 ? MF : 1); i++) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_tile_nvd<MF>(gt, ra, lo_bytes, lds, acc);
#pragma unroll
  for (int i = 0; i < MF; i++)
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = (2 * i + mh) * 16 + 4 * (lane >> 4) + r;
        if (m < gt.rows)
          yperm[(row0 + m) * H + (rg0 + t) * 16 + (lane & 15)] = td * acc[i][t][r];
      }
}

// Down on NVFP4 experts.  N-block nb covers row groups 8nb .. 8nb+7 of H
// (128 columns); A is h's two bf16 planes (lo_bytes apart).
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void down_prefill_nv_kernel(
    GroupArgs g, const uint16_t* h, uint32_t h_bytes, uint32_t lo_bytes, int H, int I, int nbn,
    size_t gateup_bytes, size_t ms_off, float* __restrict__ yperm) {
  int ti, nb;
  tile_of_block(nbn, &ti, &nb);
  if (ti >= *g.n_tiles) return;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsNvd];
  const int2 td = g.tiles[ti];
  const int grp = td.x, m0 = td.y;
  const int cnt = g.counts[grp], pos0 = g.offsets[grp];
  const int lane = threadIdx.x & 63, w = wave_id(), nq = w & 3;
  const int ngroups = H / kAtomRows;  // a multiple of 8: no partial block
  const uint8_t* rec = grp < g.E ? g.layerbuf + (size_t)grp * g.stride : g.shared_w;
  GemmTile gt;
  gt.wbase = rec + gateup_bytes;
  gt.KC = I / kAtomK;
  gt.wbytes = (uint32_t)ngroups * (uint32_t)gt.KC * kAtomBytesNV;
  gt.k0 = nb * gt.KC / nbn;
  gt.rows = min(kBM, cnt - m0);
  clear_loads(gt);
  if (w < 4) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int r = 32 * w + 4 * i + (lane >> 4);
      if (r < gt.rows) gt.aoff[i] = (uint32_t)(pos0 + m0 + r) * (uint32_t)I * 2u + a_piece(r, lane);
    }
  } else {
    const uint32_t group_bytes = (uint32_t)gt.KC * kAtomBytesNV;
    const int rgb = 8 * nb + 2 * (w - 4);
#pragma unroll
    for (int t = 0; t < 2; t++) gt.woff[t] = (uint32_t)(rgb + t) * group_bytes;
    // lane l: atom rgb + l/32, bytes 4 (l%32) of its scale block
    gt.soff[0] = (uint32_t)(rgb + (lane >> 5)) * group_bytes + kAtomData + 4u * (lane & 31);
  }
  const float tdn = reinterpret_cast<const float*>(rec + ms_off)[2];
  const __amdgpu_buffer_rsrc_t ra = rsrc(h, h_bytes);
  const size_t row0 = (size_t)(pos0 + m0);
  const int rg0 = 8 * nb + 2 * nq;
#define DNN(N) down_tile_nvd<N>(gt, ra, lo_bytes, lds, yperm, H, row0, rg0, tdn)
  MOE_MF_SWITCH(wave_mfrags(gt.rows), DNN)
#undef DNN
}

// ----------------------------------------------------- down on bf16 weights
// As gemm_tile_nvd with bf16 atoms (4 KB): 4 atoms (64 columns of H) per
// tile, so that two stages of h's two planes (64 KB each) and of the atoms
// (16 KB each) fill the 160 KB of LDS; wave w owns atom w%4.
constexpr int kBwdAtoms = 4;
constexpr int kLdsBwdB = kBwdAtoms * kAtomBytesBF16;                    // 16 KB
constexpr int kLdsBwd = kStagesA * kLdsNvdA + kStagesB * kLdsBwdB;      // 160 KB
static_assert(kLdsBwd <= 160 * 1024, "LDS per CU");

template <int MF>
__device__ __forceinline__ void gemm_tile_bwd(const GemmTile& gt, __amdgpu_buffer_rsrc_t ra,
                                              uint32_t lo_bytes, uint8_t* lds,
                                              f32x4 (&acc)[MF > 0 ? MF : 1]) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int mh = w >> 2, nq = w & 3;
  const bool a_wave = w < 4;
  const int KC = gt.KC;
  const __amdgpu_buffer_rsrc_t rw = rsrc(gt.wbase, gt.wbytes);
  uint8_t* const bstages = lds + kStagesA * kLdsNvdA;
  auto chunk = [&](int c) { return c + gt.k0 < KC ? c + gt.k0 : c + gt.k0 - KC; };
  auto issue_a = [&](int s) {
    uint8_t* buf = lds + (s % kStagesA) * kLdsNvdA;
    const bool in = s < KC;
    const uint32_t k = (uint32_t)chunk(s) * (kAtomK * 2);
#pragma unroll
    for (int pl = 0; pl < 2; pl++)
#pragma unroll
      for (int i = 0; i < 8; i++)
        if (32 * w + 4 * i < gt.rows)
          lds_load16(ra, in ? gt.aoff[i] + k + (pl ? lo_bytes : 0u) : kOOB,
                     buf + pl * kLdsA + (8 * w + i) * 1024);
  };
  // B waves: wave 4 + u loads atom u (four 1 KB pieces).
  auto issue_b = [&](int c) {
    uint8_t* buf = bstages + (c % kStagesB) * kLdsBwdB;
    const int u = w - 4;
    const bool in = c < KC;
    const uint32_t k = (uint32_t)chunk(c) * kAtomBytesBF16;
#pragma unroll
    for (int piece = 0; piece < 4; piece++)
      lds_load16_nt(rw, in ? gt.woff[0] + k + 1024u * piece + 16u * lane : kOOB,
                 buf + u * kAtomBytesBF16 + piece * 1024);
  };
  auto compute = [&](int s) {
    if constexpr (MF == 0) {
      if (!a_wave) issue_b(s + 1);
    } else {
      const uint8_t* abuf = lds + (s % kStagesA) * kLdsNvdA;
      const uint8_t* bbuf = bstages + (s % kStagesB) * kLdsBwdB;
      const int r = lane & 15;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int slot = ((4 * (lane >> 4) + j) ^ r) & 15;
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(bbuf + nq * kAtomBytesBF16 + 1024 * j + 16 * lane);
#pragma unroll
        for (int i = 0; i < MF; i++) {
          const uint8_t* row = abuf + (2 * i + mh) * 4096 + 256 * r + 16 * slot;
          const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(row);
          const bf16x8 alo = *reinterpret_cast<const bf16x8*>(row + kLdsA);
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, acc[i], 0, 0, 0);
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, acc[i], 0, 0, 0);
        }
        if (j == 0 && !a_wave) {
          __builtin_amdgcn_sched_barrier(0);
          issue_b(s + 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  if (a_wave)
    issue_a(0);
  else
    issue_b(0);
  __builtin_amdgcn_sched_barrier(0);
  for (int s = 0; s < KC; s++) {
    wait_vmem_all();
    lds_barrier();
    if (a_wave) issue_a(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(s);
  }
  wait_vmem_all();
}

template <int MF>
__device__ __forceinline__ void down_tile_bwd(const GemmTile& gt, __amdgpu_buffer_rsrc_t ra,
                                              uint32_t lo_bytes, uint8_t* lds,
                                              float* __restrict__ yperm, int H, size_t row0,
                                              int rg) {
  const int lane = threadIdx.x & 63, mh = wave_id() >> 2;
  f32x4 acc[MF > 0 ? MF : 1];
#pragma unroll
  for (int i = 0; i < (MF > 0 ? MF : 1); i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_tile_bwd<MF>(gt, ra, lo_bytes, lds, acc);
#pragma unroll
  for (int i = 0; i < MF; i++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int m = (2 * i + mh) * 16 + 4 * (lane >> 4) + r;
      if (m < gt.rows) yperm[(row0 + m) * H + rg * 16 + (lane & 15)] = acc[i][r];
    }
}

// Down on bf16 experts.  N-block nb covers row groups 4nb .. 4nb+3 of H.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void down_prefill_bw_kernel(
    GroupArgs g, const uint16_t* h, uint32_t h_bytes, uint32_t lo_bytes, int H, int I, int nbn,
    size_t gateup_bytes, float* __restrict__ yperm) {
  int ti, nb;
  tile_of_block(nbn, &ti, &nb);
  if (ti >= *g.n_tiles) return;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBwd];
  const int2 td = g.tiles[ti];
  const int grp = td.x, m0 = td.y;
  const int cnt = g.counts[grp], pos0 = g.offsets[grp];
  const int lane = threadIdx.x & 63, w = wave_id(), nq = w & 3;
  const int ngroups = H / kAtomRows;
  GemmTile gt;
  gt.wbase = (grp < g.E ? g.layerbuf + (size_t)grp * g.stride : g.shared_w) + gateup_bytes;
  gt.KC = I / kAtomK;
  gt.wbytes = (uint32_t)ngroups * (uint32_t)gt.KC * kAtomBytesBF16;
  gt.k0 = nb * gt.KC / nbn;
  gt.rows = min(kBM, cnt - m0);
  clear_loads(gt);
  if (w < 4) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int r = 32 * w + 4 * i + (lane >> 4);
      if (r < gt.rows) gt.aoff[i] = (uint32_t)(pos0 + m0 + r) * (uint32_t)I * 2u + a_piece(r, lane);
    }
  } else {
    gt.woff[0] = (uint32_t)(4 * nb + (w - 4)) * (uint32_t)gt.KC * kAtomBytesBF16;
  }
  const __amdgpu_buffer_rsrc_t ra = rsrc(h, h_bytes);
  const size_t row0 = (size_t)(pos0 + m0);
#define DNB(N) down_tile_bwd<N>(gt, ra, lo_bytes, lds, yperm, H, row0, 4 * nb + nq)
  MOE_MF_SWITCH(wave_mfrags(gt.rows), DNB)
#undef DNB
}

// ------------------------------------------------------- native-MX GEMMs
// The opt-in MXFP8 prefill mode (moe_config.prefill_format): both expert
// matrices on v_mfma_scale_f32_16x16x128_f8f6f4 with the activations block-
// quantised to MXFP8 (E4M3 elements, one E8M0 scale per 32 along K; OCP MX
// scale rule, nearest-even rounding clamped to +-448) and the MXFP4 weight
// atoms taken as stored: no dequantisation, one MFMA per 16 rows x 16
// columns x 128 K, half the activation bytes of the bf16 path.
//
// Activation stage in LDS (per K chunk of 128): fragment g (tile rows
// 16g .. 16g+15) is 2 KB laid out as the MFMA operand wants it: lane L's 32
// codes (row L%16, MX block L/16 of the chunk) as two 16-byte halves at
// 16L and 1024 + 16L, so each half is one conflict-free 16-byte read per
// lane.  A buffer-to-LDS load fills one half of one fragment (lane j fetches
// row 16g + j%16, block j/16, half h of the gathered row).  The 128 rows'
// scale bytes follow as [row][4 blocks] (one 4-byte load per row).
constexpr int kMxFrag = 2048;
constexpr int kMxCodes = 8 * kMxFrag;                    // 16 KB per stage
constexpr int kMxAStage = kMxCodes + kBM * 4;            // + 512 B of scales
constexpr int kStagesMxB = 3;                             // weights two steps ahead
constexpr int kMxBLoads = 10;                             // per B wave and step
constexpr int kLdsMx = kStagesA * kMxAStage + kStagesMxB * kLdsBStage;   // 135 KB
constexpr int kLdsMxGateUp = kLdsMx > 8 * kEpiWave ? kLdsMx : 8 * kEpiWave;
static_assert(kLdsMxGateUp <= 160 * 1024, "LDS per CU");

typedef short s16x2 __attribute__((ext_vector_type(2)));

// MXFP8 block quantisation of 32 fp32 values: exponent e = floor(log2 amax)
// - 8 clamped to [-127, 127] (-127 for an all-zero block); codes of
// v * 2^-e (exact: a power-of-two scaling that stays finite for fp32 inputs,
// since e <= 119 there) clamped to +-448 and converted to nearest E4M3 with
// the hardware convert at scale 1.  Element i goes to byte i of `codes`.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.0f)) return -127;
  const uint32_t b = __float_as_uint(amax);
  const int ex = (int)((b >> 23) & 0xFFu);
  const int fl = ex ? ex - 127 : -149 + (31 - __builtin_clz(b & 0x7FFFFFu));
  const int e = fl - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
__device__ __forceinline__ uint32_t mx_quant32(const float (&v)[32], uint32_t (&codes)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int t = 0; t < 32; t++) amax = fmaxf(amax, fabsf(v[t]));
  const int e = mx_exponent(amax);
  const float inv = ldexpf(1.0f, -e);
#pragma unroll
  for (int q = 0; q < 8; q++) {
    float t[4];
#pragma unroll
    for (int u = 0; u < 4; u++) t[u] = fminf(fmaxf(v[4 * q + u] * inv, -448.0f), 448.0f);
    s16x2 r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, t[0], t[1], 1.0f, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, t[2], t[3], 1.0f, true);
    codes[q] = __builtin_bit_cast(uint32_t, r);
  }
  return (uint32_t)(e + 127);
}

// x [T][H] bf16 -> codes [T][H] and scale bytes [T][H/32]: one thread per
// block of 32.
__global__ __launch_bounds__(256) void quantize_x_mx_kernel(const uint16_t* __restrict__ x,
                                                            int n_blocks,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int blk = blockIdx.x * blockDim.x + threadIdx.x;
  if (blk >= n_blocks) return;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)blk * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const u32x4 w = src[q];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      v[8 * q + 2 * u] = __uint_as_float(w[u] << 16);
      v[8 * q + 2 * u + 1] = __uint_as_float(w[u] & 0xFFFF0000u);
    }
  }
  uint32_t c[8];
  scales[blk] = (uint8_t)mx_quant32(v, c);
  u32x4* dst = reinterpret_cast<u32x4*>(codes + (size_t)blk * 32);
  dst[0] = u32x4{c[0], c[1], c[2], c[3]};
  dst[1] = u32x4{c[4], c[5], c[6], c[7]};
}

struct MxTile {
  const uint8_t* wbase;  // expert section start (gate/up or down)
  uint32_t wbytes;       // section bytes
  int KC;                // K chunks
  int k0;                // first K chunk of the walk
  int rows;              // valid rows in this tile
  uint32_t aoff[4];      // A waves: lane's piece of fragments 2w, 2w+1, halves 0, 1 (chunk 0)
  uint32_t asoff;        // waves 0, 1: lane's row scale word (row 64w + lane, chunk 0)
  uint32_t woff[8];      // B waves, as GemmTile
  uint32_t soff[2];
};

// Chaining (a workgroup that runs several tiles in turn): nx is the next
// tile of the same workgroup when `chain` (the same K; KC >= 2), and its
// steps 0 and 1 are issued by this tile's last steps in place of the loads
// past the end, so they land while this tile's epilogue runs; `pre` says that
// this tile's own first steps were issued that way.  sa and sb are the A and
// B stages of this tile's step 0: the stage rings run on across tiles.
template <int MF>
__device__ __forceinline__ void gemm_tile_mx(const MxTile& gt, const MxTile& nx, bool chain,
                                             bool pre, int sa, int sb, __amdgpu_buffer_rsrc_t ra,
                                             __amdgpu_buffer_rsrc_t rs, uint8_t* lds,
                                             f32x4 (&acc)[MF > 0 ? MF : 1][kFragsPerWave]) {
  const int lane = threadIdx.x & 63, w = wave_id();
  const int mh = w >> 2, nq = w & 3;
  const bool a_wave = w < 4;
  const int KC = gt.KC;
  const __amdgpu_buffer_rsrc_t rw = rsrc(gt.wbase, gt.wbytes);
  uint8_t* const bstages = lds + kStagesA * kMxAStage;
  auto chunk_of = [&](const MxTile& t, int c) { return c + t.k0 < KC ? c + t.k0 : c + t.k0 - KC; };
  // A waves: step s into stage (sa + s) % 2 (fragments 2w, 2w+1 that hold
  // rows; waves 0 and 1 also the scale words of rows 64w .. 64w+63); step KC
  // is the next tile's step 0 when chained.
  auto issue_a = [&](int s) {
    uint8_t* buf = lds + ((sa + s) % kStagesA) * kMxAStage;
    const bool nxt = s >= KC && chain;
    const MxTile& t = nxt ? nx : gt;
    const bool in = s < KC || nxt;
    const uint32_t kc = (uint32_t)chunk_of(t, nxt ? s - KC : s);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int frag = 2 * w + (i >> 1);
      if (16 * frag < t.rows)
        lds_load16(ra, in ? t.aoff[i] + kc * kAtomK : kOOB, buf + frag * kMxFrag + (i & 1) * 1024);
    }
    if (w < 2 && 64 * w < t.rows)
      lds_load4(rs, in ? t.asoff + kc * 4u : kOOB, buf + kMxCodes + 256 * w);
  };
  // B waves: always kMxBLoads instructions (chunks past the end go to the
  // out-of-range offset, or, chained, are the next tile's chunks 0 and 1).
  auto issue_b = [&](int c) {
    uint8_t* buf = bstages + ((sb + c) % kStagesMxB) * kLdsBStage;
    const int u = w - 4;
    const bool nxt = c >= KC && chain;
    const MxTile& t = nxt ? nx : gt;
    const __amdgpu_buffer_rsrc_t rb = nxt ? rsrc(nx.wbase, nx.wbytes) : rw;
    const bool in = c < KC || nxt;
    const uint32_t k = (uint32_t)chunk_of(t, nxt ? c - KC : c) * kAtomBytes;
#pragma unroll
    for (int q = 0; q < 8; q++)
      lds_load16_nt(rb, in ? t.woff[q] + k + 16u * lane : kOOB, buf + (8 * u + q) * kAtomData);
#pragma unroll
    for (int hh = 0; hh < 2; hh++)
      lds_load4_nt(rb, in ? t.soff[hh] + k : kOOB, buf + kLdsBc + (8 * u + 4 * hh) * 64);
  };
  auto compute = [&](int s) {
    if constexpr (MF == 0) {
      if (!a_wave) issue_b(s + 2);
    } else {
      const uint8_t* abuf = lds + ((sa + s) % kStagesA) * kMxAStage;
      const uint8_t* bbuf = bstages + ((sb + s) % kStagesMxB) * kLdsBStage;
      i32x8 a8[MF];
      int as[MF];
#pragma unroll
      for (int i = 0; i < MF; i++) {
        const int frag = 2 * i + mh;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(abuf + frag * kMxFrag + 16 * lane);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(abuf + frag * kMxFrag + 1024 + 16 * lane);
        a8[i] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        as[i] = abuf[kMxCodes + 4 * (16 * frag + (lane & 15)) + (lane >> 4)];
      }
#pragma unroll
      for (int f = 0; f < kFragsPerWave; f++) {
        const int atom = nq * kFragsPerWave + f;
        const u32x4 wd = *reinterpret_cast<const u32x4*>(bbuf + atom * kAtomData + 16 * lane);
        const int sd = bbuf[kLdsBc + atom * 64 + lane];
        const i32x8 b8 = {(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3], 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < MF; i++)
          acc[i][f] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              a8[i], b8, acc[i][f], 0 /* A: fp8 E4M3 */, 4 /* B: fp4 E2M1 */, 0, as[i], 0, sd);
        if (f == 1 && !a_wave) {
          __builtin_amdgcn_sched_barrier(0);
          issue_b(s + 2);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };
  // Weights three stages deep, as in gemm_tile_bw; the A waves' load count
  // depends on the tile's rows, so they keep one step in flight.  A chained
  // tile's first wait is a full one: the previous tile's epilogue stores are
  // counted too.
  if (!pre) {
    if (a_wave) {
      issue_a(0);
    } else {
      issue_b(0);
      issue_b(1);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  for (int s = 0; s < KC; s++) {
    if (a_wave || (pre && s == 0))
      wait_vmem_all();
    else
      wait_vmem_keep<kMxBLoads>();
    lds_barrier();
    if (a_wave) issue_a(s + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(s);  // the B waves issue step s+2 inside
  }
  // No buffer-to-LDS write may land after the workgroup has ended; the next
  // tile's first loads stay in flight through the epilogue.
  if (!chain) wait_vmem_all();
}

// A-wave offsets of a tile: row r's codes start at rowbase(r), its scale
// bytes at srowbase(r) (both for chunk 0).
//
// 8-bit A operand of the scaled 16x16x128 MFMA: lane l supplies row l % 16;
// with g = l / 16 its bytes 0..15 are K = 16g .. 16g+15 and its bytes 16..31
// K = 64+16g .. 64+16g+15 of the 128-wide chunk (not 32 consecutive K as for
// the 4- and 6-bit formats).  The scale operand of lane l is still that of
// row l % 16, K block l / 16, so the scale of a byte comes from another lane
// than the byte itself.  The low half is loaded into fragment bytes
// [0, 1024), the high half into [1024, 2048).
template <class RowBase, class ScaleBase>
__device__ __forceinline__ void set_mx_loads(MxTile& gt, int lane, RowBase rowbase, ScaleBase srowbase) {
  const int w = wave_id();
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int r = 16 * (2 * w + (i >> 1)) + (lane & 15);
    gt.aoff[i] = r < gt.rows ? rowbase(r) + 16u * (uint32_t)(lane >> 4) + 64u * (uint32_t)(i & 1)
                             : kOOB;
  }
  const int rs = 64 * w + lane;
  gt.asoff = (w < 2 && rs < gt.rows) ? srowbase(rs) : kOOB;
}

template <int MF>
__device__ __forceinline__ void gateup_tile_mx(const MxTile& gt, __amdgpu_buffer_rsrc_t ra,
                                               __amdgpu_buffer_rsrc_t rs, uint8_t* lds,
                                               uint8_t* __restrict__ hq, uint8_t* __restrict__ hs,
                                               int I, size_t row0, int p0) {
  const int npairs = I / kAtomRows;
  const int lane = threadIdx.x & 63, w = wave_id(), mh = w >> 2;
  f32x4 acc[MF > 0 ? MF : 1][kFragsPerWave];
#pragma unroll
  for (int i = 0; i < (MF > 0 ? MF : 1); i++)
#pragma unroll
    for (int f = 0; f < kFragsPerWave; f++) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_tile_mx<MF>(gt, gt, false, false, 0, 0, ra, rs, lds, acc);
  // h = silu(gate) * up through LDS, then one (row, 32-column block) per
  // lane quantised to MXFP8 (as in the bf16 path's epilogue)
  lds_barrier();
  float* ep = reinterpret_cast<float*>(lds + w * kEpiWave);
#pragma unroll
  for (int i = 0; i < MF; i++)
#pragma unroll
    for (int q = 0; q < kFragsPerWave / 2; q++)
#pragma unroll
      for (int r = 0; r < 4; r++)
        ep[(i * 16 + 4 * (lane >> 4) + r) * kEpiStride + 16 * q + (lane & 15)] =
            silu(acc[i][2 * q][r]) * acc[i][2 * q + 1][r];
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave reads its own writes
  const int row = lane & 15, b = (lane >> 4) & 1;
  const bool col_ok = p0 + 2 * b < npairs;
#pragma unroll
  for (int it = 0; it < (MF + 1) / 2; it++) {
    const int i = 2 * it + (lane >> 5);
    const int m = (2 * i + mh) * 16 + row;
    if (i < MF && col_ok && m < gt.rows) {
      const float* src = ep + (i * 16 + row) * kEpiStride + 32 * b;
      float v[32];
#pragma unroll
      for (int t = 0; t < 8; t++) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(src + 4 * t);
        v[4 * t] = x4[0], v[4 * t + 1] = x4[1], v[4 * t + 2] = x4[2], v[4 * t + 3] = x4[3];
      }
      uint32_t c[8];
      const uint32_t sbyte = mx_quant32(v, c);
      const size_t col = (size_t)16 * p0 + 32 * b;
      u32x4* dst = reinterpret_cast<u32x4*>(hq + (row0 + m) * I + col);
      dst[0] = u32x4{c[0], c[1], c[2], c[3]};
      dst[1] = u32x4{c[4], c[5], c[6], c[7]};
      hs[(row0 + m) * (I / 32) + col / 32] = (uint8_t)sbyte;
    }
  }
}

template <int MF>
__device__ __forceinline__ void down_tile_mx(const MxTile& gt, const MxTile& nx, bool chain,
                                             bool pre, int sa, int sb, __amdgpu_buffer_rsrc_t ra,
                                             __amdgpu_buffer_rsrc_t rs, uint8_t* lds,
                                             float* __restrict__ yperm, int H, size_t row0,
                                             int rg0, int ngroups) {
  const int lane = threadIdx.x & 63, mh = wave_id() >> 2;
  f32x4 acc[MF > 0 ? MF : 1][kFragsPerWave];
#pragma unroll
  for (int i = 0; i < (MF > 0 ? MF : 1); i++)
#pragma unroll
    for (int f = 0; f < kFragsPerWave; f++) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};
  gemm_tile_mx<MF>(gt, nx, chain, pre, sa, sb, ra, rs, lds, acc);
#pragma unroll
  for (int i = 0; i < MF; i++)
#pragma unroll
    for (int f = 0; f < kFragsPerWave; f++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int m = (2 * i + mh) * 16 + 4 * (lane >> 4) + r;
        if (m < gt.rows && rg0 + f < ngroups)
          yperm[(row0 + m) * H + (rg0 + f) * 16 + (lane & 15)] = acc[i][f][r];
      }
}

// Gate/up + SwiGLU on MXFP8 activations: tiles as gateup_prefill_kernel; A
// is the quantised token rows (codes [T][H], scales [T][H/32], gathered
// through the permutation); h leaves as MXFP8 (codes [rows][I], scales
// [rows][I/32]) for the down GEMM.
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void gateup_mx_kernel(
    GroupArgs g, const uint8_t* xq, uint32_t xq_bytes, const uint8_t* xs, uint32_t xs_bytes, int H,
    int I, int nbn, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  int ti, nb;
  tile_of_block(nbn, &ti, &nb);
  if (ti >= *g.n_tiles) return;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsMxGateUp];
  const int2 td = g.tiles[ti];
  const int grp = td.x, m0 = td.y;
  const int cnt = g.counts[grp], pos0 = g.offsets[grp];
  const int lane = threadIdx.x & 63, w = wave_id(), nq = w & 3;
  MxTile gt;
  gt.wbase = grp < g.E ? g.layerbuf + (size_t)grp * g.stride : g.shared_w;
  gt.KC = H / kAtomK;
  gt.wbytes = (uint32_t)(2 * I / kAtomRows) * (uint32_t)gt.KC * kAtomBytes;
  gt.k0 = nb * gt.KC / nbn;
  gt.rows = min(kBM, cnt - m0);
  for (int i = 0; i < 4; i++) gt.aoff[i] = kOOB;
  gt.asoff = kOOB;
  GemmTile wl;
  clear_loads(wl);
  if (w < 4) {
    const int32_t* tok = g.tok + pos0 + m0;
    set_mx_loads(gt, lane, [&](int r) { return (uint32_t)tok[r] * (uint32_t)H; },
                 [&](int r) { return (uint32_t)tok[r] * (uint32_t)(H / 32); });
  } else {
    wl.KC = gt.KC;
    set_weight_loads(wl, nb * 32 + 8 * (w - 4), lane, 2 * I / kAtomRows);
  }
  for (int t = 0; t < 8; t++) gt.woff[t] = wl.woff[t];
  gt.soff[0] = wl.soff[0];
  gt.soff[1] = wl.soff[1];
  const __amdgpu_buffer_rsrc_t ra = rsrc(xq, xq_bytes), rs = rsrc(xs, xs_bytes);
  const size_t row0 = (size_t)(pos0 + m0);
  const int p0 = nb * 16 + 4 * nq;
#define GUM(N) gateup_tile_mx<N>(gt, ra, rs, lds, hq, hs, I, row0, p0)
  MOE_MF_SWITCH(wave_mfrags(gt.rows), GUM)
#undef GUM
}

// Down on MXFP8 h: tiles as down_prefill_kernel; A rows are the tile's own
// permuted rows.  A workgroup runs work items blockIdx.x, + gridDim.x, ...
// (grid: one workgroup per CU, a multiple of 8, so every item keeps the XCD
// that tile_of_index gives it) and chains them: the next item's first two
// steps load while this one's epilogue stores its outputs.
struct DownMxItem {
  MxTile t;
  size_t row0;
  int rg0;
};

__device__ __forceinline__ bool down_mx_item(const GroupArgs& g, int L, int nbn, int H, int I,
                                             size_t gateup_bytes, DownMxItem& it) {
  int ti, nb;
  tile_of_index(L, nbn, &ti, &nb);
  if (ti >= *g.n_tiles) return false;
  const int2 td = g.tiles[ti];
  const int grp = td.x, m0 = td.y;
  const int cnt = g.counts[grp], pos0 = g.offsets[grp];
  const int lane = threadIdx.x & 63, w = wave_id(), nq = w & 3;
  const int ngroups = H / kAtomRows;
  MxTile& gt = it.t;
  gt.wbase = (grp < g.E ? g.layerbuf + (size_t)grp * g.stride : g.shared_w) + gateup_bytes;
  gt.KC = I / kAtomK;
  gt.wbytes = (uint32_t)ngroups * (uint32_t)gt.KC * kAtomBytes;
  gt.k0 = nb * gt.KC / nbn;
  gt.rows = min(kBM, cnt - m0);
  for (int i = 0; i < 4; i++) gt.aoff[i] = kOOB;
  gt.asoff = kOOB;
  GemmTile wl;
  clear_loads(wl);
  if (w < 4) {
    const uint32_t base = (uint32_t)(pos0 + m0);
    set_mx_loads(gt, lane, [&](int r) { return (base + (uint32_t)r) * (uint32_t)I; },
                 [&](int r) { return (base + (uint32_t)r) * (uint32_t)(I / 32); });
  } else {
    wl.KC = gt.KC;
    set_weight_loads(wl, nb * 32 + 8 * (w - 4), lane, ngroups);
  }
  for (int t = 0; t < 8; t++) gt.woff[t] = wl.woff[t];
  gt.soff[0] = wl.soff[0];
  gt.soff[1] = wl.soff[1];
  it.row0 = (size_t)(pos0 + m0);
  it.rg0 = nb * 32 + 8 * nq;
  return true;
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void down_mx_kernel(
    GroupArgs g, const uint8_t* hq, uint32_t hq_bytes, const uint8_t* hs, uint32_t hs_bytes, int H,
    int I, int nbn, size_t gateup_bytes, float* __restrict__ yperm) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsMx];
  const int ngroups = H / kAtomRows;
  const int KC = I / kAtomK;
  const __amdgpu_buffer_rsrc_t ra = rsrc(hq, hq_bytes), rs = rsrc(hs, hs_bytes);
  DownMxItem cur, nxt;
  int L = blockIdx.x;
  if (!down_mx_item(g, L, nbn, H, I, gateup_bytes, cur)) return;
  bool pre = false;
  int sa = 0, sb = 0;
  for (;;) {
    // every wave reads the same item list, so the loop is uniform
    const bool more = down_mx_item(g, L + (int)gridDim.x, nbn, H, I, gateup_bytes, nxt);
    const bool chain = more && KC >= 2;
#define DNM(N) \
  down_tile_mx<N>(cur.t, nxt.t, chain, pre, sa, sb, ra, rs, lds, yperm, H, cur.row0, cur.rg0, ngroups)
    MOE_MF_SWITCH(wave_mfrags(cur.t.rows), DNM)
#undef DNM
    if (!more) break;
    // the rings run on; an unchained item issues its own first steps into
    // stages no wave reads any more (they held steps KC-2 and KC-3)
    sa = (sa + KC) % kStagesA;
    sb = (sb + KC) % kStagesMxB;
    pre = chain;
    cur = nxt;
    L += (int)gridDim.x;
  }
}

#undef MOE_MF_SWITCH

template <class T>
hipError_t dalloc(T** p, size_t n) {
  return hipMalloc((void**)p, std::max<size_t>(n, 1) * sizeof(T));
}

hipError_t prefill_alloc(Ctx* c) {
  if (c->pf) return hipSuccess;
  const moe_config& f = c->cfg;
  Prefill* p = new Prefill();
  c->pf = p;
  const int T = f.max_prefill_tokens, E = f.n_experts, k = f.top_k;
  p->Tmax = T;
  p->nchunk_max = (T + kChunkTokens - 1) / kChunkTokens;
  p->max_tiles = prefill_max_tiles(T, k, E);
  const size_t rows = (size_t)T * k + T;
  hipError_t e;
  int n_cu = 0;
  if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, c->device)) !=
      hipSuccess)
    return e;
  p->resident_wgs = std::max(8, n_cu / 8 * 8);
#define PA(ptr, n) \
  if ((e = dalloc(&p->ptr, (n))) != hipSuccess) return e
  const size_t L = f.n_layers;
  PA(logits, (size_t)T * E);
  PA(ids, L * T * k);
  PA(gates, L * T * k);
  PA(chunk_cnt, (size_t)p->nchunk_max * E);
  PA(counts, L * (E + 1));
  PA(offsets, L * (E + 1));
  PA(sorted, L * T * k);
  PA(inv, L * T * k);
  PA(tok, rows);
  PA(tiles, (size_t)p->max_tiles);
  PA(n_tiles, 1);
  // bf16 and NVFP4 experts carry h as two bf16 planes; MXFP4 ones as a
  // bf16 plane and the low-order records
  const bool two_planes = f.weight_format != MOE_WEIGHTS_MXFP4;
  PA(h, (two_planes ? 2 : 1) * rows * f.inter);
  if (!two_planes) PA(hlo, prefill_lo_bytes(T, k, E, f.inter));
  PA(yperm, rows * f.hidden);
#undef PA
  const size_t layer_bytes = (size_t)E * c->stride;
  for (int b = 0; b < 2; b++)
    if ((e = hipMalloc((void**)&c->d_layerbuf[b], layer_bytes)) != hipSuccess) return e;
  for (int b = 0; b < 2; b++) {
    if ((e = hipEventCreateWithFlags(&c->ev_upload[b], hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&c->ev_compute[b], hipEventDisableTiming)) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

void prefill_free(Ctx* c) {
  if (Prefill* p = c->pf) {
    void* ptrs[] = {p->logits, p->ids, p->gates, p->chunk_cnt, p->counts, p->offsets, p->sorted,
                    p->inv, p->tok, p->tiles, p->n_tiles, p->h, p->hlo, p->yperm, p->xq};
    for (void* q : ptrs)
      if (q) (void)hipFree(q);
    delete p;
    c->pf = nullptr;
  }
  for (int b = 0; b < 2; b++) {
    if (c->d_layerbuf[b]) (void)hipFree(c->d_layerbuf[b]);
    c->d_layerbuf[b] = nullptr;
    if (c->ev_upload[b]) (void)hipEventDestroy(c->ev_upload[b]);
    if (c->ev_compute[b]) (void)hipEventDestroy(c->ev_compute[b]);
    c->ev_upload[b] = c->ev_compute[b] = nullptr;
  }
}

int prefill_layers_run(const Ctx* c) { return c->pf ? c->pf->last_layers : 0; }

hipError_t prefill_inspect(Ctx* c, int layer, int32_t* T, int32_t* ids, float* gates,
                           int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* inv) {
  *T = c->pf ? c->pf->last_T : 0;
  if (!c->pf || !*T) return hipSuccess;
  Prefill* p = c->pf;
  hipError_t e = hipDeviceSynchronize();
  const int E = c->cfg.n_experts;
  const size_t n = (size_t)*T * c->cfg.top_k, per = (size_t)p->Tmax * c->cfg.top_k;
  const size_t lo = (size_t)layer * per, lg = (size_t)layer * (E + 1);
  auto get = [&](void* dst, const void* src, size_t bytes) {
    if (e == hipSuccess && dst && bytes) e = hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
  };
  get(ids, p->ids + lo, n * 4);
  get(gates, p->gates + lo, n * 4);
  get(counts, p->counts + lg, (size_t)E * 4);
  get(offsets, p->offsets + lg, (size_t)(E + 1) * 4);
  get(sorted, p->sorted + lo, n * 4);
  get(inv, p->inv + lo, n * 4);
  return e;
}

int prefill_last_mx(const Ctx* c) { return c->pf && c->pf->last_T ? c->pf->last_mx : -1; }

hipError_t prefill_inspect_mx(Ctx* c, int32_t* T, uint8_t* xq, uint8_t* xs, uint8_t* hq,
                              uint8_t* hs) {
  *T = c->pf ? c->pf->last_T : 0;
  if (!c->pf || !*T || !c->pf->last_mx) return hipSuccess;
  Prefill* p = c->pf;
  hipError_t e = hipDeviceSynchronize();
  const moe_config& f = c->cfg;
  const int H = f.hidden, I = f.inter, k = f.top_k;
  const size_t rows = (size_t)*T * k + (f.has_shared ? *T : 0);
  const size_t rows_cap = (size_t)p->Tmax * (k + 1);
  const uint8_t* h8 = reinterpret_cast<const uint8_t*>(p->h);
  auto get = [&](void* dst, const void* src, size_t bytes) {
    if (e == hipSuccess && dst && bytes) e = hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
  };
  get(xq, p->xq, (size_t)*T * H);
  get(xs, p->xq + (size_t)p->Tmax * H, (size_t)*T * (H / 32));
  get(hq, h8, rows * I);
  get(hs, h8 + rows_cap * I, rows * (I / 32));
  return e;
}

hipError_t prefill_forward(Ctx* c, int n_layers, const void* const* xs, int T,
                           const float* const* biases, void* const* ys, float* const* y32s,
                           hipStream_t st) {
  hipError_t e = prefill_alloc(c);
  if (e != hipSuccess) {
    prefill_free(c);
    return e;
  }
  Prefill* p = c->pf;
  const moe_config& f = c->cfg;
  const int H = f.hidden, I = f.inter, E = f.n_experts, k = f.top_k;
  const bool mx = c->prefill_format == MOE_PREFILL_MXFP8;
  if (mx && !p->xq &&
      (e = hipMalloc((void**)&p->xq, (size_t)p->Tmax * H + (size_t)p->Tmax * (H / 32))) != hipSuccess) {
    p->xq = nullptr;
    return e;
  }
  p->last_T = T;
  p->last_layers = n_layers;
  p->last_mx = mx;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if ((e = hipStreamIsCapturing(st, &cs)) != hipSuccess) return e;
  const bool debug_sync = (c->debug_flags & MOE_DEBUG_SYNC) && cs == hipStreamCaptureStatusNone;
  const size_t layer_bytes = (size_t)E * c->stride;
  const int nchunk = (T + kChunkTokens - 1) / kChunkTokens;

  // Uploads wait for everything already on the caller's stream (an earlier
  // call may still read the layer buffers).
  hipEvent_t entry = c->ev_compute[0];
  if ((e = hipEventRecord(entry, st)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(c->copy_stream, entry, 0)) != hipSuccess) return e;
  if ((e = hipMemcpyAsync(c->d_layerbuf[0], c->pool, layer_bytes, hipMemcpyHostToDevice,
                          c->copy_stream)) != hipSuccess)
    return e;
  if ((e = hipEventRecord(c->ev_upload[0], c->copy_stream)) != hipSuccess) return e;

  for (int l = 0; l < n_layers; l++) {
    const int b = l & 1;
    if (l + 1 < n_layers) {
      // buffer b^1 was last read by layer l-1
      if (l >= 1 && (e = hipStreamWaitEvent(c->copy_stream, c->ev_compute[b ^ 1], 0)) != hipSuccess)
        return e;
      if ((e = hipMemcpyAsync(c->d_layerbuf[b ^ 1], c->pool + (size_t)(l + 1) * layer_bytes,
                              layer_bytes, hipMemcpyHostToDevice, c->copy_stream)) != hipSuccess)
        return e;
      if ((e = hipEventRecord(c->ev_upload[b ^ 1], c->copy_stream)) != hipSuccess) return e;
    }
    if ((e = hipStreamWaitEvent(st, c->ev_upload[b], 0)) != hipSuccess) return e;

    const uint16_t* x = (const uint16_t*)xs[l];
    const float* bias = biases ? biases[l] : nullptr;
    const float* wrt = c->d_router + (size_t)l * H * E;
    // this layer's routing arrays
    const size_t per = (size_t)p->Tmax * k;
    int32_t* ids = p->ids + l * per;
    float* gates = p->gates + l * per;
    int32_t* sorted = p->sorted + l * per;
    int32_t* inv = p->inv + l * per;
    int32_t* counts = p->counts + (size_t)l * (E + 1);
    int32_t* offsets = p->offsets + (size_t)l * (E + 1);
    Ctx::TimingRec tr{};
    const bool timed = c->timing && c->t_prefill.size() < 65536;
    if (timed)
      for (int i = 0; i < 2 * kPrefillStages; i++)
        if (!(tr.ev[i] = timing_event(c))) return hipErrorOutOfMemory;
    auto t0 = [&](int stage) { return timed ? tr.ev[2 * stage] : nullptr; };
    auto t1 = [&](int stage) { return timed ? tr.ev[2 * stage + 1] : nullptr; };
    // the routing stage runs from its first kernel's start to the dispatch's
    // end; in the MXFP8 mode it starts with the quantisation of x
    uint8_t* const xs = p->xq ? p->xq + (size_t)p->Tmax * H : nullptr;
    if (mx) {
      const int nblk = T * (H / 32);
      MOE_LAUNCH(quantize_x_mx_kernel, (nblk + 255) / 256, 256, 0, st, t0(kPfRouting), nullptr, x,
                 nblk, p->xq, xs);
    }
    MOE_LAUNCH(router_prefill_kernel, dim3((T + 63) / 64, (E + 63) / 64), 256, 0, st,
               mx ? nullptr : t0(kPfRouting), nullptr, x, T, H, E, wrt, bias, p->logits);
    const TopkArgs ta{E, k, f.renormalize, p->logits, ids, gates, nullptr, nullptr};
    const int nk = (E + 63) / 64, tb = (T + 15) / 16;
    if (nk <= 1) topk_prefill_kernel<1><<<tb, 1024, 0, st>>>(ta, T);
    else if (nk <= 2) topk_prefill_kernel<2><<<tb, 1024, 0, st>>>(ta, T);
    else if (nk <= 4) topk_prefill_kernel<4><<<tb, 1024, 0, st>>>(ta, T);
    else if (nk <= 8) topk_prefill_kernel<8><<<tb, 1024, 0, st>>>(ta, T);
    else topk_prefill_kernel<16><<<tb, 1024, 0, st>>>(ta, T);
    dispatch_count_kernel<<<nchunk, 256, 0, st>>>(ids, T, k, E, p->chunk_cnt);
    MOE_LAUNCH(dispatch_place_kernel, nchunk, 1024, 0, st, nullptr, t1(kPfRouting), ids, T, k, E,
               f.has_shared, nchunk, p->chunk_cnt, counts, offsets, sorted, inv, p->tok, p->tiles,
               p->n_tiles);
    if ((e = hipGetLastError()) != hipSuccess) return e;

    GroupArgs ga{p->tiles, p->n_tiles, counts, offsets, p->tok, c->d_layerbuf[b],
                 c->stride, f.has_shared ? c->d_shared + (size_t)l * c->stride : nullptr, E};
    const int nbn_gu = (2 * I + 511) / 512, nbn_dn = (H + 511) / 512;
    const size_t hhi_bytes = (size_t)p->Tmax * (k + 1) * I * 2;
    const size_t hlo_bytes = prefill_lo_bytes(p->Tmax, k, E, I);
    if (f.weight_format != MOE_WEIGHTS_MXFP4) {
      // bf16 or NVFP4 experts: grouped GEMMs over the same tiles, h between
      // them as two bf16 planes (hi, then lo lo_plane elements on)
      const size_t lo_plane = (size_t)p->Tmax * (k + 1) * I;
      const uint32_t lo_bytes = (uint32_t)(lo_plane * 2);
      if (f.weight_format == MOE_WEIGHTS_BF16) {
        const int nbn_g = 2 * I / (kBwAtoms * kAtomRows), nbn_d = H / (kBwdAtoms * kAtomRows);
        MOE_LAUNCH(gateup_prefill_bw_kernel, p->max_tiles * nbn_g, 64 * kGemmWaves, 0, st,
                   t0(kPfGateUp), t1(kPfGateUp), ga, x, (uint32_t)T * H * 2, H, I, nbn_g, p->h,
                   lo_plane);
        MOE_LAUNCH(down_prefill_bw_kernel, p->max_tiles * nbn_d, 64 * kGemmWaves, 0, st,
                   t0(kPfDown), t1(kPfDown), ga, p->h, 2 * lo_bytes, lo_bytes, H, I, nbn_d,
                   gateup_section_bytes(H, I, MOE_WEIGHTS_BF16), p->yperm);
      } else {
        const int nbn_d = H / (kNvdAtoms * kAtomRows);
        MOE_LAUNCH(gateup_prefill_nv_kernel, p->max_tiles * nbn_gu, 64 * kGemmWaves, 0, st,
                   t0(kPfGateUp), t1(kPfGateUp), ga, x, (uint32_t)T * H * 2, H, I, nbn_gu,
                   nv_trailer_offset(H, I), p->h, lo_plane);
        MOE_LAUNCH(down_prefill_nv_kernel, p->max_tiles * nbn_d, 64 * kGemmWaves, 0, st,
                   t0(kPfDown), t1(kPfDown), ga, p->h, 2 * lo_bytes, lo_bytes, H, I, nbn_d,
                   gateup_section_bytes(H, I, MOE_WEIGHTS_NVFP4), nv_trailer_offset(H, I),
                   p->yperm);
      }
    } else if (mx) {
      const size_t rows_cap = (size_t)p->Tmax * (k + 1);
      uint8_t* const hq = reinterpret_cast<uint8_t*>(p->h);
      uint8_t* const hs = hq + rows_cap * I;
      MOE_LAUNCH(gateup_mx_kernel, p->max_tiles * nbn_gu, 64 * kGemmWaves, 0, st, t0(kPfGateUp),
                 t1(kPfGateUp), ga, p->xq, (uint32_t)T * H, xs, (uint32_t)(T * (H / 32)), H, I,
                 nbn_gu, hq, hs);
      // one workgroup per CU, each running its items in turn; both bounds are
      // multiples of 8, so each workgroup's items stay on its XCD and come
      // in ascending tile order (its loop ends at the first one past n_tiles)
      MOE_LAUNCH(down_mx_kernel, std::min(p->max_tiles * nbn_dn, p->resident_wgs),
                 64 * kGemmWaves, 0, st, t0(kPfDown),
                 t1(kPfDown), ga, hq, (uint32_t)(rows_cap * I), hs, (uint32_t)(rows_cap * (I / 32)),
                 H, I, nbn_dn, gateup_section_bytes(H, I), p->yperm);
    } else {
      MOE_LAUNCH(gateup_prefill_kernel, p->max_tiles * nbn_gu, 64 * kGemmWaves, 0, st,
                 t0(kPfGateUp), t1(kPfGateUp), ga, x, (uint32_t)T * H * 2, H, I, nbn_gu, p->h,
                 p->hlo);
      MOE_LAUNCH(down_prefill_kernel, p->max_tiles * nbn_dn, 64 * kGemmWaves, 0, st, t0(kPfDown),
                 t1(kPfDown), ga, p->h, (uint32_t)hhi_bytes, p->hlo, (uint32_t)hlo_bytes, H, I,
                 nbn_dn, gateup_section_bytes(H, I), p->yperm);
    }
    if ((e = launch_combine_rows(p->yperm, inv, gates, T, k, H, f.has_shared,
                                 (uint16_t*)ys[l], y32s ? y32s[l] : nullptr, st, t0(kPfCombine),
                                 t1(kPfCombine))) != hipSuccess)
      return e;
    if (timed) c->t_prefill.push_back(tr);
    if ((e = hipEventRecord(c->ev_compute[b], st)) != hipSuccess) return e;
    if (debug_sync) {
      // MOE_DEBUG_SYNC: the layer's work and the next upload have finished
      if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
      if ((e = hipStreamSynchronize(c->copy_stream)) != hipSuccess) return e;
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  return hipGetLastError();
}

}  // namespace moe
