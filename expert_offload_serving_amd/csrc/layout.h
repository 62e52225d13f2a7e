// Expert record layouts of libmoe (host and device): sizes and offsets.
// Plain C++ (no HIP), so that the host repack can be built and checked on
// its own.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// MXFP4 expert record in the library's tiled layout.
//
// A matrix W [N rows][K] (rows = output features) is cut into atoms of
// 16 rows x 128 K (four MX blocks per row).  One atom is 1088 contiguous
// bytes, one lane of a wave per MX block:
//   bytes [16 l, 16 l + 16), l = 0..63: the 32 E2M1 codes (low nibble
//     first) of row (l % 16), block (l / 16) of the chunk, i.e. K range
//     [32 (l / 16), +32);
//   byte 1024 + l: that block's E8M0 scale.
// A wave loads an atom with one 16-byte and one 1-byte load per lane.  Word
// j of a lane's 16 bytes feeds MFMA step j of v_mfma_f32_16x16x32_bf16 as the
// B operand (hardware k = 8 (l / 16) + i stands for K = 32 (l / 16) + 8 j + i;
// the A operand uses the same correspondence, so the sum over K is exact).
// Gate and up are fused: row groups alternate 16 gate rows, 16 up rows
// (group 2p = gate rows 16p..16p+15, 2p+1 = up rows of the same indices).
// Record = [gate/up atoms: group-major, K-chunk minor] [down atoms: same].
// Total = 3*H*I*17/32 bytes, the MXFP4 size.
// ---------------------------------------------------------------------------
constexpr int kAtomRows = 16;
constexpr int kAtomK = 128;
constexpr int kAtomData = 1024;
constexpr int kAtomBytes = 1088;

// bf16 atom: the same 16 rows x 128 K tile as an MXFP4 atom, lane l's 32
// values (row l % 16, K block l / 16) as 4 pieces of 8 at 1024 p + 16 l.
constexpr int kAtomBytesBF16 = 4096;
// NVFP4 atom: the MXFP4 atom's 1024 code bytes, then lane l's two E4M3 block
// scales (row l % 16, K 32 (l / 16) .. +15 and +16 .. +31) at 1024 + 2 l.
// An NVFP4 record ends with a 16-byte trailer: the fp32 scales of the gate,
// up and down matrices, then 4 zero bytes.
constexpr int kAtomBytesNV = 1152;
constexpr int kNvTrailerBytes = 16;
inline size_t gateup_section_bytes(int H, int I, int fmt = MOE_WEIGHTS_MXFP4) {
  if (fmt == MOE_WEIGHTS_BF16) return (size_t)2 * I * H * 2;
  if (fmt == MOE_WEIGHTS_NVFP4) return (size_t)2 * I * H * 9 / 16;
  return (size_t)2 * I * H * 17 / 32;
}
// offset of an NVFP4 record's matrix scales: after the gate/up and down atoms
inline size_t nv_trailer_offset(int H, int I) { return (size_t)3 * H * I * 9 / 16; }
inline size_t expert_record_bytes(int H, int I, int fmt = MOE_WEIGHTS_MXFP4) {
  if (fmt == MOE_WEIGHTS_BF16) return (size_t)3 * H * I * 2;
  if (fmt == MOE_WEIGHTS_NVFP4) return nv_trailer_offset(H, I) + kNvTrailerBytes;
  return (size_t)3 * H * I * 17 / 32;
}

}  // namespace moe
