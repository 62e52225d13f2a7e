// Host-side repack of canonical expert matrices into the library's record
// layouts (layout.h).  Plain C++ (no HIP): built into libmoe and, on its
// own, into a sanitizer-checked test program.
#pragma once

#include <algorithm>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "layout.h"

namespace moe {

// Run fn(i) for i in [0, n) on up to `threads` host threads.
template <class F>
inline void parallel_for(int n, int threads, F fn) {
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

inline int host_threads() {
  unsigned n = std::thread::hardware_concurrency();
  return (int)std::max(1u, std::min(n, 16u));
}

// --------------------------------------------------------------- repacking
// Canonical row r of a [N][K] MXFP4 matrix: codes q[r][K/2], scales s[r][K/32].
// Lane l of the atom takes row row0 + l % 16, MX block 4 c + l / 16.
inline void write_atom(const uint8_t* q, const uint8_t* s, int K, int row0, int c,
                       uint8_t* atom) {
  const int kc = K / 2, sc = K / 32;
  for (int l = 0; l < 64; l++) {
    const int r = row0 + (l % 16), blk = c * 4 + l / 16;
    std::memcpy(atom + l * 16, q + (size_t)r * kc + (size_t)blk * 16, 16);
    atom[kAtomData + l] = s[(size_t)r * sc + blk];
  }
}

inline void repack_gateup(const uint8_t* qg, const uint8_t* sg, const uint8_t* qu,
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

inline void repack_down(const uint8_t* qd, const uint8_t* sd, int H, int I, uint8_t* out) {
  const int KC = I / kAtomK, groups = H / kAtomRows;
  parallel_for(groups, (size_t)I * H > (1 << 22) ? host_threads() : 1, [&](int rg) {
    for (int c = 0; c < KC; c++)
      write_atom(qd, sd, I, rg * kAtomRows, c, out + ((size_t)rg * KC + c) * kAtomBytes);
  });
}

// bf16 [N][K] matrix: lane l of the atom takes row row0 + l % 16, values
// K = 32 (4 c + l / 16) .. +31, as 4 pieces of 8 at 1024 p + 16 l (piece p is
// what the lane feeds the MFMA at K step p).
inline void write_atom_bf16(const uint16_t* w, int K, int row0, int c, uint8_t* atom) {
  for (int l = 0; l < 64; l++) {
    const uint16_t* src = w + (size_t)(row0 + l % 16) * K + (size_t)(c * 4 + l / 16) * 32;
    for (int p = 0; p < 4; p++) std::memcpy(atom + 1024 * p + 16 * l, src + 8 * p, 16);
  }
}

inline void repack_gateup_bf16(const uint16_t* wg, const uint16_t* wu, int I, int H, uint8_t* out) {
  const int KC = H / kAtomK, groups = 2 * I / kAtomRows;
  parallel_for(groups, (size_t)I * H > (1 << 22) ? host_threads() : 1, [&](int rg) {
    for (int c = 0; c < KC; c++)
      write_atom_bf16((rg & 1) ? wu : wg, H, (rg / 2) * kAtomRows, c,
                      out + ((size_t)rg * KC + c) * kAtomBytesBF16);
  });
}

inline void repack_down_bf16(const uint16_t* wd, int H, int I, uint8_t* out) {
  const int KC = I / kAtomK, groups = H / kAtomRows;
  parallel_for(groups, (size_t)I * H > (1 << 22) ? host_threads() : 1, [&](int rg) {
    for (int c = 0; c < KC; c++)
      write_atom_bf16(wd, I, rg * kAtomRows, c, out + ((size_t)rg * KC + c) * kAtomBytesBF16);
  });
}

// NVFP4 [N][K] matrix: codes as MXFP4 (lane l: row row0 + l % 16, K block
// of 32 number 4 c + l / 16); its two E4M3 block scales of 16 from s[r][K/16]
// at 1024 + 2 l.
inline void write_atom_nv(const uint8_t* q, const uint8_t* s, int K, int row0, int c,
                          uint8_t* atom) {
  const int kc = K / 2, sc = K / 16;
  for (int l = 0; l < 64; l++) {
    const int r = row0 + (l % 16), blk = c * 4 + l / 16;
    std::memcpy(atom + l * 16, q + (size_t)r * kc + (size_t)blk * 16, 16);
    atom[kAtomData + 2 * l] = s[(size_t)r * sc + 2 * blk];
    atom[kAtomData + 2 * l + 1] = s[(size_t)r * sc + 2 * blk + 1];
  }
}

inline void repack_nv(const uint8_t* qg, const uint8_t* sg, const uint8_t* qu, const uint8_t* su,
                      const uint8_t* qd, const uint8_t* sd, int H, int I, uint8_t* rec) {
  const int KCg = H / kAtomK, KCd = I / kAtomK;
  const int threads = (size_t)I * H > (1 << 22) ? host_threads() : 1;
  parallel_for(2 * I / kAtomRows, threads, [&](int rg) {
    const bool up = rg & 1;
    for (int c = 0; c < KCg; c++)
      write_atom_nv(up ? qu : qg, up ? su : sg, H, (rg / 2) * kAtomRows, c,
                    rec + ((size_t)rg * KCg + c) * kAtomBytesNV);
  });
  uint8_t* down = rec + gateup_section_bytes(H, I, MOE_WEIGHTS_NVFP4);
  parallel_for(H / kAtomRows, threads, [&](int rg) {
    for (int c = 0; c < KCd; c++)
      write_atom_nv(qd, sd, I, rg * kAtomRows, c, down + ((size_t)rg * KCd + c) * kAtomBytesNV);
  });
  // matrix scales: each scale array ends with its matrix's fp32 scale
  const size_t ng = (size_t)I * H / 16;
  float t[4] = {0.f, 0.f, 0.f, 0.f};
  std::memcpy(&t[0], sg + ng, 4);
  std::memcpy(&t[1], su + ng, 4);
  std::memcpy(&t[2], sd + ng, 4);
  std::memcpy(rec + nv_trailer_offset(H, I), t, sizeof t);
}

// One expert of weight format `fmt` into `rec` (expert_record_bytes(H, I,
// fmt) bytes).  MXFP4 and NVFP4: codes qg, qu [I][H/2], qd [H][I/2] and
// scales sg, su [I][H/32 or H/16], sd [H][I/32 or I/16] (NVFP4 scale arrays
// end with the matrix's fp32 scale); bf16: qg, qu [I][H], qd [H][I] as
// 16-bit patterns, no scales.
inline void repack_record(int fmt, int H, int I, const uint8_t* qg, const uint8_t* qu,
                          const uint8_t* qd, const uint8_t* sg, const uint8_t* su,
                          const uint8_t* sd, uint8_t* rec) {
  if (fmt == MOE_WEIGHTS_NVFP4) {
    repack_nv(qg, sg, qu, su, qd, sd, H, I, rec);
  } else if (fmt == MOE_WEIGHTS_BF16) {
    repack_gateup_bf16(reinterpret_cast<const uint16_t*>(qg), reinterpret_cast<const uint16_t*>(qu),
                       I, H, rec);
    repack_down_bf16(reinterpret_cast<const uint16_t*>(qd), H, I,
                     rec + gateup_section_bytes(H, I, fmt));
  } else {
    repack_gateup(qg, sg, qu, su, I, H, rec);
    repack_down(qd, sd, H, I, rec + gateup_section_bytes(H, I, fmt));
  }
}

}  // namespace moe
