// Runs the library's host-side expert repack (expert_offload_serving_amd/
// csrc/repack.h) on its own: reads one expert's canonical matrices from
// files, writes the record.  Built with the address and undefined-behaviour
// sanitizers by tests/test_repack.py; every input buffer has exactly the
// size the format defines, so a read past one is reported.
//
// usage: repack_check <format 0|1|2> <H> <I> <dir>
//   dir holds qg.bin qu.bin qd.bin (codes, or bf16 patterns) and, for
//   MXFP4/NVFP4, sg.bin su.bin sd.bin; rec.bin is written there.
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../expert_offload_serving_amd/csrc/repack.h"

static std::vector<uint8_t> read_exact(const std::string& path, size_t n) {
  std::vector<uint8_t> v(n);
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f || std::fread(v.data(), 1, n, f) != n) {
    std::fprintf(stderr, "cannot read %zu bytes from %s\n", n, path.c_str());
    std::exit(2);
  }
  std::fclose(f);
  return v;
}

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  const int fmt = std::atoi(argv[1]), H = std::atoi(argv[2]), I = std::atoi(argv[3]);
  const std::string dir = argv[4];
  const size_t HI = (size_t)H * I;
  size_t qb, sb;  // bytes of one matrix's codes and scales
  if (fmt == MOE_WEIGHTS_BF16) {
    qb = HI * 2;
    sb = 0;
  } else if (fmt == MOE_WEIGHTS_NVFP4) {
    qb = HI / 2;
    sb = HI / 16 + 4;  // E4M3 per 16, then the fp32 matrix scale
  } else {
    qb = HI / 2;
    sb = HI / 32;
  }
  std::vector<uint8_t> qg = read_exact(dir + "/qg.bin", qb), qu = read_exact(dir + "/qu.bin", qb),
                       qd = read_exact(dir + "/qd.bin", qb);
  std::vector<uint8_t> sg, su, sd;
  if (sb) {
    sg = read_exact(dir + "/sg.bin", sb);
    su = read_exact(dir + "/su.bin", sb);
    sd = read_exact(dir + "/sd.bin", sb);
  }
  std::vector<uint8_t> rec(moe::expert_record_bytes(H, I, fmt), 0xAB);
  moe::repack_record(fmt, H, I, qg.data(), qu.data(), qd.data(), sb ? sg.data() : nullptr,
                     sb ? su.data() : nullptr, sb ? sd.data() : nullptr, rec.data());
  FILE* f = std::fopen((dir + "/rec.bin").c_str(), "wb");
  if (!f || std::fwrite(rec.data(), 1, rec.size(), f) != rec.size()) return 3;
  std::fclose(f);
  return 0;
}
