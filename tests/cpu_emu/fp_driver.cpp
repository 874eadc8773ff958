// Runs the fingerprint kernels of fingerprint.hip on the host (emulated):
//   fp_driver in.bin nbytes chunk out.bin   writes the 1 + chunks uint64 words.
#include "fingerprint.hip"

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  const uint64_t n = std::strtoull(argv[2], nullptr, 10), chunk = std::strtoull(argv[3], nullptr, 10);
  std::vector<uint64_t> buf(n / 8 + 1, 0);  // 8-byte aligned storage
  FILE* f = std::fopen(argv[1], "rb");
  if (!f || std::fread(buf.data(), 1, n, f) != n) return 3;
  std::fclose(f);
  std::vector<uint64_t> out(1 + mshard::fingerprint_chunk_count(n, chunk), 0);
  if (mshard::launch_fingerprint(buf.data(), n, chunk, out.data(), nullptr) != hipSuccess) return 4;
  FILE* g = std::fopen(argv[4], "wb");
  std::fwrite(out.data(), 8, out.size(), g);
  std::fclose(g);
  return 0;
}
