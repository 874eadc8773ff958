// Runs the attention core kernels of attention.hip on the host (emulated) for one shape:
//   attn_driver b s n d causal dir   reads dir/qkv.bin (bf16 [T x 3nd]) and dir/dout.bin (bf16 [T x nd]),
//   writes dir/o.bin (bf16 [T x nd]), dir/lse.bin (fp32 [n x T]), dir/dqkv.bin (bf16 [T x 3nd]).
#include "attention.hip"

#include <cstdio>
#include <string>

template <class T>
static std::vector<T> readf(const std::string& p, size_t n) {
  std::vector<T> v(n);
  FILE* f = std::fopen(p.c_str(), "rb");
  if (!f || std::fread(v.data(), sizeof(T), n, f) != n) { std::fprintf(stderr, "read %s\n", p.c_str()); std::exit(2); }
  std::fclose(f);
  return v;
}
template <class T>
static void writef(const std::string& p, const std::vector<T>& v) {
  FILE* f = std::fopen(p.c_str(), "wb");
  std::fwrite(v.data(), sizeof(T), v.size(), f);
  std::fclose(f);
}

int main(int argc, char** argv) {
  if (argc != 7) return 2;
  const int b = std::atoi(argv[1]), s = std::atoi(argv[2]), n = std::atoi(argv[3]), d = std::atoi(argv[4]);
  const bool causal = std::atoi(argv[5]) != 0;
  const std::string dir = argv[6];
  const size_t T = (size_t)b * s, nd = (size_t)n * d;
  auto qkv = readf<uint16_t>(dir + "/qkv.bin", T * 3 * nd);
  auto dout = readf<uint16_t>(dir + "/dout.bin", T * nd);
  std::vector<uint16_t> o(T * nd, 0xffff), dqkv(T * 3 * nd, 0xffff);
  std::vector<float> lse(n * T, NAN), delta(n * T, NAN);
  mshard::AttnGeom g;
  g.b = b; g.s = s; g.n = n; g.d = d; g.ld_qkv = (int)(3 * nd); g.ld_o = (int)nd;
  g.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  if (mshard::launch_attn_core_fwd(g, causal, qkv.data(), o.data(), lse.data(), nullptr) != hipSuccess) return 3;
  if (mshard::launch_attn_core_bwd(g, causal, qkv.data(), o.data(), dout.data(), lse.data(), delta.data(), dqkv.data(),
                                   nullptr) != hipSuccess)
    return 4;
  writef(dir + "/o.bin", o);
  writef(dir + "/lse.bin", lse);
  writef(dir + "/dqkv.bin", dqkv);
  return 0;
}
