// Runs the library's launch sequences (kernels.hip, attention.hip) on the host,
// with the kernel sources prepared by prep.py and the HIP subset of
// hip/hip_runtime.h.  Every buffer is a file of raw little-endian values in the
// case directory; outputs and the workspace start filled with 0xff bytes (NaN
// in bf16 and fp32), so an element a kernel fails to write shows up.  With
// EMU_WRITE_DL set, ce_bwd also writes the logit gradient from its workspace.
//   lib_driver mlp_fwd  T h f gelu bias dir : X A [b1] B              -> H Y Z
//   lib_driver mlp_bwd  T h f gelu bias dir : X A B H Y dZ            -> dX dA dB [db1]
//   lib_driver ce_fwd   T h v vstart dir    : X E target              -> m s z
//   lib_driver ce_bwd   T h v vstart t scale dloss dir : X E target m s [dloss] -> dX dE
//   lib_driver combine  t T dir             : m s z                   -> loss mean
//   lib_driver combine_nomean t T dir       : m s z                   -> loss_only (no mean asked)
//   lib_driver attn_fwd b s h n d causal dir: X Wqkv Wo               -> QKV O lse Z
//   lib_driver attn_bwd b s h n d causal dir: X Wqkv Wo QKV O lse dZ  -> dX dWqkv dWo
//   lib_driver attn_core b s n d causal dir : qkv dout                -> o lse dqkv (the core alone)
//   lib_driver fingerprint bytes chunk dir  : buf                     -> fp (1 + chunks words)
//   lib_driver plan     T h f v b s n d dir : prints the backward launch plans of these shapes
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "launch.hpp"

namespace mshard {
void record_armed_event(int, bool, hipStream_t) {}
}  // namespace mshard

static std::string g_dir;

static std::vector<char> rd(const char* name, size_t bytes) {
  std::vector<char> v(bytes ? bytes : 1);
  const std::string p = g_dir + "/" + name + ".bin";
  FILE* f = std::fopen(p.c_str(), "rb");
  if (!f || std::fread(v.data(), 1, bytes, f) != bytes) {
    std::fprintf(stderr, "read %s (%zu bytes)\n", p.c_str(), bytes);
    std::exit(2);
  }
  std::fclose(f);
  return v;
}
static std::vector<char> out(size_t bytes) { return std::vector<char>(bytes ? bytes : 1, (char)0xff); }
static void wr(const char* name, const std::vector<char>& v, size_t bytes) {
  const std::string p = g_dir + "/" + name + ".bin";
  FILE* f = std::fopen(p.c_str(), "wb");
  std::fwrite(v.data(), 1, bytes, f);
  std::fclose(f);
}
template <class T>
static T* P(std::vector<char>& v) { return (T*)v.data(); }
template <class T>
static const T* C(const std::vector<char>& v) { return (const T*)v.data(); }
static void ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s returned %d\n", what, (int)e);
    std::exit(3);
  }
}

int main(int argc, char** argv) {
  if (argc < 3) return 2;
  const std::string op = argv[1];
  g_dir = argv[argc - 1];
  auto I = [&](int i) { return (int64_t)std::atoll(argv[2 + i]); };
  if (op == "mlp_fwd") {
    const int64_t T = I(0), h = I(1), f = I(2), gelu = I(3), bias = I(4);
    auto X = rd("X", T * h * 2), A = rd("A", h * f * 2), B = rd("B", f * h * 2);
    std::vector<char> b1 = bias ? rd("b1", f * 2) : std::vector<char>();
    auto H = out(T * f * 2), Y = out(T * f * 2), Z = out(T * h * 4);
    auto ws = out(mshard::mlp_workspace_layout(T, h, f).bytes);
    ok(mshard::launch_mlp_fwd(C<uint16_t>(X), C<uint16_t>(A), bias ? C<uint16_t>(b1) : nullptr, C<uint16_t>(B), T, h,
                              f, (int)gelu, P<uint16_t>(H), P<uint16_t>(Y), P<float>(Z), ws.data(), nullptr),
       "launch_mlp_fwd");
    wr("H", H, T * f * 2), wr("Y", Y, T * f * 2), wr("Z", Z, T * h * 4);
  } else if (op == "mlp_bwd") {
    const int64_t T = I(0), h = I(1), f = I(2), gelu = I(3), bias = I(4);
    auto X = rd("X", T * h * 2), A = rd("A", h * f * 2), B = rd("B", f * h * 2);
    auto H = rd("H", T * f * 2), Y = rd("Y", T * f * 2), dZ = rd("dZ", T * h * 2);
    auto dX = out(T * h * 4), dA = out(h * f * 2), dB = out(f * h * 2), db1 = out(f * 2);
    auto ws = out(mshard::mlp_workspace_layout(T, h, f).bytes);
    ok(mshard::launch_mlp_bwd(C<uint16_t>(X), C<uint16_t>(A), C<uint16_t>(B), C<uint16_t>(H), C<uint16_t>(Y),
                              C<uint16_t>(dZ), T, h, f, (int)gelu, P<float>(dX), P<uint16_t>(dA), P<uint16_t>(dB),
                              bias ? P<uint16_t>(db1) : nullptr, ws.data(), nullptr),
       "launch_mlp_bwd");
    wr("dX", dX, T * h * 4), wr("dA", dA, h * f * 2), wr("dB", dB, f * h * 2);
    if (bias) wr("db1", db1, f * 2);
  } else if (op == "ce_fwd") {
    const int64_t T = I(0), h = I(1), v = I(2), vstart = I(3);
    auto X = rd("X", T * h * 2), E = rd("E", h * v * 2), tg = rd("target", T * 8);
    auto m = out(T * 4), s = out(T * 4), z = out(T * 4);
    auto ws = out(mshard::ce_workspace_layout(T, v).bytes);
    ok(mshard::launch_vocab_ce(C<uint16_t>(X), C<uint16_t>(E), C<int64_t>(tg), T, h, v, vstart, P<float>(m),
                               P<float>(s), P<float>(z), ws.data(), nullptr),
       "launch_vocab_ce");
    wr("m", m, T * 4), wr("s", s, T * 4), wr("z", z, T * 4);
  } else if (op == "ce_bwd") {
    const int64_t T = I(0), h = I(1), v = I(2), vstart = I(3), t = I(4), has_dloss = I(6);
    const float scale = (float)std::atof(argv[2 + 5]);
    auto X = rd("X", T * h * 2), E = rd("E", h * v * 2), tg = rd("target", T * 8);
    auto m = rd("m", t * T * 4), s = rd("s", t * T * 4);
    std::vector<char> dl = has_dloss ? rd("dloss", T * 4) : std::vector<char>();
    auto dX = out(T * h * 4), dE = out(h * v * 2);
    auto ws = out(mshard::ce_bwd_workspace_layout(T, h, v).bytes);
    ok(mshard::launch_vocab_ce_bwd(C<uint16_t>(X), C<uint16_t>(E), C<int64_t>(tg), C<float>(m), C<float>(s), (int)t,
                                   has_dloss ? C<float>(dl) : nullptr, scale, T, h, v, vstart, P<float>(dX),
                                   P<uint16_t>(dE), ws.data(), nullptr),
       "launch_vocab_ce_bwd");
    wr("dX", dX, T * h * 4), wr("dE", dE, h * v * 2);
    if (std::getenv("EMU_WRITE_DL")) {  // the logit gradient, from the workspace
      std::vector<char> dL(ws.begin() + mshard::ce_bwd_workspace_layout(T, h, v).off_dL,
                           ws.begin() + mshard::ce_bwd_workspace_layout(T, h, v).off_dL + T * v * 2);
      wr("dL", dL, T * v * 2);
    }
  } else if (op == "combine" || op == "combine_nomean") {
    const int64_t t = I(0), T = I(1);
    const bool mean_too = op == "combine";
    auto m = rd("m", t * T * 4), s = rd("s", t * T * 4), z = rd("z", t * T * 4);
    auto loss = out(T * 4), mean = out(4);
    ok(mshard::launch_ce_combine(C<float>(m), C<float>(s), C<float>(z), (int)t, T, P<float>(loss),
                                 mean_too ? P<float>(mean) : nullptr, nullptr),
       "launch_ce_combine");
    wr(mean_too ? "loss" : "loss_only", loss, T * 4);
    if (mean_too) wr("mean", mean, 4);
  } else if (op == "attn_fwd" || op == "attn_bwd") {
    const int64_t b = I(0), s = I(1), h = I(2), n = I(3), d = I(4), causal = I(5);
    const int64_t T = b * s, nd = n * d;
    auto X = rd("X", T * h * 2), Wqkv = rd("Wqkv", h * 3 * nd * 2), Wo = rd("Wo", nd * h * 2);
    if (op == "attn_fwd") {
      auto QKV = out(T * 3 * nd * 2), O = out(T * nd * 2), lse = out(n * T * 4), Z = out(T * h * 4);
      ok(mshard::launch_attn_fwd(C<uint16_t>(X), C<uint16_t>(Wqkv), C<uint16_t>(Wo), b, s, h, n, d, causal != 0,
                                 P<uint16_t>(QKV), P<uint16_t>(O), P<float>(lse), P<float>(Z), nullptr),
         "launch_attn_fwd");
      wr("QKV", QKV, T * 3 * nd * 2), wr("O", O, T * nd * 2), wr("lse", lse, n * T * 4), wr("Z", Z, T * h * 4);
    } else {
      auto QKV = rd("QKV", T * 3 * nd * 2), O = rd("O", T * nd * 2), lse = rd("lse", n * T * 4),
           dZ = rd("dZ", T * h * 2);
      auto dX = out(T * h * 4), dWqkv = out(h * 3 * nd * 2), dWo = out(nd * h * 2);
      auto ws = out(mshard::attn_workspace_layout(b, s, h, n, d).bytes);
      ok(mshard::launch_attn_bwd(C<uint16_t>(X), C<uint16_t>(Wqkv), C<uint16_t>(Wo), C<uint16_t>(QKV),
                                 C<uint16_t>(O), C<float>(lse), C<uint16_t>(dZ), b, s, h, n, d, causal != 0,
                                 P<float>(dX), P<uint16_t>(dWqkv), P<uint16_t>(dWo), ws.data(), nullptr),
         "launch_attn_bwd");
      wr("dX", dX, T * h * 4), wr("dWqkv", dWqkv, h * 3 * nd * 2), wr("dWo", dWo, nd * h * 2);
    }
  } else if (op == "attn_core") {
    const int64_t b = I(0), s = I(1), n = I(2), d = I(3), causal = I(4);
    const int64_t T = b * s, nd = n * d;
    auto qkv = rd("qkv", T * 3 * nd * 2), dout = rd("dout", T * nd * 2);
    auto o = out(T * nd * 2), lse = out(n * T * 4), delta = out(n * T * 4), dqkv = out(T * 3 * nd * 2);
    mshard::AttnGeom g{(int)b, (int)s, (int)n, (int)d, (int)(3 * nd), (int)nd,
                       (float)(1.4426950408889634 / std::sqrt((double)d))};
    ok(mshard::launch_attn_core_fwd(g, causal != 0, C<uint16_t>(qkv), P<uint16_t>(o), P<float>(lse), nullptr),
       "launch_attn_core_fwd");
    ok(mshard::launch_attn_core_bwd(g, causal != 0, C<uint16_t>(qkv), C<uint16_t>(o), C<uint16_t>(dout), C<float>(lse),
                                    P<float>(delta), P<uint16_t>(dqkv), nullptr),
       "launch_attn_core_bwd");
    wr("o", o, T * nd * 2), wr("lse", lse, n * T * 4), wr("dqkv", dqkv, T * 3 * nd * 2);
  } else if (op == "fingerprint") {
    const int64_t bytes = I(0), chunk = I(1);
    const uint64_t words = 1 + mshard::fingerprint_chunk_count(bytes, chunk);
    auto buf = rd("buf", bytes), fp = out(words * 8);
    ok(mshard::launch_fingerprint(buf.data(), bytes, chunk, P<uint64_t>(fp), nullptr), "launch_fingerprint");
    wr("fp", fp, words * 8);
  } else if (op == "plan") {
    const int64_t T = I(0), h = I(1), f = I(2), v = I(3), b = I(4), s = I(5), n = I(6), d = I(7);
    const mshard::MlpWorkspace mw = mshard::mlp_workspace_layout(T, h, f);
    const mshard::CeBwdWorkspace cw = mshard::ce_bwd_workspace_layout(T, h, v);
    const mshard::AttnWorkspace aw = mshard::attn_workspace_layout(b, s, h, n, d);
    std::printf("mlp splits_dB=%d splits_dA=%d pair_bh=%d pair_ax=%d dh_first=%d dx_first=%d db1_parts=%d "
                "fwd_tail_n=%d fwd_tail_splits=%d z_tail_n=%d z_tail_splits=%d\n",
                mw.plan.splits_dB, mw.plan.splits_dA, (int)mw.plan.pair_bh, (int)mw.plan.pair_ax,
                (int)mw.plan.dh_first, (int)mw.plan.dx_first, mw.db1_parts, mw.fwd.tail_n, mw.fwd.tail_splits,
                mw.fwd.z_tail_n, mw.fwd.z_tail_splits);
    std::printf("ce_bwd splits_dE=%d paired=%d dx_first=%d\n", cw.splits_dE, (int)cw.paired, (int)cw.dx_first);
    std::printf("attn splits_wo=%d splits_wqkv=%d pair_o=%d o_first=%d pair_x=%d x_first=%d\n", aw.splits_wo,
                aw.splits_wqkv, (int)aw.pair_o, (int)aw.o_first, (int)aw.pair_x, (int)aw.x_first);
  } else {
    return 2;
  }
  return 0;
}
