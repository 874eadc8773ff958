// Runs the cross-entropy backward epilogue (EpiCEGrad of epilogues.hpp) on the
// host (emulated) over every 256 x 256 tile of an M x N logit matrix:
//   ce_grad_driver M N dir   reads dir/logits.bin (fp32 [M x N]) and dir/stats.bin
//   (16-byte records [M]); writes dir/dl.bin (bf16 [M x N], pre-filled with 0xFFFF).
#include "epilogues.hpp"

#include <cstdio>
#include <string>

static char g_lds[4][32768];
static const float* g_logits;

static void tile_kernel(mshard::EpiCEGrad epi, int M, int N) {
  using namespace mshard;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave / kWavesN, wn = wave % kWavesN;
  const int tm = blockIdx.x, tn = blockIdx.y, m0 = tm * kBM, n0 = tn * kBN;
  AccTile acc;
  for (int mi = 0; mi < kSubM; ++mi)
    for (int ni = 0; ni < kSubN; ++ni)
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * kWaveM + mi * 16 + (lane & 15), col = n0 + wn * kWaveN + ni * 16 + 4 * (lane >> 4) + r;
        acc[mi][ni][r] = (row < M && col < N) ? g_logits[(int64_t)row * N + col] : 0.f;  // as the GEMM leaves them
      }
  const EpiCtx ctx{m0, n0, tm, tn, 0, wm, wn, lane, g_lds[0], g_lds[1], g_lds[2], g_lds[3], g_lds[0]};
  epi(acc, ctx);
}

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  const int M = std::atoi(argv[1]), N = std::atoi(argv[2]);
  const std::string dir = argv[3];
  std::vector<float> logits((size_t)M * N);
  std::vector<mshard::f32x4_t> stats(M);
  FILE* f = std::fopen((dir + "/logits.bin").c_str(), "rb");
  if (!f || std::fread(logits.data(), 4, logits.size(), f) != logits.size()) return 3;
  std::fclose(f);
  f = std::fopen((dir + "/stats.bin").c_str(), "rb");
  if (!f || std::fread(stats.data(), 16, stats.size(), f) != stats.size()) return 3;
  std::fclose(f);
  std::vector<uint16_t> dl((size_t)M * N, 0xffff);
  g_logits = logits.data();
  const mshard::EpiCEGrad epi{stats.data(), dl.data(), N, M, N};
  emu::launch(dim3((M + 255) / 256, (N + 255) / 256, 1), dim3(mshard::kThreads), tile_kernel, epi, M, N);
  f = std::fopen((dir + "/dl.bin").c_str(), "wb");
  std::fwrite(dl.data(), 2, dl.size(), f);
  std::fclose(f);
  return 0;
}
