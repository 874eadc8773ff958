// kernels.hip - launchers for the MLP shard and CE shard, plus the small
// fixed-order reduction kernels (split-K slices, bias-gradient partials, CE
// tile partials, CE shard combine).  Every reduction adds its terms in an order
// fixed by the shapes alone, with one private slot per writer and no atomics,
// which is what makes repeated calls bitwise identical (Megatron Core
// bitwise-determinism news item, news.hamidun.com: fixed reduction order and
// private per-writer output space).
#include "launch.hpp"

#include "epilogues.hpp"

namespace mshard {

// ---------------------------------------------------------------------------
// Small kernels

// out[i] = bf16( sum_{s = 0..S-1} ws[s*stride + i] ), s ascending; 8 elements per thread.
__global__ void __launch_bounds__(256) splitk_reduce_bf16(const float* __restrict__ ws, int64_t stride, int S,
                                                          int64_t n, uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  float acc[8];
  const f32x4_t* p = (const f32x4_t*)(ws + i);
  f32x4_t a = p[0], b = p[1];
#pragma unroll
  for (int r = 0; r < 4; ++r) { acc[r] = a[r]; acc[4 + r] = b[r]; }
  for (int s = 1; s < S; ++s) {
    const f32x4_t* q = (const f32x4_t*)(ws + (int64_t)s * stride + i);
    a = q[0];
    b = q[1];
#pragma unroll
    for (int r = 0; r < 4; ++r) { acc[r] += a[r]; acc[4 + r] += b[r]; }
  }
  u32x4_t o{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
            pack_bf16x2(acc[6], acc[7])};
  *(u32x4_t*)(out + i) = o;
}

// db1[j] = bf16( sum_{p = 0..P-1} part[p*N + j] ), p ascending.
__global__ void __launch_bounds__(256) colsum_reduce_bf16(const float* __restrict__ part, int P, int N,
                                                          uint16_t* __restrict__ out) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= N) return;
  float acc = 0.f;
  for (int p = 0; p < P; ++p) acc += part[(int64_t)p * N + j];
  out[j] = __builtin_bit_cast(uint16_t, (__bf16)acc);
}

// Log-sum-exp merge of (m2, s2) into (M, S): afterwards S = sum exp(. - M) over
// both parts and M = the larger max.  Parts with s <= 0 are empty.
__device__ __forceinline__ void lse_merge(float& M, float& S, float m2, float s2) {
  if (!(s2 > 0.f)) return;
  if (!(S > 0.f)) {
    M = m2;
    S = s2;
  } else if (m2 > M) {
    S = S * expf(M - m2) + s2;
    M = m2;
  } else {
    S += s2 * expf(m2 - M);
  }
}

// Per token row: merge the P tile partials of the logits GEMM into the shard's
// (m, s, z).  A block covers 64 rows with 8 waves; wave w merges partials
// [w*P/8, (w+1)*P/8) in ascending order (one row per lane, coalesced over
// rows), then wave 0 merges the 8 wave results in ascending wave order.
__global__ void __launch_bounds__(512) ce_tile_combine(const float* __restrict__ pm, const float* __restrict__ ps,
                                                       const float* __restrict__ pz, int P, int T,
                                                       float* __restrict__ m, float* __restrict__ s,
                                                       float* __restrict__ z) {
  __shared__ float xm[8][64], xs[8][64], xz[8][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = blockIdx.x * 64 + lane;
  const int p0 = (int)(((int64_t)w * P) / 8), p1 = (int)(((int64_t)(w + 1) * P) / 8);
  float M = -INFINITY, S = 0.f, Z = 0.f;
  if (row < T) {
    for (int p = p0; p < p1; ++p) {
      const int64_t o = (int64_t)p * T + row;
      lse_merge(M, S, pm[o], ps[o]);
      Z += pz[o];
    }
  }
  xm[w][lane] = M;
  xs[w][lane] = S;
  xz[w][lane] = Z;
  __syncthreads();
  if (w == 0 && row < T) {
    for (int q = 1; q < 8; ++q) {
      lse_merge(M, S, xm[q][lane], xs[q][lane]);
      Z += xz[q][lane];
    }
    m[row] = M;
    s[row] = S;
    z[row] = Z;
  }
}

// Per token: merge t shards' partials in ascending rank order into the loss.
__global__ void __launch_bounds__(256) ce_combine_tokens(const float* __restrict__ m, const float* __restrict__ s,
                                                         const float* __restrict__ z, int t, int64_t T,
                                                         float* __restrict__ loss) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T) return;
  float M = -INFINITY, S = 0.f, Z = 0.f;
  for (int r = 0; r < t; ++r) {
    const int64_t o = (int64_t)r * T + i;
    lse_merge(M, S, m[o], s[o]);
    Z += z[o];
  }
  loss[i] = logf(S) + M - Z;
}

// Mean of loss[0..T): thread j sums j, j+1024, ... in order, then a fixed
// binary tree over the 1024 thread sums.  One workgroup.
__global__ void __launch_bounds__(1024) mean_fixed_tree(const float* __restrict__ x, int64_t T,
                                                        float* __restrict__ out) {
  __shared__ float red[1024];
  float acc = 0.f;
  for (int64_t i = threadIdx.x; i < T; i += 1024) acc += x[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0] / (float)T;
}

// ---------------------------------------------------------------------------
// GEMM launch helper

static GemmGeom make_geom(int64_t M, int64_t N, int64_t K, int splits) {
  GemmGeom g;
  g.M = (int)M;
  g.N = (int)N;
  g.K = (int)K;
  g.tiles_m = (int)((M + kBM - 1) / kBM);
  g.tiles_n = (int)((N + kBN - 1) / kBN);
  // every K split must own at least one k tile (the kernel always runs its first tile)
  const int64_t nk = (K + kBK - 1) / kBK;
  g.splits = (int)(splits < nk ? splits : nk);
  return g;
}

template <bool AK, bool BK, class Epi>
static hipError_t launch_gemm(int id, const GemmGeom& g, const Operand& a, const Operand& b, const Epi& epi,
                              hipStream_t stream) {
  const int blocks = g.tiles_m * g.tiles_n * g.splits;
  record_armed_event(id, false, stream);
  hipLaunchKernelGGL((gemm_kernel<AK, BK, Epi>), dim3(blocks), dim3(kThreads), 0, stream, g, a, b, epi);
  const hipError_t err = hipGetLastError();
  record_armed_event(id, true, stream);
  return err;
}

int weight_grad_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  const int64_t nk = (K + kBK - 1) / kBK;
  int S = 1;
  while (tiles * S < 256 && nk / (S * 2) >= 16 && S < 8) S *= 2;
  return S;
}

MlpWorkspace mlp_workspace_layout(int64_t T, int64_t h, int64_t f) {
  MlpWorkspace w;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t tiles_m = (T + kBM - 1) / kBM;
  const int Sb = weight_grad_splits(f, h, T);
  const int Sa = weight_grad_splits(h, f, T);
  w.splits_dB = Sb;
  w.splits_dA = Sa;
  w.off_dH = 0;
  w.off_db1 = align((size_t)T * f * 2);
  w.db1_parts = (int)(tiles_m * 2);
  w.off_splitk = w.off_db1 + align((size_t)w.db1_parts * f * 4);
  const int S = Sb > Sa ? Sb : Sa;
  w.bytes = w.off_splitk + (S > 1 ? align((size_t)S * h * f * 4) : 0);
  return w;
}

CeWorkspace ce_workspace_layout(int64_t T, int64_t v) {
  CeWorkspace w;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  w.parts = (int)((v + kBN - 1) / kBN);
  const size_t one = align((size_t)w.parts * T * 4);
  w.off_m = 0;
  w.off_s = one;
  w.off_z = 2 * one;
  w.bytes = 3 * one;
  return w;
}

// ---------------------------------------------------------------------------
// Entry-point launch sequences (arguments already validated by the ABI layer)

template <int FORM>
static hipError_t mlp_fwd_impl(const uint16_t* X, const uint16_t* A, const uint16_t* b1, const uint16_t* B,
                               int64_t T, int64_t h, int64_t f, uint16_t* H, uint16_t* Y, float* Z,
                               hipStream_t st) {
  // H = X A (+ b1), Y = GeLU(H):  NN, M = T, N = f, K = h
  {
    GemmGeom g = make_geom(T, f, h, 1);
    Operand a{X, h, T * h}, b{A, f, h * f};
    EpiGeluFwd<FORM> e{H, Y, b1, f, (int)T, (int)f};
    hipError_t err = launch_gemm<true, false>(kTkFwdH, g, a, b, e, st);
    if (err != hipSuccess) return err;
  }
  // Z = Y B:  NN, M = T, N = h, K = f
  {
    GemmGeom g = make_geom(T, h, f, 1);
    Operand a{Y, f, T * f}, b{B, h, f * h};
    EpiStoreF32 e{Z, h, (int)T, (int)h, 0};
    return launch_gemm<true, false>(kTkFwdZ, g, a, b, e, st);
  }
}

hipError_t launch_mlp_fwd(const uint16_t* X, const uint16_t* A, const uint16_t* b1, const uint16_t* B,
                          int64_t T, int64_t h, int64_t f, int gelu, uint16_t* H, uint16_t* Y, float* Z,
                          hipStream_t st) {
  return gelu == kGeluErf ? mlp_fwd_impl<kGeluErf>(X, A, b1, B, T, h, f, H, Y, Z, st)
                          : mlp_fwd_impl<kGeluTanh>(X, A, b1, B, T, h, f, H, Y, Z, st);
}

// Weight gradient C[M x N] = sum_t P[t, m] Q[t, n] (TN), bf16 result, with an
// optional deterministic K split through fp32 workspace slices.
static hipError_t weight_grad(int id, const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq, int64_t Kt,
                              int64_t M, int64_t N, int S, uint16_t* C, float* splitk, hipStream_t st) {
  GemmGeom g = make_geom(M, N, Kt, S);
  S = g.splits;
  Operand a{P, ldp, Kt * ldp}, b{Q, ldq, Kt * ldq};
  if (S == 1) {
    EpiStoreBF16 e{C, N, (int)M, (int)N};
    return launch_gemm<false, false>(id, g, a, b, e, st);
  }
  EpiStoreF32 e{splitk, N, (int)M, (int)N, M * N};
  hipError_t err = launch_gemm<false, false>(id, g, a, b, e, st);
  if (err != hipSuccess) return err;
  const int64_t n = M * N;  // multiple of 8
  const int64_t blocks = (n / 8 + 255) / 256;
  hipLaunchKernelGGL(splitk_reduce_bf16, dim3((unsigned)blocks), dim3(256), 0, st, splitk, M * N, S, n, C);
  return hipGetLastError();
}

template <int FORM>
static hipError_t mlp_bwd_impl(const uint16_t* X, const uint16_t* A, const uint16_t* B, const uint16_t* H,
                               const uint16_t* Y, const uint16_t* dZ, int64_t T, int64_t h, int64_t f,
                               float* dX, uint16_t* dA, uint16_t* dB, uint16_t* db1, char* ws, hipStream_t st) {
  const MlpWorkspace w = mlp_workspace_layout(T, h, f);
  uint16_t* dH = (uint16_t*)(ws + w.off_dH);
  float* db1_part = db1 ? (float*)(ws + w.off_db1) : nullptr;
  float* splitk = (float*)(ws + w.off_splitk);
  hipError_t err;
  // dH = (dZ B^T) * GeLU'(H):  NT, M = T, N = f, K = h; B stored [f x h] = [N x K]
  {
    GemmGeom g = make_geom(T, f, h, 1);
    Operand a{dZ, h, T * h}, b{B, h, f * h};
    EpiDGelu<FORM> e{H, dH, db1_part, f, (int)T, (int)f};
    err = launch_gemm<true, true>(kTkBwdDH, g, a, b, e, st);
    if (err != hipSuccess) return err;
  }
  // dB = Y^T dZ:  [f x h], contraction over tokens
  err = weight_grad(kTkBwdDB, Y, f, dZ, h, T, f, h, w.splits_dB, dB, splitk, st);
  if (err != hipSuccess) return err;
  // dA = X^T dH:  [h x f]
  err = weight_grad(kTkBwdDA, X, h, dH, f, T, h, f, w.splits_dA, dA, splitk, st);
  if (err != hipSuccess) return err;
  // dX = dH A^T:  NT, M = T, N = h, K = f; A stored [h x f] = [N x K]
  {
    GemmGeom g = make_geom(T, h, f, 1);
    Operand a{dH, f, T * f}, b{A, f, h * f};
    EpiStoreF32 e{dX, h, (int)T, (int)h, 0};
    err = launch_gemm<true, true>(kTkBwdDX, g, a, b, e, st);
    if (err != hipSuccess) return err;
  }
  if (db1) {
    hipLaunchKernelGGL(colsum_reduce_bf16, dim3((unsigned)((f + 255) / 256)), dim3(256), 0, st, db1_part,
                       w.db1_parts, (int)f, db1);
    err = hipGetLastError();
  }
  return err;
}

hipError_t launch_mlp_bwd(const uint16_t* X, const uint16_t* A, const uint16_t* B, const uint16_t* H,
                          const uint16_t* Y, const uint16_t* dZ, int64_t T, int64_t h, int64_t f, int gelu,
                          float* dX, uint16_t* dA, uint16_t* dB, uint16_t* db1, void* ws, hipStream_t st) {
  return gelu == kGeluErf
             ? mlp_bwd_impl<kGeluErf>(X, A, B, H, Y, dZ, T, h, f, dX, dA, dB, db1, (char*)ws, st)
             : mlp_bwd_impl<kGeluTanh>(X, A, B, H, Y, dZ, T, h, f, dX, dA, dB, db1, (char*)ws, st);
}

hipError_t launch_vocab_ce(const uint16_t* X, const uint16_t* E, const int64_t* target, int64_t T, int64_t h,
                           int64_t v, int64_t vocab_start, float* m, float* s, float* z, void* ws,
                           hipStream_t st) {
  const CeWorkspace w = ce_workspace_layout(T, v);
  float* pm = (float*)((char*)ws + w.off_m);
  float* ps = (float*)((char*)ws + w.off_s);
  float* pz = (float*)((char*)ws + w.off_z);
  GemmGeom g = make_geom(T, v, h, 1);
  Operand a{X, h, T * h}, b{E, v, h * v};
  EpiCE e{target, vocab_start, pm, (int)((w.off_s - w.off_m) / 4), (int)T, (int)v, 0};
  hipError_t err = launch_gemm<true, false>(kTkCeGemm, g, a, b, e, st);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(ce_tile_combine, dim3((unsigned)((T + 63) / 64)), dim3(512), 0, st, pm, ps, pz, w.parts,
                     (int)T, m, s, z);
  return hipGetLastError();
}

hipError_t launch_ce_combine(const float* m, const float* s, const float* z, int t, int64_t T, float* loss,
                             float* loss_mean, hipStream_t st) {
  hipLaunchKernelGGL(ce_combine_tokens, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, m, s, z, t, T, loss);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !loss_mean) return err;
  hipLaunchKernelGGL(mean_fixed_tree, dim3(1), dim3(1024), 0, st, loss, T, loss_mean);
  return hipGetLastError();
}

}  // namespace mshard
