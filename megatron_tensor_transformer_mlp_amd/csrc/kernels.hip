// kernels.hip - the GEMM instantiations and launch sequences of every entry
// point (MLP shard forward and backward, CE shard forward and backward,
// attention shard forward and backward: its core kernels are in
// attention.hip), the backward launch planner, the workspace layouts, and the
// small fixed-order reduction kernels (split-K slices, bias-gradient partials,
// CE tile partials, CE shard combine, CE backward row statistics).  Every
// reduction adds its terms in an order
// fixed by the shapes alone, with one private slot per writer and no atomics,
// which is what makes repeated calls bitwise identical (Megatron Core
// bitwise-determinism news item, news.hamidun.com: fixed reduction order and
// private per-writer output space).
#include "launch.hpp"

#include <algorithm>
#include <array>
#include <cmath>
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <vector>

#include "epilogues.hpp"

namespace mshard {

// ---------------------------------------------------------------------------
// Small kernels

// out[i] = bf16( sum_{s = 0..S-1} ws[s*stride + i] ), s ascending; 8 elements per thread.
// The slices are read once and the result is not read back soon: both
// non-temporal (see the cache-policy note in gemm_core.hpp).
__global__ void __launch_bounds__(256) splitk_reduce_bf16(const float* __restrict__ ws, int64_t stride, int S,
                                                          int64_t n, uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  float acc[8];
  const f32x4_t* p = (const f32x4_t*)(ws + i);
  f32x4_t a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
  for (int r = 0; r < 4; ++r) { acc[r] = a[r]; acc[4 + r] = b[r]; }
  for (int s = 1; s < S; ++s) {
    const f32x4_t* q = (const f32x4_t*)(ws + (int64_t)s * stride + i);
    a = __builtin_nontemporal_load(q);
    b = __builtin_nontemporal_load(q + 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) { acc[r] += a[r]; acc[4 + r] += b[r]; }
  }
  u32x4_t o{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]), pack_bf16x2(acc[4], acc[5]),
            pack_bf16x2(acc[6], acc[7])};
  __builtin_nontemporal_store(o, (u32x4_t*)(out + i));
}

// The forward's tail columns: for element (t, c) of [T x tn], the
// pre-activation is the sum of the S split slices ws[s*T*tn + t*tn + c] in
// ascending s, plus the bias b1[c] when there is one (with none, no addition),
// as the GeLU epilogue forms it; H and GeLU(H) are stored in bf16 at row t, column c of H and Y
// (row pitch ld).  8 elements per thread.
template <int FORM>
__global__ void __launch_bounds__(256) splitk_gelu_reduce(const float* __restrict__ ws, int S, int64_t T, int tn,
                                                          const uint16_t* __restrict__ b1, int64_t ld,
                                                          uint16_t* __restrict__ H, uint16_t* __restrict__ Y) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  const int64_t n = T * tn;
  if (i >= n) return;
  const int64_t t = i / tn;
  const int c = (int)(i - t * tn);
  float acc[8];
  const f32x4_t* p = (const f32x4_t*)(ws + i);
  f32x4_t a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
  for (int r = 0; r < 4; ++r) { acc[r] = a[r]; acc[4 + r] = b[r]; }
  for (int sl = 1; sl < S; ++sl) {
    const f32x4_t* q = (const f32x4_t*)(ws + (int64_t)sl * n + i);
    a = __builtin_nontemporal_load(q);
    b = __builtin_nontemporal_load(q + 1);
#pragma unroll
    for (int r = 0; r < 4; ++r) { acc[r] += a[r]; acc[4 + r] += b[r]; }
  }
  float hv[8], yv[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) hv[r] = acc[r];
  if (b1) {  // without a bias, the sum itself (no addition), as in the epilogue
    const u32x4_t w = *(const u32x4_t*)(b1 + c);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hv[2 * r] += bf16_lo(w[r]);
      hv[2 * r + 1] += bf16_hi(w[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) yv[r] = gelu_f<FORM>(hv[r]);
  const int64_t o = t * ld + c;
  *(u32x4_t*)(H + o) = u32x4_t{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]), pack_bf16x2(hv[4], hv[5]),
                               pack_bf16x2(hv[6], hv[7])};
  *(u32x4_t*)(Y + o) = u32x4_t{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]), pack_bf16x2(yv[4], yv[5]),
                               pack_bf16x2(yv[6], yv[7])};
}

// The second forward GEMM's tail columns: element (t, c) of [T x tn] is the
// sum of the S split slices ws[s*T*tn + t*tn + c] in ascending s, stored in
// fp32 at row t, column c of Z (row pitch ld).  8 elements per thread.
__global__ void __launch_bounds__(256) splitk_reduce_f32(const float* __restrict__ ws, int S, int64_t T, int tn,
                                                         int64_t ld, float* __restrict__ Z) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  const int64_t n = T * tn;
  if (i >= n) return;
  const int64_t t = i / tn;
  const int c = (int)(i - t * tn);
  const f32x4_t* p = (const f32x4_t*)(ws + i);
  f32x4_t a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
  for (int sl = 1; sl < S; ++sl) {
    const f32x4_t* q = (const f32x4_t*)(ws + (int64_t)sl * n + i);
    a += __builtin_nontemporal_load(q);
    b += __builtin_nontemporal_load(q + 1);
  }
  f32x4_t* o = (f32x4_t*)(Z + t * ld + c);
  __builtin_nontemporal_store(a, o);
  __builtin_nontemporal_store(b, o + 1);
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
// (m, s, z).  A block covers 32 rows with 16 groups of 32 lanes (two per wave,
// one row per lane, 128-byte loads); group g takes partials
// [g*P/16, (g+1)*P/16) in ascending chunks of 8: a chunk's loads are issued
// together, its maximum raises the running maximum (rescaling the running sum
// once), and its terms s_p exp(m_p - max) are added in ascending p.  Group 0
// then merges the 16 group results in ascending g.  T/32 blocks fill the chip
// at the workloads' token counts.
constexpr int kCombineRows = 32, kCombineGroups = 16, kCombineChunk = 8;
__global__ void __launch_bounds__(512) ce_tile_combine(const float* __restrict__ pm, const float* __restrict__ ps,
                                                       const float* __restrict__ pz, int P, int T,
                                                       float* __restrict__ m, float* __restrict__ s,
                                                       float* __restrict__ z) {
  __shared__ float xm[kCombineGroups][kCombineRows], xs[kCombineGroups][kCombineRows],
      xz[kCombineGroups][kCombineRows];
  const int r = threadIdx.x % kCombineRows, gi = threadIdx.x / kCombineRows;
  const int row = blockIdx.x * kCombineRows + r;
  const int p0 = (int)(((int64_t)gi * P) / kCombineGroups), p1 = (int)(((int64_t)(gi + 1) * P) / kCombineGroups);
  float M = -INFINITY, S = 0.f, Z = 0.f;
  if (row < T) {
    for (int p = p0; p < p1; p += kCombineChunk) {
      float cm[kCombineChunk], cs[kCombineChunk], cz[kCombineChunk];
#pragma unroll
      for (int j = 0; j < kCombineChunk; ++j) {
        const bool in = p + j < p1;
        const int64_t o = (int64_t)(p + j) * T + row;
        cm[j] = in ? __builtin_nontemporal_load(pm + o) : -INFINITY;
        cs[j] = in ? __builtin_nontemporal_load(ps + o) : 0.f;
        cz[j] = in ? __builtin_nontemporal_load(pz + o) : 0.f;
      }
      float mx = cm[0];
#pragma unroll
      for (int j = 1; j < kCombineChunk; ++j) mx = fmaxf(mx, cm[j]);
      if (mx > M) {
        S = S > 0.f ? S * expf(M - mx) : 0.f;
        M = mx;
      }
#pragma unroll
      for (int j = 0; j < kCombineChunk; ++j) {
        S += cs[j] > 0.f ? cs[j] * expf(cm[j] - M) : 0.f;  // empty parts and padding add nothing
        Z += cz[j];
      }
    }
  }
  xm[gi][r] = M;
  xs[gi][r] = S;
  xz[gi][r] = Z;
  __syncthreads();
  if (gi == 0 && row < T) {
    for (int q = 1; q < kCombineGroups; ++q) {
      lse_merge(M, S, xm[q][r], xs[q][r]);
      Z += xz[q][r];
    }
    m[row] = M;
    s[row] = S;
    z[row] = Z;
  }
}

// Loss of token i: the t shards' partials merged in ascending rank order.
__device__ __forceinline__ float token_loss(const float* __restrict__ m, const float* __restrict__ s,
                                            const float* __restrict__ z, int t, int64_t T, int64_t i) {
  float M = -INFINITY, S = 0.f, Z = 0.f;
  for (int r = 0; r < t; ++r) {
    const int64_t o = (int64_t)r * T + i;
    lse_merge(M, S, m[o], s[o]);
    Z += z[o];
  }
  return logf(S) + M - Z;
}

// Per token: merge t shards' partials in ascending rank order into the loss.
__global__ void __launch_bounds__(256) ce_combine_tokens(const float* __restrict__ m, const float* __restrict__ s,
                                                         const float* __restrict__ z, int t, int64_t T,
                                                         float* __restrict__ loss) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T) return;
  loss[i] = token_loss(m, s, z, t, T, i);
}

// Per token, the record the cross-entropy backward's epilogue reads: the
// ranks' (m, s) merged in ascending rank order as in ce_combine_tokens, then
// {M log2 e, coef / S, coef, target column in this shard or -1}, with
// coef = scale * dloss[i] (dloss may be null: 1).
__global__ void __launch_bounds__(256) ce_bwd_rowstats(const float* __restrict__ m, const float* __restrict__ s,
                                                       int t, int64_t T, const float* __restrict__ dloss,
                                                       float scale, const int64_t* __restrict__ target,
                                                       int64_t vocab_start, int64_t v, f32x4_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T) return;
  float M = -INFINITY, S = 0.f;
  for (int r = 0; r < t; ++r) {
    const int64_t o = (int64_t)r * T + i;
    lse_merge(M, S, m[o], s[o]);
  }
  const float coef = dloss ? scale * dloss[i] : scale;
  const int64_t tc = target[i] - vocab_start;
  const int col = (tc >= 0 && tc < v) ? (int)tc : -1;
  out[i] = f32x4_t{M * kLog2e, coef / S, coef, __int_as_float(col)};
}

// The fixed binary tree over the 1024 per-thread sums of one workgroup: out = sum / T.
__device__ __forceinline__ void mean_tree_1024(float acc, int64_t T, float* __restrict__ out) {
  __shared__ float red[1024];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0] / (float)T;
}

// Mean of loss[0..T): thread j sums j, j+1024, ... in order, then a fixed
// binary tree over the 1024 thread sums.  One workgroup.
__global__ void __launch_bounds__(1024) mean_fixed_tree(const float* __restrict__ x, int64_t T,
                                                        float* __restrict__ out) {
  float acc = 0.f;
  for (int64_t i = threadIdx.x; i < T; i += 1024) acc += x[i];
  mean_tree_1024(acc, T, out);
}

// Largest t*T that ce_combine_mean_small takes (64 partials per thread).
constexpr int64_t kCombineSmall = 65536;

// ce_combine_tokens followed by mean_fixed_tree in one workgroup, for small
// t*T: thread j forms the losses of tokens j, j+1024, ... and sums them in that
// order, so loss and mean are the same bits as the two-kernel path's.
__global__ void __launch_bounds__(1024) ce_combine_mean_small(const float* __restrict__ m,
                                                              const float* __restrict__ s,
                                                              const float* __restrict__ z, int t, int64_t T,
                                                              float* __restrict__ loss, float* __restrict__ out) {
  float acc = 0.f;
  for (int64_t i0 = threadIdx.x; i0 < T; i0 += 8 * 1024) {
    float l[8];  // eight tokens' losses formed together, then summed in token order
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t i = i0 + (int64_t)j * 1024;
      l[j] = i < T ? token_loss(m, s, z, t, T, i) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t i = i0 + (int64_t)j * 1024;
      if (i < T) {
        loss[i] = l[j];
        acc += l[j];
      }
    }
  }
  mean_tree_1024(acc, T, out);
}

// ---------------------------------------------------------------------------
// GEMM launch helpers

// Compute units of the current device (queried once per device).
static hipError_t device_compute_units(int* cus) {
  static std::mutex mu;
  static std::map<int, int> per_device;
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(mu);
  auto it = per_device.find(dev);
  if (it != per_device.end()) {
    *cus = it->second;
    return hipSuccess;
  }
  int n = 0;
  err = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  per_device.emplace(dev, n);
  *cus = n;
  return hipSuccess;
}

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

// ---------------------------------------------------------------------------
// Backward schedule.  For each independent pair of backward GEMMs -- (dB, dH)
// and (dA, dX) -- the host chooses two launches or one paired launch, and the
// weight gradient's K split, by a list-scheduling model of the 256 CUs:
// blocks are handed in order to the earliest free CU, each costing ~1400
// cycles per 32-k step + ~4000 to fill the pipeline + an epilogue cost by
// kind (measured on this kernel at ~2 GHz), and a split-K reduction costs its
// bytes at ~4 TB/s.  Only launch shapes and the (fixed) order of the fp32
// additions depend on the plan, and equal shapes always get equal plans.
namespace {
constexpr int kModelCUs = 256;
constexpr double kCyclesPerKStep = 1400.0, kFillCycles = 4000.0, kCyclesPerUs = 2000.0;
constexpr double kEpiDGelu = 40000.0, kEpiF32 = 12000.0, kEpiBF16 = 10000.0, kEpiGelu = 29000.0;

struct BlockList {
  int64_t n;
  double cost;  // cycles per block
};

double block_cost(int64_t K, int S, double epi) {
  const int64_t nk = (K + kBK - 1) / kBK;
  return kCyclesPerKStep * (double)((nk + S - 1) / S) + kFillCycles + epi;
}

int64_t tile_count(int64_t M, int64_t N) { return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN); }

// Completion time (us) of the block lists dispatched in order to the earliest free CU.
double makespan_us(std::initializer_list<BlockList> lists) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> q;
  for (int i = 0; i < kModelCUs; ++i) q.push(0.0);
  double end = 0.0;
  for (const BlockList& l : lists)
    for (int64_t i = 0; i < l.n; ++i) {
      const double t = q.top() + l.cost;
      q.pop();
      q.push(t);
      end = t > end ? t : end;
    }
  return end / kCyclesPerUs;
}

double reduce_us(int64_t M, int64_t N, int S) {
  return S == 1 ? 0.0 : (double)(4 * S + 2) * (double)M * (double)N / 4e6 + 3.0;
}

// Weight gradient [M x N] (contraction over T) with partner GEMM blocks `p`;
// K splits above max_splits are not considered.
void plan_pair(int64_t M, int64_t N, int64_t T, BlockList p, int& S_out, bool& paired, bool& partner_first,
               int max_splits = 8) {
  const int64_t nk = (T + kBK - 1) / kBK;
  const double alone = makespan_us({p});
  double best = 1e300;
  for (int S = 1; S <= max_splits; S *= 2) {
    if (S > 1 && nk / S < 8) break;
    const BlockList w{tile_count(M, N) * S, block_cost(T, S, S == 1 ? kEpiBF16 : kEpiF32)};
    const double seq = makespan_us({w}) + alone + reduce_us(M, N, S);
    const bool pf = p.cost > w.cost;
    const double par = (pf ? makespan_us({p, w}) : makespan_us({w, p})) + reduce_us(M, N, S);
    if (seq < best) {
      best = seq;
      S_out = S;
      paired = false;
      partner_first = false;
    }
    if (par <= best) {  // on a tie the paired launch saves a launch
      best = par;
      S_out = S;
      paired = true;
      partner_first = pf;
    }
  }
}
}  // namespace

BwdPlan plan_backward(int64_t T, int64_t h, int64_t f) {
  // plans are cached per shape: the model simulates up to tens of thousands of blocks
  static std::mutex mu;
  static std::map<std::array<int64_t, 3>, BwdPlan> cache;
  const std::array<int64_t, 3> key{T, h, f};
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  BwdPlan pl;
  const BlockList dh{tile_count(T, f), block_cost(h, 1, kEpiDGelu)};
  const BlockList dx{tile_count(T, h), block_cost(f, 1, kEpiF32)};
  plan_pair(f, h, T, dh, pl.splits_dB, pl.pair_bh, pl.dh_first);
  plan_pair(h, f, T, dx, pl.splits_dA, pl.pair_ax, pl.dx_first);
  std::lock_guard<std::mutex> lock(mu);
  cache.emplace(key, pl);
  return pl;
}

// Forward plan: for each GEMM of the forward, the plain launch or its last
// tile columns split over K (see FwdPlan), whichever the same model gives the
// shorter time, the split only when it wins by at least 3%.  The split blocks
// are dispatched first (see mlp_fwd_impl).  The reduction is charged its bytes
// (S fp32 slices read, 4 bytes per element written: H and Y, or Z) at ~4 TB/s
// plus a launch.  Considered only where the plain launch has more tiles than
// CUs and at most 16 rounds of them (beyond that the last round's idle share is
// small).
namespace {
void plan_tail(int64_t M, int64_t N, int64_t K, double epi, int& tail_n, int& tail_splits) {
  tail_n = 0;
  tail_splits = 1;
  const int64_t tm = (M + kBM - 1) / kBM, tn = (N + kBN - 1) / kBN, nk = (K + kBK - 1) / kBK;
  if (tm * tn <= kModelCUs || tm * tn > 16 * kModelCUs || nk < 8) return;
  double best = 0.97 * makespan_us({BlockList{tm * tn, block_cost(K, 1, epi)}});
  for (int64_t nc = 1; nc < tn && nc <= 32; ++nc) {
    const int64_t tail = N - (tn - nc) * kBN;
    for (int S = 2; S <= 8 && nk / S >= 4; S *= 2) {
      const double t = makespan_us({BlockList{tm * nc * S, block_cost(K, S, kEpiF32)},
                                    BlockList{tm * (tn - nc), block_cost(K, 1, epi)}}) +
                       (double)(4 * S + 4) * (double)M * (double)tail / 4e6 + 3.0;
      if (t < best) {
        best = t;
        tail_n = (int)tail;
        tail_splits = S;
      }
    }
  }
}
}  // namespace

FwdPlan plan_forward(int64_t T, int64_t h, int64_t f) {
  static std::mutex mu;
  static std::map<std::array<int64_t, 3>, FwdPlan> cache;
  const std::array<int64_t, 3> key{T, h, f};
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  FwdPlan pl;
  plan_tail(T, f, h, kEpiGelu, pl.tail_n, pl.tail_splits);    // H = X A_i: M = T, N = f, K = h
  plan_tail(T, h, f, kEpiF32, pl.z_tail_n, pl.z_tail_splits);  // Z = Y B_i: M = T, N = h, K = f
  std::lock_guard<std::mutex> lock(mu);
  cache.emplace(key, pl);
  return pl;
}

MlpWorkspace mlp_workspace_layout(int64_t T, int64_t h, int64_t f) {
  MlpWorkspace w;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t tiles_m = (T + kBM - 1) / kBM;
  w.plan = plan_backward(T, h, f);
  w.off_dH = 0;
  w.off_db1 = align((size_t)T * f * 2);
  w.db1_parts = (int)(tiles_m * kWavesM);
  w.off_splitk = w.off_db1 + align((size_t)w.db1_parts * f * 4);
  const int S = w.plan.splits_dB > w.plan.splits_dA ? w.plan.splits_dB : w.plan.splits_dA;
  w.bytes = w.off_splitk + (S > 1 ? align((size_t)S * h * f * 4) : 0);
  w.max_region = std::max({(size_t)T * f * 2, (size_t)w.db1_parts * f * 4, S > 1 ? (size_t)h * f * 4 : (size_t)0});
  w.fwd = plan_forward(T, h, f);
  w.off_fwd_tail = 0;
  if (w.fwd.tail_n > 0) {
    const size_t slice = (size_t)T * w.fwd.tail_n * 4;
    w.bytes = std::max(w.bytes, align(slice * w.fwd.tail_splits));
    w.max_region = std::max(w.max_region, slice);
  }
  if (w.fwd.z_tail_n > 0) {
    const size_t slice = (size_t)T * w.fwd.z_tail_n * 4;
    w.bytes = std::max(w.bytes, align(slice * w.fwd.z_tail_splits));
    w.max_region = std::max(w.max_region, slice);
  }
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
  w.max_region = (size_t)w.parts * T * 4;
  return w;
}

// Cross-entropy backward: per-token records, the bf16 logit gradient dL
// [T x v], and the split-K slices of dE when the plan splits it.  dE = X^T dL
// and dX = dL E^T are independent and planned like the MLP's (dA, dX); the
// split is capped so that the whole workspace stays below 2^31 bytes.
CeBwdWorkspace ce_bwd_workspace_layout(int64_t T, int64_t h, int64_t v) {
  static std::mutex mu;
  static std::map<std::array<int64_t, 3>, CeBwdWorkspace> cache;
  const std::array<int64_t, 3> key{T, h, v};
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  CeBwdWorkspace w;
  w.off_stats = 0;
  w.off_dL = align((size_t)T * 16);
  w.off_splitk = w.off_dL + align((size_t)T * v * 2);
  const size_t slice = (size_t)h * v * 4;
  int max_splits = 1;
  while (max_splits < 8 && w.off_splitk + align(slice * 2 * max_splits) < ((size_t)1 << 31)) max_splits *= 2;
  const BlockList dx{tile_count(T, h), block_cost(v, 1, kEpiF32)};
  plan_pair(h, v, T, dx, w.splits_dE, w.paired, w.dx_first, max_splits);
  w.bytes = w.off_splitk + (w.splits_dE > 1 ? align(slice * w.splits_dE) : 0);
  w.max_region = std::max({(size_t)T * 16, (size_t)T * v * 2, w.splits_dE > 1 ? slice : (size_t)0});
  std::lock_guard<std::mutex> lock(mu);
  cache.emplace(key, w);
  return w;
}

AttnWorkspace attn_workspace_layout(int64_t b, int64_t s, int64_t h, int64_t n, int64_t d) {
  static std::mutex mu;
  static std::map<std::array<int64_t, 5>, AttnWorkspace> cache;
  const std::array<int64_t, 5> key{b, s, h, n, d};
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const int64_t T = b * s, nd = n * d;
  AttnWorkspace w;
  w.off_dO = 0;
  w.off_delta = align((size_t)T * nd * 2);
  w.off_dqkv = w.off_delta + align((size_t)n * T * 4);
  w.off_splitk = w.off_dqkv + align((size_t)T * 3 * nd * 2);
  const size_t slice = (size_t)h * 3 * nd * 4;  // the larger of the two weight gradients
  int max_splits = 1;
  while (max_splits < 8 && w.off_splitk + align(slice * 2 * max_splits) < ((size_t)1 << 31)) max_splits *= 2;
  const BlockList dO{tile_count(T, nd), block_cost(h, 1, kEpiBF16)};
  const BlockList dx{tile_count(T, h), block_cost(3 * nd, 1, kEpiF32)};
  plan_pair(nd, h, T, dO, w.splits_wo, w.pair_o, w.o_first, max_splits);
  plan_pair(h, 3 * nd, T, dx, w.splits_wqkv, w.pair_x, w.x_first, max_splits);
  const int S = w.splits_wo > w.splits_wqkv ? w.splits_wo : w.splits_wqkv;
  w.bytes = w.off_splitk + (S > 1 ? align(slice * S) : 0);
  w.max_region = std::max({(size_t)T * nd * 2, (size_t)n * T * 4, (size_t)T * 3 * nd * 2, S > 1 ? slice : (size_t)0});
  std::lock_guard<std::mutex> lock(mu);
  cache.emplace(key, w);
  return w;
}

// ---------------------------------------------------------------------------
// Entry-point launch sequences (arguments already validated by the ABI layer)

template <int FORM>
static hipError_t mlp_fwd_impl(const uint16_t* X, const uint16_t* A, const uint16_t* b1, const uint16_t* B,
                               int64_t T, int64_t h, int64_t f, uint16_t* H, uint16_t* Y, float* Z, char* ws,
                               hipStream_t st) {
  // H = X A (+ b1), Y = GeLU(H):  NN, M = T, N = f, K = h
  const FwdPlan pl = plan_forward(T, h, f);
  const Operand a{X, h, T * h};
  if (pl.tail_n == 0) {
    GemmGeom g = make_geom(T, f, h, 1);
    Operand b{A, f, h * f};
    EpiGeluFwd<FORM> e{H, Y, b1, f, (int)T, (int)f};
    hipError_t err = launch_gemm<true, false>(kTkFwdH, g, a, b, e, st);
    if (err != hipSuccess) return err;
  } else {
    // columns [0, n1) with the GeLU epilogue, and the tail columns [n1, f) split
    // over K into fp32 slices, in one launch; then the slices are summed with
    // the bias and GeLU.  The short split blocks are dispatched first: the CUs
    // that take them start their full tiles a fraction of a tile later, so the
    // full tiles' store-heavy GeLU epilogues fall at two different times instead
    // of on every CU at once (measured about 3% faster than the full tiles first)
    const int64_t n1 = f - pl.tail_n;
    float* slices = (float*)(ws + mlp_workspace_layout(T, h, f).off_fwd_tail);
    const GemmGeom g1 = make_geom(T, n1, h, 1);
    const Operand b1o{A, f, h * f};
    const EpiGeluFwd<FORM> e1{H, Y, b1, f, (int)T, (int)n1};
    const GemmGeom g2 = make_geom(T, pl.tail_n, h, pl.tail_splits);
    const Operand b2o{A + n1, f, h * f - n1};
    const EpiStoreF32 e2{slices, pl.tail_n, (int)T, (int)pl.tail_n, T * pl.tail_n};
    const int nb1 = g1.tiles_m * g1.tiles_n * g1.splits, nb2 = g2.tiles_m * g2.tiles_n * g2.splits;
    record_armed_event(kTkFwdH, false, st);
    hipLaunchKernelGGL((gemm_pair_kernel<true, false, EpiGeluFwd<FORM>, true, false, EpiStoreF32>),
                       dim3(((nb2 + 7) & ~7) + nb1), dim3(kThreads), 0, st, g1, a, b1o, e1, nb1, g2, a, b2o, e2, nb2, 1);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t n8 = T * pl.tail_n / 8;
    hipLaunchKernelGGL((splitk_gelu_reduce<FORM>), dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, slices,
                       g2.splits, T, pl.tail_n, b1 ? b1 + n1 : nullptr, f, H + n1, Y + n1);
    err = hipGetLastError();
    record_armed_event(kTkFwdH, true, st);
    if (err != hipSuccess) return err;
  }
  // Z = Y B:  NN, M = T, N = h, K = f
  const Operand ay{Y, f, T * f};
  if (pl.z_tail_n == 0) {
    GemmGeom g = make_geom(T, h, f, 1);
    Operand b{B, h, f * h};
    EpiStoreF32 e{Z, h, (int)T, (int)h, 0};
    return launch_gemm<true, false>(kTkFwdZ, g, ay, b, e, st);
  }
  // columns [0, n1) stored straight into Z, and the tail columns [n1, h) split
  // over K into fp32 slices (those blocks first, as above), then summed into Z
  const int64_t n1 = h - pl.z_tail_n;
  float* slices = (float*)(ws + mlp_workspace_layout(T, h, f).off_fwd_tail);
  const GemmGeom g1 = make_geom(T, n1, f, 1);
  const Operand b1o{B, h, f * h};
  const EpiStoreF32 e1{Z, h, (int)T, (int)n1, 0};
  const GemmGeom g2 = make_geom(T, pl.z_tail_n, f, pl.z_tail_splits);
  const Operand b2o{B + n1, h, f * h - n1};
  const EpiStoreF32 e2{slices, pl.z_tail_n, (int)T, (int)pl.z_tail_n, T * pl.z_tail_n};
  const int nb1 = g1.tiles_m * g1.tiles_n * g1.splits, nb2 = g2.tiles_m * g2.tiles_n * g2.splits;
  record_armed_event(kTkFwdZ, false, st);
  hipLaunchKernelGGL((gemm_pair_kernel<true, false, EpiStoreF32, true, false, EpiStoreF32>),
                     dim3(((nb2 + 7) & ~7) + nb1), dim3(kThreads), 0, st, g1, ay, b1o, e1, nb1, g2, ay, b2o, e2, nb2, 1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t n8 = T * pl.z_tail_n / 8;
  hipLaunchKernelGGL(splitk_reduce_f32, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st, slices, g2.splits, T,
                     pl.z_tail_n, h, Z + n1);
  err = hipGetLastError();
  record_armed_event(kTkFwdZ, true, st);
  return err;
}

hipError_t launch_mlp_fwd(const uint16_t* X, const uint16_t* A, const uint16_t* b1, const uint16_t* B,
                          int64_t T, int64_t h, int64_t f, int gelu, uint16_t* H, uint16_t* Y, float* Z, void* ws,
                          hipStream_t st) {
  return gelu == kGeluErf ? mlp_fwd_impl<kGeluErf>(X, A, b1, B, T, h, f, H, Y, Z, (char*)ws, st)
                          : mlp_fwd_impl<kGeluTanh>(X, A, b1, B, T, h, f, H, Y, Z, (char*)ws, st);
}

// Two independent GEMMs as one launch (see gemm_pair_kernel); both kernel ids'
// armed events bracket the shared launch.
template <bool AK1, bool BK1, bool AK2, bool BK2, class E1, class E2>
static hipError_t launch_gemm_pair(int id1, const GemmGeom& g1, const Operand& a1, const Operand& b1, const E1& e1,
                                   int id2, const GemmGeom& g2, const Operand& a2, const Operand& b2, const E2& e2,
                                   bool second_first, hipStream_t stream) {
  const int n1 = g1.tiles_m * g1.tiles_n * g1.splits, n2 = g2.tiles_m * g2.tiles_n * g2.splits;
  const int lead = second_first ? n2 : n1, trail = second_first ? n1 : n2;
  const int blocks = ((lead + 7) & ~7) + trail;
  record_armed_event(id1, false, stream);
  record_armed_event(id2, false, stream);
  hipLaunchKernelGGL((gemm_pair_kernel<AK1, BK1, E1, AK2, BK2, E2>), dim3(blocks), dim3(kThreads), 0, stream, g1, a1,
                     b1, e1, n1, g2, a2, b2, e2, n2, second_first ? 1 : 0);
  const hipError_t err = hipGetLastError();
  record_armed_event(id1, true, stream);
  record_armed_event(id2, true, stream);
  return err;
}

static hipError_t launch_splitk_reduce(const float* splitk, int64_t M, int64_t N, int S, uint16_t* C, hipStream_t st) {
  const int64_t n = M * N;  // multiple of 8
  const int64_t blocks = (n / 8 + 255) / 256;
  hipLaunchKernelGGL(splitk_reduce_bf16, dim3((unsigned)blocks), dim3(256), 0, st, splitk, M * N, S, n, C);
  return hipGetLastError();
}

// Weight gradient C[M x N] = sum_t P[t, m] Q[t, n] (TN): its GEMM geometry,
// operands and epilogue -- the bf16 result, or with a K split the fp32
// workspace slices that splitk_reduce_bf16 sums in fixed order.
struct WeightGrad {
  GemmGeom g;
  Operand a, b;
  EpiStoreWGrad e;
  int S;
};

static WeightGrad weight_grad_setup(const uint16_t* P, int64_t ldp, const uint16_t* Q, int64_t ldq, int64_t Kt,
                                    int64_t M, int64_t N, int S, uint16_t* C, float* splitk) {
  WeightGrad w;
  w.g = make_geom(M, N, Kt, S);
  w.S = w.g.splits;
  w.a = Operand{P, ldp, Kt * ldp};
  w.b = Operand{Q, ldq, Kt * ldq};
  w.e = w.S == 1 ? EpiStoreWGrad{C, N, (int)M, (int)N, 0} : EpiStoreWGrad{splitk, N, (int)M, (int)N, M * N};
  return w;
}

template <int FORM>
static hipError_t mlp_bwd_impl(const uint16_t* X, const uint16_t* A, const uint16_t* B, const uint16_t* H,
                               const uint16_t* Y, const uint16_t* dZ, int64_t T, int64_t h, int64_t f,
                               float* dX, uint16_t* dA, uint16_t* dB, uint16_t* db1, char* ws, hipStream_t st) {
  const MlpWorkspace w = mlp_workspace_layout(T, h, f);
  const BwdPlan& pl = w.plan;
  uint16_t* dH = (uint16_t*)(ws + w.off_dH);
  float* db1_part = db1 ? (float*)(ws + w.off_db1) : nullptr;
  float* splitk = (float*)(ws + w.off_splitk);
  hipError_t err;
  // dH = (dZ B^T) * GeLU'(H):  NT, M = T, N = f, K = h; B stored [f x h] = [N x K]
  const GemmGeom gh = make_geom(T, f, h, 1);
  const Operand ah{dZ, h, T * h}, bh{B, h, f * h};
  const EpiDGelu<FORM> eh{H, dH, db1_part, f, (int)T, (int)f};
  // dB = Y^T dZ:  [f x h], contraction over tokens (independent of dH)
  const WeightGrad wb = weight_grad_setup(Y, f, dZ, h, T, f, h, pl.splits_dB, dB, splitk);
  if (pl.pair_bh) {
    err = launch_gemm_pair<false, false, true, true>(kTkBwdDB, wb.g, wb.a, wb.b, wb.e, kTkBwdDH, gh, ah, bh, eh,
                                                     pl.dh_first, st);
  } else {
    err = launch_gemm<true, true>(kTkBwdDH, gh, ah, bh, eh, st);
    if (err == hipSuccess) err = launch_gemm<false, false>(kTkBwdDB, wb.g, wb.a, wb.b, wb.e, st);
  }
  if (err != hipSuccess) return err;
  if (wb.S > 1 && (err = launch_splitk_reduce(splitk, f, h, wb.S, dB, st)) != hipSuccess) return err;
  // dA = X^T dH:  [h x f];  dX = dH A^T:  NT, M = T, N = h, K = f; A stored [h x f] = [N x K]
  const WeightGrad wa = weight_grad_setup(X, h, dH, f, T, h, f, pl.splits_dA, dA, splitk);
  const GemmGeom gx = make_geom(T, h, f, 1);
  const Operand ax{dH, f, T * f}, bx{A, f, h * f};
  const EpiStoreF32 ex{dX, h, (int)T, (int)h, 0};
  if (pl.pair_ax) {
    err = launch_gemm_pair<false, false, true, true>(kTkBwdDA, wa.g, wa.a, wa.b, wa.e, kTkBwdDX, gx, ax, bx, ex,
                                                     pl.dx_first, st);
  } else {
    err = launch_gemm<false, false>(kTkBwdDA, wa.g, wa.a, wa.b, wa.e, st);
    if (err == hipSuccess) err = launch_gemm<true, true>(kTkBwdDX, gx, ax, bx, ex, st);
  }
  if (err != hipSuccess) return err;
  if (wa.S > 1 && (err = launch_splitk_reduce(splitk, h, f, wa.S, dA, st)) != hipSuccess) return err;
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
  // persistent: at most one workgroup per CU, a multiple of 8 of them, each walking its tiles
  int cus = 0;
  hipError_t err = device_compute_units(&cus);
  if (err != hipSuccess) return err;
  const int vg = g.tiles_m * g.tiles_n * g.splits;
  int P = cus - cus % 8;
  if (P < 8) P = 8;
  if (P > vg) P = vg;
  record_armed_event(kTkCeGemm, false, st);
  hipLaunchKernelGGL((gemm_persistent_kernel<true, false, EpiCE>), dim3(P), dim3(kThreads), 0, st, g, a, b, e, vg);
  err = hipGetLastError();
  record_armed_event(kTkCeGemm, true, st);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(ce_tile_combine, dim3((unsigned)((T + kCombineRows - 1) / kCombineRows)),
                     dim3(kCombineRows * kCombineGroups), 0, st, pm, ps, pz, w.parts, (int)T, m, s, z);
  return hipGetLastError();
}

hipError_t launch_vocab_ce_bwd(const uint16_t* X, const uint16_t* E, const int64_t* target, const float* m,
                               const float* s, int t, const float* dloss, float scale, int64_t T, int64_t h,
                               int64_t v, int64_t vocab_start, float* dX, uint16_t* dE, void* ws, hipStream_t st) {
  const CeBwdWorkspace w = ce_bwd_workspace_layout(T, h, v);
  f32x4_t* stats = (f32x4_t*)((char*)ws + w.off_stats);
  uint16_t* dL = (uint16_t*)((char*)ws + w.off_dL);
  float* splitk = (float*)((char*)ws + w.off_splitk);
  hipLaunchKernelGGL(ce_bwd_rowstats, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, m, s, t, T, dloss,
                     scale, target, vocab_start, v, stats);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // dL from the recomputed logits X E:  NN, M = T, N = v, K = h
  {
    const GemmGeom g = make_geom(T, v, h, 1);
    const Operand a{X, h, T * h}, b{E, v, h * v};
    const EpiCEGrad e{stats, dL, v, (int)T, (int)v};
    if ((err = launch_gemm<true, false>(kTkCeBwdL, g, a, b, e, st)) != hipSuccess) return err;
  }
  // dE = X^T dL:  [h x v], contraction over tokens;  dX = dL E^T:  NT, M = T, N = h, K = v;
  // E stored [h x v] = [N x K]
  const WeightGrad we = weight_grad_setup(X, h, dL, v, T, h, v, w.splits_dE, dE, splitk);
  const GemmGeom gx = make_geom(T, h, v, 1);
  const Operand ax{dL, v, T * v}, bx{E, v, h * v};
  const EpiStoreF32 ex{dX, h, (int)T, (int)h, 0};
  if (w.paired) {
    err = launch_gemm_pair<false, false, true, true>(kTkCeBwdDE, we.g, we.a, we.b, we.e, kTkCeBwdDX, gx, ax, bx, ex,
                                                     w.dx_first, st);
  } else {
    err = launch_gemm<true, true>(kTkCeBwdDX, gx, ax, bx, ex, st);
    if (err == hipSuccess) err = launch_gemm<false, false>(kTkCeBwdDE, we.g, we.a, we.b, we.e, st);
  }
  if (err != hipSuccess) return err;
  if (we.S > 1) err = launch_splitk_reduce(splitk, h, v, we.S, dE, st);
  return err;
}

// Self-attention shard ([EXPL] "attention"; [NOTES] "self-attention block
// split"): QKV = X Wqkv_i (column shard, this rank's heads), the attention
// core per head, Z_i = O_i W_O,i (row shard: this rank's fp32 partial).
static AttnGeom attn_geom(int64_t b, int64_t s, int64_t n, int64_t d) {
  AttnGeom g;
  g.b = (int)b;
  g.s = (int)s;
  g.n = (int)n;
  g.d = (int)d;
  g.ld_qkv = (int)(3 * n * d);
  g.ld_o = (int)(n * d);
  g.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)d));
  return g;
}

hipError_t launch_attn_fwd(const uint16_t* X, const uint16_t* Wqkv, const uint16_t* Wo, int64_t b, int64_t s,
                           int64_t h, int64_t n, int64_t d, bool causal, uint16_t* QKV, uint16_t* O, float* lse,
                           float* Z, hipStream_t st) {
  const int64_t T = b * s, nd = n * d;
  hipError_t err;
  {  // QKV = X Wqkv:  NN, M = T, N = 3nd, K = h
    const GemmGeom g = make_geom(T, 3 * nd, h, 1);
    const Operand a{X, h, T * h}, bo{Wqkv, 3 * nd, h * 3 * nd};
    const EpiStoreBF16 e{QKV, 3 * nd, (int)T, (int)(3 * nd)};
    if ((err = launch_gemm<true, false>(kTkAttnQkv, g, a, bo, e, st)) != hipSuccess) return err;
  }
  record_armed_event(kTkAttnCoreFwd, false, st);
  err = launch_attn_core_fwd(attn_geom(b, s, n, d), causal, QKV, O, lse, st);
  record_armed_event(kTkAttnCoreFwd, true, st);
  if (err != hipSuccess) return err;
  // Z = O Wo:  NN, M = T, N = h, K = nd
  const GemmGeom g = make_geom(T, h, nd, 1);
  const Operand a{O, nd, T * nd}, bo{Wo, h, nd * h};
  const EpiStoreF32 e{Z, h, (int)T, (int)h, 0};
  return launch_gemm<true, false>(kTkAttnOut, g, a, bo, e, st);
}

hipError_t launch_attn_bwd(const uint16_t* X, const uint16_t* Wqkv, const uint16_t* Wo, const uint16_t* QKV,
                           const uint16_t* O, const float* lse, const uint16_t* dZ, int64_t b, int64_t s, int64_t h,
                           int64_t n, int64_t d, bool causal, float* dX, uint16_t* dWqkv, uint16_t* dWo, void* ws,
                           hipStream_t st) {
  const int64_t T = b * s, nd = n * d;
  const AttnWorkspace w = attn_workspace_layout(b, s, h, n, d);
  uint16_t* dO = (uint16_t*)((char*)ws + w.off_dO);
  float* delta = (float*)((char*)ws + w.off_delta);
  uint16_t* dqkv = (uint16_t*)((char*)ws + w.off_dqkv);
  float* splitk = (float*)((char*)ws + w.off_splitk);
  hipError_t err;
  // dO = dZ Wo^T:  NT, M = T, N = nd, K = h; Wo stored [nd x h] = [N x K]
  const GemmGeom go = make_geom(T, nd, h, 1);
  const Operand ao{dZ, h, T * h}, bo{Wo, h, nd * h};
  const EpiStoreBF16 eo{dO, nd, (int)T, (int)nd};
  // dW_O = O^T dZ:  [nd x h], contraction over tokens (independent of dO)
  const WeightGrad wo = weight_grad_setup(O, nd, dZ, h, T, nd, h, w.splits_wo, dWo, splitk);
  if (w.pair_o) {
    err = launch_gemm_pair<false, false, true, true>(kTkAttnBwdDWo, wo.g, wo.a, wo.b, wo.e, kTkAttnBwdDO, go, ao, bo,
                                                     eo, w.o_first, st);
  } else {
    err = launch_gemm<true, true>(kTkAttnBwdDO, go, ao, bo, eo, st);
    if (err == hipSuccess) err = launch_gemm<false, false>(kTkAttnBwdDWo, wo.g, wo.a, wo.b, wo.e, st);
  }
  if (err != hipSuccess) return err;
  if (wo.S > 1 && (err = launch_splitk_reduce(splitk, nd, h, wo.S, dWo, st)) != hipSuccess) return err;
  record_armed_event(kTkAttnCoreBwd, false, st);
  err = launch_attn_core_bwd(attn_geom(b, s, n, d), causal, QKV, O, dO, lse, delta, dqkv, st);
  record_armed_event(kTkAttnCoreBwd, true, st);
  if (err != hipSuccess) return err;
  // dWqkv = X^T dQKV:  [h x 3nd];  dX = dQKV Wqkv^T:  NT, M = T, N = h, K = 3nd; Wqkv stored [h x 3nd] = [N x K]
  const WeightGrad wq = weight_grad_setup(X, h, dqkv, 3 * nd, T, h, 3 * nd, w.splits_wqkv, dWqkv, splitk);
  const GemmGeom gx = make_geom(T, h, 3 * nd, 1);
  const Operand ax{dqkv, 3 * nd, T * 3 * nd}, bx{Wqkv, 3 * nd, h * 3 * nd};
  const EpiStoreF32 ex{dX, h, (int)T, (int)h, 0};
  if (w.pair_x) {
    err = launch_gemm_pair<false, false, true, true>(kTkAttnBwdDWqkv, wq.g, wq.a, wq.b, wq.e, kTkAttnBwdDX, gx, ax, bx,
                                                     ex, w.x_first, st);
  } else {
    err = launch_gemm<true, true>(kTkAttnBwdDX, gx, ax, bx, ex, st);
    if (err == hipSuccess) err = launch_gemm<false, false>(kTkAttnBwdDWqkv, wq.g, wq.a, wq.b, wq.e, st);
  }
  if (err != hipSuccess) return err;
  if (wq.S > 1) err = launch_splitk_reduce(splitk, h, 3 * nd, wq.S, dWqkv, st);
  return err;
}

// Device-resident scratch of the allocation-free CE entry point: the per-tile
// (m, s, z) partials, up to kNoAllocScratchBytes.  One copy per GPU, kept for
// the life of the process; every call on a GPU uses that GPU's copy.  Host code
// never passes the array's name to a kernel (in host code it is only a
// stand-in for the symbol): it looks the device address up once per device
// and passes that.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  static std::mutex mu;
  static std::map<int, void*> per_device;
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(mu);
  auto it = per_device.find(dev);
  if (it != per_device.end()) {
    *ptr = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (err != hipSuccess) return err;
  per_device.emplace(dev, p);
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_ce_combine(const float* m, const float* s, const float* z, int t, int64_t T, float* loss,
                             float* loss_mean, hipStream_t st) {
  if (loss_mean && (int64_t)t * T <= kCombineSmall) {
    hipLaunchKernelGGL(ce_combine_mean_small, dim3(1), dim3(1024), 0, st, m, s, z, t, T, loss, loss_mean);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(ce_combine_tokens, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, st, m, s, z, t, T, loss);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !loss_mean) return err;
  hipLaunchKernelGGL(mean_fixed_tree, dim3(1), dim3(1024), 0, st, loss, T, loss_mean);
  return hipGetLastError();
}

}  // namespace mshard
