// epilogues.hpp - what each GEMM does with its fp32 accumulators.
//
// Accumulator element acc[mi][ni][r] of wave (wm, wn) in the tile at (m0, n0)
// is C[m0 + wm*kWaveM + mi*16 + (lane & 15)][n0 + wn*kWaveN + ni*16 + 4*(lane >> 4) + r].
//
// Epilogues hand the accumulators over through LDS: each wave writes its
// kWaveM x kWaveN fp32 sub-tile, 64 rows at a time, into a private region of
// the LDS stages (row pitch 4*kWaveN bytes, 16-byte chunk q of row r at slot
// q ^ (r & 15), so that every 8 lanes written or read together hit distinct
// 16-byte slots of a 128-byte window), then reads it back in a row-major lane
// order.  The accumulators are therefore only ever stored,
// which keeps them in the accumulation registers through the main loop, and
// global stores become full 256/512-byte row segments.  N is a multiple of 8,
// so every 4-column group is entirely inside or outside the matrix; rows are
// masked one by one.
#pragma once

#include "gemm_core.hpp"

namespace mshard {

enum GeluForm { kGeluErf = 0, kGeluTanh = 1 };

constexpr float kInvSqrt2 = 0.70710678118654752440f;
constexpr float kInvSqrt2Pi = 0.39894228040143267794f;
constexpr float kSqrt2OverPi = 0.79788456080286535588f;
constexpr float kTanhC = 0.044715f;
constexpr float kLog2e = 1.44269504088896340736f;

// GeLU and its derivative in fp32.
//
// Erf form, GeLU(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2.  erf is evaluated
// with Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: for z >= 0, erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5))))
// exp(-z^2), t = 1 / (1 + p z), with absolute error below 1.5e-7 (far below the
// bf16 rounding of the outputs); erf(-z) = -erf(z).  With z = |x|/sqrt 2 and
// tail = (1 - erf(z)) / 2 = q(t) exp(-x^2/2), q = t (a1/2 + ... ) (the 1/2
// folded into the coefficients):
//   GeLU(x)  = max(x, 0) - |x| tail                (x Phi(x) for either sign)
//   GeLU'(x) = Phi(x) + x phi(x),  Phi(x) = 1/2 + sign(x) (1/2 - tail),
//              phi(x) = exp(-x^2/2) / sqrt(2 pi)  (the same exponential).
// One reciprocal and one exp2 per element (hardware v_rcp_f32 / v_exp_f32).
// Tanh form: the GELU paper's approximation 0.5 x (1 + tanh(u)),
// u = sqrt(2/pi) (x + 0.044715 x^3), written as x * sigmoid(2u).
constexpr float kAsP = 0.3275911f;
constexpr float kAsH1 = 0.5f * 0.254829592f, kAsH2 = 0.5f * -0.284496736f, kAsH3 = 0.5f * 1.421413741f,
                kAsH4 = 0.5f * -1.453152027f, kAsH5 = 0.5f * 1.061405429f;

struct ErfTail {
  float tail;  // (1 - erf(|x|/sqrt 2)) / 2
  float e;     // exp(-x^2/2)
};

__device__ __forceinline__ ErfTail erf_tail(float x) {
  const float z = fabsf(x) * kInvSqrt2;
  const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(kAsP, z, 1.0f));
  const float q = t * __builtin_fmaf(t, __builtin_fmaf(t, __builtin_fmaf(t, __builtin_fmaf(t, kAsH5, kAsH4), kAsH3), kAsH2), kAsH1);
  const float e = __builtin_amdgcn_exp2f(z * z * -kLog2e);  // exp(-z^2) = exp(-x^2/2)
  return ErfTail{q * e, e};
}

template <int FORM>
__device__ __forceinline__ float gelu_f(float x) {
  if constexpr (FORM == kGeluErf) {
    const ErfTail r = erf_tail(x);
    return __builtin_fmaf(-fabsf(x), r.tail, fmaxf(x, 0.0f));
  } else {
    const float u2 = 2.0f * kSqrt2OverPi * x * __builtin_fmaf(kTanhC * x, x, 1.0f);
    return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u2 * kLog2e));
  }
}

template <int FORM>
__device__ __forceinline__ float gelu_grad_f(float x) {
  if constexpr (FORM == kGeluErf) {
    const ErfTail r = erf_tail(x);
    const float phi_cdf = 0.5f + __builtin_copysignf(0.5f - r.tail, x);
    return __builtin_fmaf(x * kInvSqrt2Pi, r.e, phi_cdf);
  } else {
    // d/dx [x s(2u)] = s + x s (1 - s) 2u',  s = sigmoid(2u),  u' = sqrt(2/pi)(1 + 3c x^2)
    const float u2 = 2.0f * kSqrt2OverPi * x * __builtin_fmaf(kTanhC * x, x, 1.0f);
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-u2 * kLog2e));
    const float du2 = 2.0f * kSqrt2OverPi * __builtin_fmaf(3.0f * kTanhC * x, x, 1.0f);
    return __builtin_fmaf(x * sg * (1.0f - sg), du2, sg);
  }
}

// ---------------------------------------------------------------------------
// LDS hand-over of the accumulators

// Each wave stages 64 rows of its sub-tile at a time: 64 x kWaveN fp32 in a
// private region of the four LDS stages.
constexpr int kEpiRows = 64;
constexpr int kWavesPerStage = kWaves / 4;
static_assert(kEpiRows * kWaveN * 4 * kWavesPerStage <= kStageBytes, "staging regions fit the LDS stages");
// The row-major read-back: kLanesPerRow lanes (4 values each) cover one row of
// the sub-tile, so one read instruction covers kRowsPerRead rows.
constexpr int kLanesPerRow = kWaveN / 4;
constexpr int kRowsPerRead = 64 / kLanesPerRow;

__device__ __forceinline__ char* epi_region(const EpiCtx& c) {
  const int wave = c.wm * kWavesN + c.wn;
  const int st = wave / kWavesPerStage;
  char* base = st == 0 ? c.lds0 : (st == 1 ? c.lds1 : (st == 2 ? c.lds2 : c.lds3));
  return base + (wave % kWavesPerStage) * (kEpiRows * kWaveN * 4);
}

// Row pitch kWaveN * 4 bytes; chunk q of row lr at slot q ^ (lr & 15).
__device__ __forceinline__ int epi_slot(int lr, int q) { return lr * (kWaveN * 4) + ((q ^ (lr & 15)) << 4); }

// Write rows [64h, 64h + 64) of the wave's sub-tile (row blocks mi = 4h .. 4h+3).
static_assert(kWaveM == 128, "the sub-tile is staged in two halves of 64 rows");
__device__ __forceinline__ void epi_stage_half(const AccTile& acc, char* region, int h, int lane) {
  if (h == 0) acc_settle();
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4) {
    const int lr = m4 * 16 + (lane & 15);
#pragma unroll
    for (int ni = 0; ni < kSubN; ++ni) acc_store_lds(region + epi_slot(lr, ni * 4 + (lane >> 4)), acc[4 * h + m4][ni]);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

// Local row lr (0..63) of the staged half, columns 4q .. 4q+3 (q < kLanesPerRow).
__device__ __forceinline__ f32x4_t epi_read(const char* region, int lr, int q) {
  return *(const f32x4_t*)(region + epi_slot(lr, q));
}

// Row-major walk of the staged sub-tile: calls f(row, col, v) with tile-local
// row/col of 4 consecutive values; kLanesPerRow lanes cover one row.  Reads
// are taken 4 at a time with their LDS reads issued together, so the read
// latency is paid once per group.
template <class F>
__device__ __forceinline__ void epi_rows(const AccTile& acc, const EpiCtx& c, F&& f) {
  char* region = epi_region(c);
  const int q = c.lane % kLanesPerRow, sub = c.lane / kLanesPerRow;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    epi_stage_half(acc, region, h, c.lane);  // h must be a constant: acc is indexed by it
#pragma unroll 1
    for (int it0 = 0; it0 < kEpiRows / kRowsPerRead; it0 += 4) {
      f32x4_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = epi_read(region, (it0 + u) * kRowsPerRead + sub, q);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int lr = (it0 + u) * kRowsPerRead + sub;
        f(c.wm * kWaveM + h * 64 + lr, c.wn * kWaveN + q * 4, v[u]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------

// fp32 store of C (optionally into split slice `split` of a workspace).
struct EpiStoreF32 {
  float* C;
  int64_t ld;
  int M, N;
  int64_t split_stride;  // elements between split slices (0 when splits == 1)
  __device__ void operator()(AccTile& acc, const EpiCtx& c) const {
    const int64_t base = (int64_t)c.split * split_stride + (int64_t)c.m0 * ld + c.n0;
    const rsrc_t rs = make_rsrc(C + base, ((int64_t)c.split * split_stride + (int64_t)M * ld - base) * 4);
    const int mrem = M - c.m0, nrem = N - c.n0;
    epi_rows(acc, c, [&](int rl, int cl, f32x4_t v) {
      const bool ok = rl < mrem && cl < nrem;
      buf_store16<kNonTemporal>(__builtin_bit_cast(u32x4_t, v), rs, ok ? (uint32_t)(((int64_t)rl * ld + cl) * 4) : kOOB);
    });
  }
};

// bf16 store of C (store cache policy POLICY; the call operator: the default).
struct EpiStoreBF16 {
  uint16_t* C;
  int64_t ld;
  int M, N;
  template <int POLICY>
  __device__ void store(AccTile& acc, const EpiCtx& c) const {
    const int64_t base = (int64_t)c.m0 * ld + c.n0;
    const rsrc_t rs = make_rsrc(C + base, ((int64_t)M * ld - base) * 2);
    const int mrem = M - c.m0, nrem = N - c.n0;
    epi_rows(acc, c, [&](int rl, int cl, f32x4_t v) {
      const bool ok = rl < mrem && cl < nrem;
      buf_store8<POLICY>(u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}, rs,
                         ok ? (uint32_t)(((int64_t)rl * ld + cl) * 2) : kOOB);
    });
  }
  __device__ void operator()(AccTile& acc, const EpiCtx& c) const { store<0>(acc, c); }
};

// Weight-gradient store for the paired launches: the bf16 result when the
// contraction is not split (slice_stride == 0), else this split's fp32 slice
// of the workspace (summed in fixed order by the split-K reduction).
struct EpiStoreWGrad {
  void* C;
  int64_t ld;
  int M, N;
  int64_t slice_stride;  // elements between fp32 slices; 0: bf16 output
  __device__ void operator()(AccTile& acc, const EpiCtx& c) const {
    if (slice_stride == 0) {
      EpiStoreBF16{(uint16_t*)C, ld, M, N}.store<kNonTemporal>(acc, c);
    } else {
      EpiStoreF32{(float*)C, ld, M, N, slice_stride}(acc, c);
    }
  }
};

// Forward column-parallel epilogue: H = acc (+ b1), Y = GeLU(H) from the fp32
// value; both stored as bf16.
template <int FORM>
struct EpiGeluFwd {
  uint16_t* H;
  uint16_t* Y;
  const uint16_t* b1;  // may be null: its resource is then empty and reads give 0
  int64_t ld;
  int M, N;
  __device__ void operator()(AccTile& acc, const EpiCtx& c) const {
    const int64_t base = (int64_t)c.m0 * ld + c.n0;
    const int64_t bytes = ((int64_t)M * ld - base) * 2;
    const rsrc_t rh = make_rsrc(H + base, bytes);
    const rsrc_t ry = make_rsrc(Y + base, bytes);
    const int mrem = M - c.m0, nrem = N - c.n0;
    // this lane always owns the same 4 columns: load their bias once
    const int col = c.n0 + c.wn * kWaveN + (c.lane % kLanesPerRow) * 4;
    const rsrc_t rb = make_rsrc(b1, b1 ? (int64_t)N * 2 : 0);
    const u32x2_t bb = buf_load8(rb, col < N ? (uint32_t)col * 2u : kOOB);
    const float bv[4] = {bf16_lo(bb[0]), bf16_hi(bb[0]), bf16_lo(bb[1]), bf16_hi(bb[1])};
    // without a bias the pre-activation is the accumulator itself (no addition)
    auto body = [&](auto with_bias) {
      epi_rows(acc, c, [&](int rl, int cl, f32x4_t v) {
        const bool ok = rl < mrem && cl < nrem;
        const uint32_t off = ok ? (uint32_t)(((int64_t)rl * ld + cl) * 2) : kOOB;
        float hv[4], yv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          hv[r] = decltype(with_bias)::value ? v[r] + bv[r] : v[r];
          yv[r] = gelu_f<FORM>(hv[r]);
        }
        buf_store8(u32x2_t{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])}, rh, off);
        buf_store8(u32x2_t{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])}, ry, off);
      });
    };
    if (b1) body(std::true_type{});
    else body(std::false_type{});
  }
};

// Backward epilogue of dY = dZ B_i^T: dH = dY * GeLU'(H) stored as bf16.  If
// db1_part is set, also writes this wave's column sums of the fp32 dH over its
// 128 rows to db1_part[(tile_m*kWavesM + wm) * N + col] (one private slot per
// writer).
template <int FORM>
struct EpiDGelu {
  const uint16_t* H;
  uint16_t* dH;
  float* db1_part;
  int64_t ld;
  int M, N;
  __device__ void operator()(AccTile& acc, const EpiCtx& c) const {
    const int64_t base = (int64_t)c.m0 * ld + c.n0;
    const int64_t bytes = ((int64_t)M * ld - base) * 2;
    const rsrc_t rh = make_rsrc(H + base, bytes);
    const rsrc_t rd = make_rsrc(dH + base, bytes);
    const int mrem = M - c.m0, nrem = N - c.n0;
    char* region = epi_region(c);
    const int q = c.lane % kLanesPerRow, sub = c.lane / kLanesPerRow;
    const int cl = c.wn * kWaveN + q * 4;
    constexpr int kIters = kEpiRows / kRowsPerRead;  // read instructions per staged half
    float csum[4] = {0.f, 0.f, 0.f, 0.f};
    // compile-time paths: column sums only with a bias gradient to form, and no
    // per-row bounds tests for tiles wholly inside the matrix
    auto body = [&](auto with_db1, auto interior) {
      constexpr bool kDb1 = decltype(with_db1)::value, kInterior = decltype(interior)::value;
      auto in = [&](int rl) { return kInterior || (rl < mrem && cl < nrem); };
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        epi_stage_half(acc, region, h, c.lane);  // h must be a constant: acc is indexed by it
        // H of 8 reads per batch; the next batch's loads are issued before the
        // current batch is processed, so their latency overlaps the arithmetic
        auto load_h = [&](int it0, u32x2_t (&hh)[8]) {
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int rl = c.wm * kWaveM + h * 64 + (it0 + u) * kRowsPerRead + sub;
            hh[u] = buf_load8<kNonTemporal>(rh, in(rl) ? (uint32_t)(((int64_t)rl * ld + cl) * 2) : kOOB);
          }
        };
        u32x2_t hcur[8], hnext[8];
        load_h(0, hcur);
#pragma unroll 2
        for (int it0 = 0; it0 < kIters; it0 += 8) {
          if (it0 + 8 < kIters) load_h(it0 + 8, hnext);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int lr = (it0 + u) * kRowsPerRead + sub;
            const int rl = c.wm * kWaveM + h * 64 + lr;
            const bool ok = in(rl);
            const f32x4_t v = epi_read(region, lr, q);
            const float hv[4] = {bf16_lo(hcur[u][0]), bf16_hi(hcur[u][0]), bf16_lo(hcur[u][1]),
                                 bf16_hi(hcur[u][1])};
            float dv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              dv[r] = v[r] * gelu_grad_f<FORM>(hv[r]);
              if constexpr (!kInterior) dv[r] = ok ? dv[r] : 0.0f;
              if constexpr (kDb1) csum[r] += dv[r];
            }
            buf_store8(u32x2_t{pack_bf16x2(dv[0], dv[1]), pack_bf16x2(dv[2], dv[3])}, rd,
                       ok ? (uint32_t)(((int64_t)rl * ld + cl) * 2) : kOOB);
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) hcur[u] = hnext[u];
        }
        __builtin_amdgcn_wave_barrier();
      }
    };
    const bool interior = mrem >= kBM && nrem >= kBN;
    if (db1_part) {
      if (interior) body(std::true_type{}, std::true_type{});
      else body(std::true_type{}, std::false_type{});
    } else {
      if (interior) body(std::false_type{}, std::true_type{});
      else body(std::false_type{}, std::false_type{});
    }
    if (db1_part) {
      // the lanes holding the same columns (sub = 0 .. kRowsPerRead-1) add their
      // sums pairwise; each addition is commutative, so every lane of a group
      // ends with the same bits
#pragma unroll
      for (int x = kLanesPerRow; x < 64; x *= 2)
#pragma unroll
        for (int r = 0; r < 4; ++r) csum[r] += __shfl_xor(csum[r], x, 64);
      if (sub == 0 && cl < nrem) {
        const int64_t slot = (int64_t)(c.tm * kWavesM + c.wm) * N + c.n0 + cl;
        *(f32x4_t*)(db1_part + slot) = f32x4_t{csum[0], csum[1], csum[2], csum[3]};
      }
    }
  }
};

// Fused cross-entropy epilogue of the logits GEMM L = X E_i.  Per token row of
// the tile, computes over the tile's valid columns
//   pm = max L,  ps = sum exp(L - pm),  pz = L at the target column if it lies
//   in this tile, else 0,
// straight from the accumulators.  Lane l holds 4*kSubN columns of each of
// its kSubM rows and 4 lanes (l, l^16, l^32, l^48) share a row: each lane
// reduces its values to (max, sum of exp(L - max)), then the four are merged
// by log-sum-exp over two lane-pair exchanges (v_permlane16_swap, then
// v_permlane32_swap).  Each exchange hands every lane the pair's two values
// in the same order, so all four lanes end with bitwise-equal results.  The
// kWavesN column-waves of each row are merged in LDS in fixed order (wn = 0,
// 1, ...) and the triple goes to partial slot tile_n of arrays laid out
// [tiles_n][T].
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// One accumulator copied to an ordinary register at this point of the program.
// The copy is an asm statement, so the compiler neither hoists nor merges it:
// the CE epilogue then holds one 16-row block's values at a time instead of
// all of them (which left no registers and spilled).
__device__ __forceinline__ float acc_read(float a) {
  float x;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(a));
  return x;
}

// Both lanes of each exchanged pair receive (value of the lower lane, value of the upper lane).
__device__ __forceinline__ void xswap16(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ void xswap32(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// Maximum of n values by a fixed tree of v_max3 (exact in any order).
template <int N>
__device__ __forceinline__ float max_tree(const float* v) {
  if constexpr (N == 1) return v[0];
  else if constexpr (N == 2) return fmaxf(v[0], v[1]);
  else if constexpr (N == 3) return max3f(v[0], v[1], v[2]);
  else {
    constexpr int a = (N + 2) / 3, b = (N - a + 1) / 2;
    return max3f(max_tree<a>(v), max_tree<b>(v + a), max_tree<N - a - b>(v + a + b));
  }
}

// Sum of n values by a fixed pairwise tree.
template <int N>
__device__ __forceinline__ float sum_tree(const float* v) {
  if constexpr (N == 1) return v[0];
  else return sum_tree<N / 2>(v) + sum_tree<N - N / 2>(v + N / 2);
}

// (m, s) pairs -> merged pair; m = -inf means an empty set (s = 0).
__device__ __forceinline__ void lse_pair(float ma, float sa, float mb, float sb, float& m, float& s) {
  m = fmaxf(ma, mb);
  const float ml = m == -INFINITY ? 0.f : m * kLog2e;
  s = sa * __builtin_amdgcn_exp2f(__builtin_fmaf(ma, kLog2e, -ml)) +
      sb * __builtin_amdgcn_exp2f(__builtin_fmaf(mb, kLog2e, -ml));
}

struct EpiCE {
  static constexpr bool kKeepsStages = true;  // uses only the exchange buffer, never the LDS stages
  // bytes of the small LDS buffer the column-waves' triples are merged through
  static constexpr int kXchBytes = (kWavesN - 1) * kBM * 3 * 4;
  const int64_t* target;
  int64_t vocab_start;
  float* part;  // pm at part, ps at part + stride, pz at part + 2*stride (floats)
  int stride;
  int M, N;     // M = T tokens, N = v_i
  int pad_;
  __device__ void operator()(AccTile& acc, const EpiCtx& c) const {
    const rsrc_t rt = make_rsrc(target, (int64_t)M * 8);
    const int l16 = c.lane & 15, g = c.lane >> 4;
    const int col0 = c.n0 + c.wn * kWaveN;                // first column of this wave
    const int ncol = min(N - col0, kWaveN);               // valid columns (may be <= 0)
    const int row0 = c.m0 + c.wm * kWaveM + l16;          // row of block mi is row0 + 16 mi
    u32x2_t tw[kSubM];
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) {
      const int row = row0 + mi * 16;
      tw[mi] = buf_load8(rt, row < M ? (uint32_t)row * 8u : kOOB);
    }
    acc_settle();
    // A 4-column group is entirely valid or entirely padding (N % 8 == 0);
    // padding is added as -inf, and waves with no padding take a branch without it.
    float rm[kSubM], rs[kSubM], rz[kSubM];
    auto rows = [&](auto masked) {
      constexpr bool kMasked = decltype(masked)::value;
      float pad[kSubN];
#pragma unroll
      for (int ni = 0; ni < kSubN; ++ni) pad[ni] = (!kMasked || ni * 16 + 4 * g < ncol) ? 0.f : -INFINITY;
#pragma unroll
      for (int mi = 0; mi < kSubM; ++mi) {
        float v[kSubN * 4];
#pragma unroll
        for (int ni = 0; ni < kSubN; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = acc_read(acc[mi][ni][r]);
            v[ni * 4 + r] = kMasked ? a + pad[ni] : a;
          }
        const float mx = max_tree<kSubN * 4>(v);
        const float ml = mx == -INFINITY ? 0.f : mx * kLog2e;  // no valid column: every term is 0
        float e[kSubN];
#pragma unroll
        for (int ni = 0; ni < kSubN; ++ni) {
          float q[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) q[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[ni * 4 + r], kLog2e, -ml));
          e[ni] = (q[0] + q[1]) + (q[2] + q[3]);
        }
        rm[mi] = mx;
        rs[mi] = sum_tree<kSubN>(e);
      }
    };
    if (ncol >= kWaveN) rows(std::false_type{});
    else rows(std::true_type{});
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) {
      float ma, mb, sa, sb;
      xswap16(rm[mi], ma, mb);
      xswap16(rs[mi], sa, sb);
      lse_pair(ma, sa, mb, sb, rm[mi], rs[mi]);
    }
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) {
      float ma, mb, sa, sb;
      xswap32(rm[mi], ma, mb);
      xswap32(rs[mi], sa, sb);
      lse_pair(ma, sa, mb, sb, rm[mi], rs[mi]);
    }
    // the target logit: searched only in the 16-row blocks that hold some
    // row's target in this wave's 128 columns (one block in 25 at v_i = 50304),
    // so waves do not wait at the barrier below for a search over all their
    // accumulators; at most one lane of a row's four holds it
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) {
      const int64_t t = (int64_t)(((uint64_t)tw[mi][1] << 32) | tw[mi][0]) - vocab_start - col0;
      const int tl = (t >= 0 && t < ncol) ? (int)t : -1;
      rz[mi] = 0.f;
      if (__any(tl >= 0)) {
        float zz = 0.f;
#pragma unroll
        for (int ni = 0; ni < kSubN; ++ni)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = acc_read(acc[mi][ni][r]);
            zz = (ni * 16 + 4 * g + r) == tl ? x : zz;
          }
        float za, zb;
        xswap16(zz, za, zb);
        zz = za + zb;
        xswap32(zz, za, zb);
        rz[mi] = za + zb;
      }
    }
    // merge the column-waves of each row: waves wn >= 1 hand their triples to
    // wn = 0 through the exchange buffer, which merges them in ascending wn
    float* xch = (float*)c.xch;  // [wn - 1][kBM rows][3]
    if (c.wn > 0 && g == 0) {
#pragma unroll
      for (int mi = 0; mi < kSubM; ++mi) {
        float* e = xch + ((c.wn - 1) * kBM + c.wm * kWaveM + mi * 16 + l16) * 3;
        e[0] = rm[mi];
        e[1] = rs[mi];
        e[2] = rz[mi];
      }
    }
    __syncthreads();
    if (c.wn == 0 && g == 0) {
#pragma unroll
      for (int mi = 0; mi < kSubM; ++mi) {
        const int row = row0 + mi * 16;
        if (row < M) {
          float mm = rm[mi], ss = rs[mi], zz = rz[mi];
#pragma unroll
          for (int w = 1; w < kWavesN; ++w) {
            const float* e = xch + ((w - 1) * kBM + c.wm * kWaveM + mi * 16 + l16) * 3;
            float m2, s2;
            lse_pair(mm, ss, e[0], e[1], m2, s2);
            mm = m2;
            ss = s2;
            zz += e[2];
          }
          float* o = part + (int64_t)c.tn * M + row;
          o[0] = mm;
          o[stride] = ss;
          o[2 * (int64_t)stride] = zz;
        }
      }
    }
  }
};

// Cross-entropy backward epilogue of the recomputed logits L = X E_i: the
// logit gradient of sum_t coef_t loss_t,
//   dL[t, j] = coef_t (exp(L[t, j] - M_t) / S_t - [j is y_t's shard column])
//            = exp2(L log2 e - M_t log2 e) (coef_t / S_t) - [j is the target] coef_t,
// stored as bf16.  (M_t, S_t) are the token's statistics over the whole
// vocabulary, so the softmax is the global one.  Each token has a 16-byte
// record {M log2 e, coef / S, coef, target column in this shard or -1 (int
// bits)}; the rows are walked like EpiDGelu's, with the next 8 rows' records
// loaded while the current 8 are computed.
struct EpiCEGrad {
  const f32x4_t* stats;  // [M] records
  uint16_t* dL;
  int64_t ld;
  int M, N;
  __device__ void operator()(AccTile& acc, const EpiCtx& c) const {
    const int64_t base = (int64_t)c.m0 * ld + c.n0;
    const rsrc_t rd = make_rsrc(dL + base, ((int64_t)M * ld - base) * 2);
    const rsrc_t rs = make_rsrc(stats + c.m0, (int64_t)(M - c.m0) * 16);
    const int mrem = M - c.m0, nrem = N - c.n0;
    char* region = epi_region(c);
    const int q = c.lane % kLanesPerRow, sub = c.lane / kLanesPerRow;
    const int cl = c.wn * kWaveN + q * 4;
    const int col = c.n0 + cl;  // shard column of this lane's first value
    constexpr int kIters = kEpiRows / kRowsPerRead;  // read instructions per staged half
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      epi_stage_half(acc, region, h, c.lane);  // h must be a constant: acc is indexed by it
      auto load_s = [&](int it0, u32x4_t (&ss)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int rl = c.wm * kWaveM + h * 64 + (it0 + u) * kRowsPerRead + sub;
          ss[u] = buf_load16(rs, rl < mrem ? (uint32_t)rl * 16u : kOOB);
        }
      };
      u32x4_t scur[8], snext[8];
      load_s(0, scur);
#pragma unroll 2
      for (int it0 = 0; it0 < kIters; it0 += 8) {
        if (it0 + 8 < kIters) load_s(it0 + 8, snext);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int lr = (it0 + u) * kRowsPerRead + sub;
          const int rl = c.wm * kWaveM + h * 64 + lr;
          const bool ok = rl < mrem && cl < nrem;
          const f32x4_t v = epi_read(region, lr, q);
          const float ml = __uint_as_float(scur[u][0]);
          const float cs = __uint_as_float(scur[u][1]);
          const float cf = __uint_as_float(scur[u][2]);
          const int tcol = (int)scur[u][3];
          float d[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(v[r], kLog2e, -ml));
            d[r] = __builtin_fmaf(e, cs, col + r == tcol ? -cf : 0.0f);
          }
          buf_store8<kNonTemporal>(u32x2_t{pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3])}, rd,
                                   ok ? (uint32_t)(((int64_t)rl * ld + cl) * 2) : kOOB);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) scur[u] = snext[u];
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
};

}  // namespace mshard
