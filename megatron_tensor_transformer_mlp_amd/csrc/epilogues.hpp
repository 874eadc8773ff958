// epilogues.hpp - what each GEMM does with its fp32 accumulators.
//
// Accumulator element acc[mi][ni][r] of wave (wm, wn) in the tile at (m0, n0)
// is C[m0 + wm*128 + mi*16 + (lane & 15)][n0 + wn*128 + ni*16 + (lane >> 4)*4 + r].
// N is a multiple of 8, so each lane's 4-column group is entirely inside or
// entirely outside the matrix; rows are masked one by one.
#pragma once

#include "gemm_core.hpp"

namespace mshard {

enum GeluForm { kGeluErf = 0, kGeluTanh = 1 };

constexpr float kInvSqrt2 = 0.70710678118654752440f;
constexpr float kInvSqrt2Pi = 0.39894228040143267794f;
constexpr float kSqrt2OverPi = 0.79788456080286535588f;
constexpr float kTanhC = 0.044715f;
constexpr float kLog2e = 1.44269504088896340736f;

// GeLU and its derivative in fp32.  Erf form: x*Phi(x) with Phi from erff;
// tanh form: the GELU paper's approximation 0.5x(1 + tanh(sqrt(2/pi)(x + c x^3))).
template <int FORM>
__device__ __forceinline__ float gelu_f(float x) {
  if constexpr (FORM == kGeluErf) {
    return 0.5f * x * (1.0f + erff(x * kInvSqrt2));
  } else {
    const float u = kSqrt2OverPi * x * (1.0f + kTanhC * x * x);
    return 0.5f * x * (1.0f + tanhf(u));
  }
}

template <int FORM>
__device__ __forceinline__ float gelu_grad_f(float x) {
  if constexpr (FORM == kGeluErf) {
    const float cdf = 0.5f * (1.0f + erff(x * kInvSqrt2));
    const float pdf = kInvSqrt2Pi * expf(-0.5f * x * x);
    return cdf + x * pdf;
  } else {
    const float u = kSqrt2OverPi * x * (1.0f + kTanhC * x * x);
    const float th = tanhf(u);
    const float du = kSqrt2OverPi * (1.0f + 3.0f * kTanhC * x * x);
    return 0.5f * (1.0f + th) + 0.5f * x * (1.0f - th * th) * du;
  }
}

__device__ __forceinline__ int epi_row(const EpiCtx& c, int mi) { return c.wm * kWaveM + mi * 16 + (c.lane & 15); }
__device__ __forceinline__ int epi_col(const EpiCtx& c, int ni) { return c.wn * kWaveN + ni * 16 + (c.lane >> 4) * 4; }

// fp32 store of C (optionally into split slice `split` of a workspace).
struct EpiStoreF32 {
  float* C;
  int64_t ld;
  int M, N;
  int64_t split_stride;  // elements between split slices (0 when splits == 1)
  __device__ void operator()(f32x4_t (&acc)[kSubM][kSubN], const EpiCtx& c) const {
    const int64_t base = (int64_t)c.split * split_stride + (int64_t)c.m0 * ld + c.n0;
    const rsrc_t rs = make_rsrc(C + base, ((int64_t)c.split * split_stride + (int64_t)M * ld - base) * 4);
#pragma unroll
    for (int ni = 0; ni < kSubN; ++ni) {
      const int cl = epi_col(c, ni);
      const bool cok = c.n0 + cl < N;
#pragma unroll
      for (int mi = 0; mi < kSubM; ++mi) {
        const int rl = epi_row(c, mi);
        const bool ok = cok && (c.m0 + rl) < M;
        const uint32_t off = ok ? (uint32_t)(((int64_t)rl * ld + cl) * 4) : kOOB;
        buf_store16(__builtin_bit_cast(u32x4_t, acc[mi][ni]), rs, off);
      }
    }
  }
};

// bf16 store of C.
struct EpiStoreBF16 {
  uint16_t* C;
  int64_t ld;
  int M, N;
  __device__ void operator()(f32x4_t (&acc)[kSubM][kSubN], const EpiCtx& c) const {
    const int64_t base = (int64_t)c.m0 * ld + c.n0;
    const rsrc_t rs = make_rsrc(C + base, ((int64_t)M * ld - base) * 2);
#pragma unroll
    for (int ni = 0; ni < kSubN; ++ni) {
      const int cl = epi_col(c, ni);
      const bool cok = c.n0 + cl < N;
#pragma unroll
      for (int mi = 0; mi < kSubM; ++mi) {
        const int rl = epi_row(c, mi);
        const bool ok = cok && (c.m0 + rl) < M;
        const uint32_t off = ok ? (uint32_t)(((int64_t)rl * ld + cl) * 2) : kOOB;
        const f32x4_t v = acc[mi][ni];
        buf_store8(u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}, rs, off);
      }
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
  __device__ void operator()(f32x4_t (&acc)[kSubM][kSubN], const EpiCtx& c) const {
    const int64_t base = (int64_t)c.m0 * ld + c.n0;
    const int64_t bytes = ((int64_t)M * ld - base) * 2;
    const rsrc_t rh = make_rsrc(H + base, bytes);
    const rsrc_t ry = make_rsrc(Y + base, bytes);
    const rsrc_t rb = make_rsrc(b1, b1 ? (int64_t)N * 2 : 0);
#pragma unroll
    for (int ni = 0; ni < kSubN; ++ni) {
      const int cl = epi_col(c, ni);
      const bool cok = c.n0 + cl < N;
      const u32x2_t bb = buf_load8(rb, cok ? (uint32_t)((c.n0 + cl) * 2) : kOOB);
      const float bias[4] = {bf16_lo(bb[0]), bf16_hi(bb[0]), bf16_lo(bb[1]), bf16_hi(bb[1])};
#pragma unroll
      for (int mi = 0; mi < kSubM; ++mi) {
        const int rl = epi_row(c, mi);
        const bool ok = cok && (c.m0 + rl) < M;
        const uint32_t off = ok ? (uint32_t)(((int64_t)rl * ld + cl) * 2) : kOOB;
        float hv[4], yv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          hv[r] = acc[mi][ni][r] + bias[r];
          yv[r] = gelu_f<FORM>(hv[r]);
        }
        buf_store8(u32x2_t{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])}, rh, off);
        buf_store8(u32x2_t{pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3])}, ry, off);
      }
    }
  }
};

// Backward epilogue of dY = dZ B_i^T: dH = dY * GeLU'(H) stored as bf16.  If
// db1_part is set, also writes this wave's column sums of the fp32 dH over its
// 128 rows to db1_part[(tile_m*2 + wm) * N + col] (one private slot per writer).
template <int FORM>
struct EpiDGelu {
  const uint16_t* H;
  uint16_t* dH;
  float* db1_part;
  int64_t ld;
  int M, N;
  __device__ void operator()(f32x4_t (&acc)[kSubM][kSubN], const EpiCtx& c) const {
    const int64_t base = (int64_t)c.m0 * ld + c.n0;
    const int64_t bytes = ((int64_t)M * ld - base) * 2;
    const rsrc_t rh = make_rsrc(H + base, bytes);
    const rsrc_t rd = make_rsrc(dH + base, bytes);
#pragma unroll
    for (int ni = 0; ni < kSubN; ++ni) {
      const int cl = epi_col(c, ni);
      const bool cok = c.n0 + cl < N;
      float csum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mi = 0; mi < kSubM; ++mi) {
        const int rl = epi_row(c, mi);
        const bool ok = cok && (c.m0 + rl) < M;
        const uint32_t off = ok ? (uint32_t)(((int64_t)rl * ld + cl) * 2) : kOOB;
        const u32x2_t hh = buf_load8(rh, off);
        const float hv[4] = {bf16_lo(hh[0]), bf16_hi(hh[0]), bf16_lo(hh[1]), bf16_hi(hh[1])};
        float dv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dv[r] = ok ? acc[mi][ni][r] * gelu_grad_f<FORM>(hv[r]) : 0.0f;
          csum[r] += dv[r];
        }
        buf_store8(u32x2_t{pack_bf16x2(dv[0], dv[1]), pack_bf16x2(dv[2], dv[3])}, rd, off);
      }
      if (db1_part) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int sh = 1; sh < 16; sh <<= 1) csum[r] += __shfl_xor(csum[r], sh, 64);
        }
        if ((c.lane & 15) == 0 && cok) {
          const int64_t slot = (int64_t)(c.tm * 2 + c.wm) * N + c.n0 + cl;
          *(f32x4_t*)(db1_part + slot) = f32x4_t{csum[0], csum[1], csum[2], csum[3]};
        }
      }
    }
  }
};

// Fused cross-entropy epilogue of the logits GEMM L = X E_i.  Per token row and
// per wave (128 columns), writes the partial triple
//   pm = max over the wave's valid columns, ps = sum exp(L - pm),
//   pz = L at the target column if it lies in these columns, else 0
// to partial slot p = tile_n*2 + wn of arrays laid out [P][T].
struct EpiCE {
  const int64_t* target;
  int64_t vocab_start;
  float* pm;
  float* ps;
  float* pz;
  int M, N;  // M = T tokens, N = v_i
  __device__ void operator()(f32x4_t (&acc)[kSubM][kSubN], const EpiCtx& c) const {
    const int p = c.tn * 2 + c.wn;
    const rsrc_t rt = make_rsrc(target, (int64_t)M * 8);
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) {
      const int row = c.m0 + epi_row(c, mi);
      const bool rok = row < M;
      const u32x2_t tw = buf_load8(rt, rok ? (uint32_t)row * 8u : kOOB);
      const int64_t tgt = (int64_t)(((uint64_t)tw[1] << 32) | tw[0]) - vocab_start;
      float mx = -INFINITY;
#pragma unroll
      for (int ni = 0; ni < kSubN; ++ni) {
        const bool cok = c.n0 + epi_col(c, ni) < N;
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = cok ? fmaxf(mx, acc[mi][ni][r]) : mx;
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mxl = mx * kLog2e;
      float sm = 0.f, zz = 0.f;
#pragma unroll
      for (int ni = 0; ni < kSubN; ++ni) {
        const int col = c.n0 + epi_col(c, ni);
        const bool cok = col < N;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = acc[mi][ni][r];
          sm += cok ? __builtin_amdgcn_exp2f(__builtin_fmaf(v, kLog2e, -mxl)) : 0.f;
          zz = ((int64_t)(col + r) == tgt) ? v : zz;
        }
      }
      sm += __shfl_xor(sm, 16, 64);
      sm += __shfl_xor(sm, 32, 64);
      zz += __shfl_xor(zz, 16, 64);
      zz += __shfl_xor(zz, 32, 64);
      if ((c.lane >> 4) == 0 && rok) {
        const int64_t o = (int64_t)p * M + row;
        pm[o] = mx;
        ps[o] = sm;
        pz[o] = zz;
      }
    }
  }
};

}  // namespace mshard
