// attention.hip - the attention core of one rank's self-attention shard:
// per sequence and head, O = softmax(Q K^T / sqrt(d) + mask) V (Megatron-LM
// explainer, azimuth.plus, "attention", and paper notes, notes.yuuk.io,
// "self-attention block split": heads are independent, so each rank runs its
// own heads with no exchange; the per-head computation is the textbook scaled
// dot-product attention).
//
// Layout: Q, K, V are the column blocks of QKV [T x 3nd] (T = b*s rows,
// sequence-major; head j at columns j*d of each block), O is [T x nd] and the
// per-row log-sum-exp of the scaled scores is lse [n x T].
//
// Forward, one workgroup per (128 query rows, head, sequence), 4 waves of 32
// query rows.  Keys advance 64 at a time through LDS (K and V tiles, row-major
// with a 16-byte pad per row, double-buffered, staged through registers).
//   S = Q K^T: v_mfma_f32_16x16x32_bf16 with the K fragment first, so lane l
//     holds S[query l%16][key 4(l/16) + r] of each 16-key block; the four
//     lanes of a query row merge its max and sum over lanes l^16 and l^32.
//   Online softmax in base 2 (scores scaled by log2(e)/sqrt(d)).
//   O += P V: P stays in registers as the MFMA's second operand.  A lane's
//     8 keys of a 32-key step are {4g..4g+3, 16+4g..16+4g+3} (g = l/16), the
//     keys its S registers hold; the V fragment is gathered in the same key
//     order with two transposing LDS reads (ds_read_b64_tr_b16), so the
//     contraction pairs every key with itself.
#include <type_traits>

#include "epilogues.hpp"
#include "launch.hpp"

namespace mshard {

namespace {

constexpr int kAttnBM = 128;  // query rows per workgroup
constexpr int kAttnBN = 64;   // keys per step
constexpr float kLn2 = 0.69314718055994530942f;

typedef short s16x8_t __attribute__((ext_vector_type(8)));

// LDS tile of 64 rows x D columns (bf16), row pitch 2D + 16 bytes.
template <int D>
struct AttnTile {
  static constexpr int kPitch = 2 * D + 16;
  static constexpr int kBytes = kAttnBN * kPitch;
  static constexpr int kChunks = D / 8;             // 16-byte chunks per row
  static constexpr int kPerThread = 64 * kChunks / 256;  // = D / 32
};

// Registers staging one tile: chunk i = tid + 256u is row i / (D/8), chunk i % (D/8).
template <int D>
struct TileRegs {
  u32x4_t v[AttnTile<D>::kPerThread];
};

// Rows [row0, row0 + 64) of the column block at `base` (row stride ld elements);
// rows at or beyond `nrows` and columns at or beyond `dvalid` read as zero.
template <int D>
__device__ __forceinline__ void tile_gload(TileRegs<D>& t, const uint16_t* base, int64_t ld, int row0, int nrows,
                                           int dvalid, int tid) {
#pragma unroll
  for (int u = 0; u < AttnTile<D>::kPerThread; ++u) {
    const int i = tid + 256 * u;
    const int row = i / AttnTile<D>::kChunks, c = i % AttnTile<D>::kChunks;
    const bool ok = row0 + row < nrows && c * 8 < dvalid;
    t.v[u] = ok ? *(const u32x4_t*)(base + (int64_t)(row0 + row) * ld + c * 8) : u32x4_t{0u, 0u, 0u, 0u};
  }
}

template <int D>
__device__ __forceinline__ void tile_swrite(char* lds, const TileRegs<D>& t, int tid) {
#pragma unroll
  for (int u = 0; u < AttnTile<D>::kPerThread; ++u) {
    const int i = tid + 256 * u;
    const int row = i / AttnTile<D>::kChunks, c = i % AttnTile<D>::kChunks;
    *(u32x4_t*)(lds + row * AttnTile<D>::kPitch + c * 16) = t.v[u];
  }
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ bf16x8_t lds_read_b128(const char* p) { return as_bf16x8(*(const u32x4_t*)p); }

__device__ __forceinline__ s16x4_t lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(lds_char*)p);
}

__device__ __forceinline__ bf16x8_t concat_bf16(s16x4_t lo, s16x4_t hi) {
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x4_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Max and sum of a query row over its four lanes (l, l^16, l^32, l^48); every
// lane of the row ends with the same bits.
__device__ __forceinline__ float row_max4(float x) {
  float a, b;
  xswap16(x, a, b);
  x = fmaxf(a, b);
  xswap32(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float row_sum4(float x) {
  float a, b;
  xswap16(x, a, b);
  x = a + b;
  xswap32(x, a, b);
  return a + b;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) attn_fwd_kernel(AttnGeom g, const uint16_t* __restrict__ qkv,
                                                       uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int KD = D / 32, ND = D / 16;
  using Tile = AttnTile<D>;
  __shared__ __attribute__((aligned(16))) char kt[2][Tile::kBytes];
  __shared__ __attribute__((aligned(16))) char vt[2][Tile::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int q0 = blockIdx.x * kAttnBM, j = blockIdx.y, bi = blockIdx.z;
  const int64_t tok0 = (int64_t)bi * g.s;
  const int64_t ld = g.ld_qkv;
  const uint16_t* Qb = qkv + tok0 * ld + (int64_t)j * g.d;
  const uint16_t* Kb = Qb + (int64_t)g.n * g.d;
  const uint16_t* Vb = Qb + 2 * (int64_t)g.n * g.d;

  bf16x8_t qf[2][KD];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = q0 + 32 * w + 16 * rb + l16;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const int c = kk * 4 + g4;
      const bool ok = row < g.s && c * 8 < g.d;
      qf[rb][kk] = as_bf16x8(ok ? *(const u32x4_t*)(Qb + (int64_t)row * ld + c * 8) : u32x4_t{0u, 0u, 0u, 0u});
    }
  }
  f32x4_t o[2][ND];
  float m[2], l[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int nb = 0; nb < ND; ++nb) o[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const int kv_end = CAUSAL ? min(g.s, q0 + kAttnBM) : g.s;
  const int nkb = (kv_end + kAttnBN - 1) / kAttnBN;
  TileRegs<D> kr, vr;
  tile_gload<D>(kr, Kb, ld, 0, g.s, g.d, tid);
  tile_gload<D>(vr, Vb, ld, 0, g.s, g.d, tid);
  tile_swrite<D>(kt[0], kr, tid);
  tile_swrite<D>(vt[0], vr, tid);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) {  // next tile in flight while this one is consumed
      tile_gload<D>(kr, Kb, ld, (kb + 1) * kAttnBN, g.s, g.d, tid);
      tile_gload<D>(vr, Vb, ld, (kb + 1) * kAttnBN, g.s, g.d, tid);
    }
    const char* K = kt[cur];
    const char* V = vt[cur];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int q = q0 + 32 * w + 16 * rb + l16;  // this lane's query position
      f32x4_t sacc[4];
#pragma unroll
      for (int kb16 = 0; kb16 < 4; ++kb16) {
        sacc[kb16] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk)
          sacc[kb16] = mfma16(lds_read_b128(K + (kb16 * 16 + l16) * Tile::kPitch + (kk * 4 + g4) * 16), qf[rb][kk],
                              sacc[kb16]);
      }
      float t[4][4];
      float mx = -INFINITY;
#pragma unroll
      for (int kb16 = 0; kb16 < 4; ++kb16)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb * kAttnBN + kb16 * 16 + 4 * g4 + r;
          const bool valid = key < g.s && (!CAUSAL || key <= q);
          t[kb16][r] = valid ? sacc[kb16][r] * g.scale_log2 : -INFINITY;
          mx = fmaxf(mx, t[kb16][r]);
        }
      mx = row_max4(mx);
      const float mnew = fmaxf(m[rb], mx);
      const float msub = mnew == -INFINITY ? 0.f : mnew;
      const float corr = __builtin_amdgcn_exp2f(m[rb] - msub);
      float p[4][4];
      float ps = 0.f;
#pragma unroll
      for (int kb16 = 0; kb16 < 4; ++kb16)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[kb16][r] = __builtin_amdgcn_exp2f(t[kb16][r] - msub);
          ps += p[kb16][r];
        }
      ps = row_sum4(ps);
      l[rb] = l[rb] * corr + ps;
      m[rb] = mnew;
#pragma unroll
      for (int nb = 0; nb < ND; ++nb) o[rb][nb] *= corr;
      bf16x8_t pf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
        pf[c] = as_bf16x8(u32x4_t{pack_bf16x2(p[2 * c][0], p[2 * c][1]), pack_bf16x2(p[2 * c][2], p[2 * c][3]),
                                  pack_bf16x2(p[2 * c + 1][0], p[2 * c + 1][1]),
                                  pack_bf16x2(p[2 * c + 1][2], p[2 * c + 1][3])});
      // source lane 16G + s of a transposing read addresses key 4G + s/4 (+ 16 for the second half)
      // and columns 16nb + 4(s%4) .. +3
      const int vrow = 4 * g4 + (l16 >> 2), vcol = 4 * (l16 & 3);
#pragma unroll
      for (int nb = 0; nb < ND; ++nb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const s16x4_t lo = lds_read_tr(V + (32 * c + vrow) * Tile::kPitch + (16 * nb + vcol) * 2);
          const s16x4_t hi = lds_read_tr(V + (32 * c + 16 + vrow) * Tile::kPitch + (16 * nb + vcol) * 2);
          o[rb][nb] = mfma16(concat_bf16(lo, hi), pf[c], o[rb][nb]);
        }
    }
    if (more) {
      tile_swrite<D>(kt[cur ^ 1], kr, tid);
      tile_swrite<D>(vt[cur ^ 1], vr, tid);
    }
    __syncthreads();
  }
  const int64_t T = (int64_t)g.b * g.s;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int q = q0 + 32 * w + 16 * rb + l16;
    if (q >= g.s) continue;
    const float inv = l[rb] > 0.f ? 1.f / l[rb] : 0.f;
    uint16_t* orow = out + (tok0 + q) * (int64_t)g.ld_o + (int64_t)j * g.d;
#pragma unroll
    for (int nb = 0; nb < ND; ++nb) {
      const int col = 16 * nb + 4 * g4;
      if (col < g.d) {
        const f32x4_t v = o[rb][nb] * inv;
        *(u32x2_t*)(orow + col) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
    if (g4 == 0) lse[(int64_t)j * T + tok0 + q] = (m[rb] + __builtin_log2f(l[rb])) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_attn_fwd_t(const AttnGeom& g, const uint16_t* qkv, uint16_t* out, float* lse, hipStream_t st) {
  const dim3 grid((unsigned)((g.s + kAttnBM - 1) / kAttnBM), (unsigned)g.n, (unsigned)g.b);
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL>), grid, dim3(256), 0, st, g, qkv, out, lse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_attn_fwd_d(const AttnGeom& g, bool causal, const uint16_t* qkv, uint16_t* out, float* lse,
                             hipStream_t st) {
  return causal ? launch_attn_fwd_t<D, true>(g, qkv, out, lse, st) : launch_attn_fwd_t<D, false>(g, qkv, out, lse, st);
}

// Backward: delta[j][t] = sum over the head's columns of dO * O (fp32, in
// column order), the row term of dS = P * (dP - delta).
__global__ void __launch_bounds__(256) attn_bwd_delta(AttnGeom g, const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dout, float* __restrict__ delta) {
  const int64_t T = (int64_t)g.b * g.s;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * g.n) return;
  const int j = (int)(i / T);
  const int64_t t = i - (int64_t)j * T;
  const uint16_t* a = o + t * g.ld_o + (int64_t)j * g.d;
  const uint16_t* b = dout + t * g.ld_o + (int64_t)j * g.d;
  float acc = 0.f;
  for (int c = 0; c < g.d; c += 8) {
    const u32x4_t x = *(const u32x4_t*)(a + c), y = *(const u32x4_t*)(b + c);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc += bf16_lo(x[k]) * bf16_lo(y[k]);
      acc += bf16_hi(x[k]) * bf16_hi(y[k]);
    }
  }
  delta[(int64_t)j * T + t] = acc;
}

// Backward, dK and dV: one workgroup per (64 keys, head, sequence); wave w owns
// keys k0 + 16w .. +15 and loops over the query blocks that see them (64
// queries per step, through LDS: the Q and dO tiles plus each query's lse
// and delta).  With the Q fragment as the MFMA's first operand, lane l holds
// S[query 4(l/16) + r][key l%16] of each 16-query block: the transposed
// layout, so P^T and dS^T stay in registers as the second operand of
//   dV += P^T dO  and  dK += dS^T Q,
// whose first operands (dO and Q gathered per column) come from transposing
// LDS reads, and dP^T = V dO^T takes the wave's V rows from registers.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) attn_bwd_dkdv_kernel(AttnGeom g, const uint16_t* __restrict__ qkv,
                                                            const uint16_t* __restrict__ dout,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ delta,
                                                            uint16_t* __restrict__ dqkv) {
  constexpr int KD = D / 32, ND = D / 16;
  using Tile = AttnTile<D>;
  __shared__ __attribute__((aligned(16))) char qt[2][Tile::kBytes];
  __shared__ __attribute__((aligned(16))) char dt[2][Tile::kBytes];
  __shared__ float sl[2][kAttnBN], sd[2][kAttnBN];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int k0 = blockIdx.x * kAttnBN, j = blockIdx.y, bi = blockIdx.z;
  const int64_t tok0 = (int64_t)bi * g.s, T = (int64_t)g.b * g.s;
  const int64_t ld = g.ld_qkv;
  const uint16_t* Qb = qkv + tok0 * ld + (int64_t)j * g.d;
  const uint16_t* Kb = Qb + (int64_t)g.n * g.d;
  const uint16_t* Vb = Qb + 2 * (int64_t)g.n * g.d;
  const uint16_t* dOb = dout + tok0 * (int64_t)g.ld_o + (int64_t)j * g.d;
  const float* lseb = lse + (int64_t)j * T + tok0;
  const float* delb = delta + (int64_t)j * T + tok0;
  const int key = k0 + 16 * w + l16;  // this lane's key row
  bf16x8_t kf[KD], vf[KD];
#pragma unroll
  for (int kk = 0; kk < KD; ++kk) {
    const int c = kk * 4 + g4;
    const bool ok = key < g.s && c * 8 < g.d;
    kf[kk] = as_bf16x8(ok ? *(const u32x4_t*)(Kb + (int64_t)key * ld + c * 8) : u32x4_t{0u, 0u, 0u, 0u});
    vf[kk] = as_bf16x8(ok ? *(const u32x4_t*)(Vb + (int64_t)key * ld + c * 8) : u32x4_t{0u, 0u, 0u, 0u});
  }
  f32x4_t dk[ND], dv[ND];
#pragma unroll
  for (int nb = 0; nb < ND; ++nb) dk[nb] = dv[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int qstart = CAUSAL ? k0 : 0;  // causal: only queries at or after the block's first key
  const int nqb = qstart < g.s ? (g.s - qstart + kAttnBN - 1) / kAttnBN : 0;
  TileRegs<D> qr, dr;
  float lr = 0.f, dl = 0.f;
  auto gload = [&](int qb) {
    const int r0 = qstart + qb * kAttnBN;
    tile_gload<D>(qr, Qb, ld, r0, g.s, g.d, tid);
    tile_gload<D>(dr, dOb, g.ld_o, r0, g.s, g.d, tid);
    if (tid < kAttnBN) lr = r0 + tid < g.s ? lseb[r0 + tid] * kLog2e : 0.f;
    else if (tid < 2 * kAttnBN) dl = r0 + tid - kAttnBN < g.s ? delb[r0 + tid - kAttnBN] : 0.f;
  };
  auto swrite = [&](int buf) {
    tile_swrite<D>(qt[buf], qr, tid);
    tile_swrite<D>(dt[buf], dr, tid);
    if (tid < kAttnBN) sl[buf][tid] = lr;
    else if (tid < 2 * kAttnBN) sd[buf][tid - kAttnBN] = dl;
  };
  if (nqb > 0) {
    gload(0);
    swrite(0);
  }
  __syncthreads();
  const int vrow = 4 * g4 + (l16 >> 2), vcol = 4 * (l16 & 3);
  for (int qb = 0; qb < nqb; ++qb) {
    const int cur = qb & 1;
    const bool more = qb + 1 < nqb;
    if (more) gload(qb + 1);
    const char* Q = qt[cur];
    const char* dO = dt[cur];
    const int qbase = qstart + qb * kAttnBN;
    float p[4][4], ds[4][4];
#pragma unroll
    for (int qb16 = 0; qb16 < 4; ++qb16) {
      f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f}, dpacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        const int off = (qb16 * 16 + l16) * Tile::kPitch + (kk * 4 + g4) * 16;
        sacc = mfma16(lds_read_b128(Q + off), kf[kk], sacc);
        dpacc = mfma16(lds_read_b128(dO + off), vf[kk], dpacc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ql = qb16 * 16 + 4 * g4 + r;  // query within the block
        const int q = qbase + ql;
        const bool valid = q < g.s && key < g.s && (!CAUSAL || key <= q);
        p[qb16][r] = valid ? __builtin_amdgcn_exp2f(sacc[r] * g.scale_log2 - sl[cur][ql]) : 0.f;
        ds[qb16][r] = p[qb16][r] * (dpacc[r] - sd[cur][ql]);
      }
    }
    bf16x8_t pf[2], dsf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      pf[c] = as_bf16x8(u32x4_t{pack_bf16x2(p[2 * c][0], p[2 * c][1]), pack_bf16x2(p[2 * c][2], p[2 * c][3]),
                                pack_bf16x2(p[2 * c + 1][0], p[2 * c + 1][1]),
                                pack_bf16x2(p[2 * c + 1][2], p[2 * c + 1][3])});
      dsf[c] = as_bf16x8(u32x4_t{pack_bf16x2(ds[2 * c][0], ds[2 * c][1]), pack_bf16x2(ds[2 * c][2], ds[2 * c][3]),
                                 pack_bf16x2(ds[2 * c + 1][0], ds[2 * c + 1][1]),
                                 pack_bf16x2(ds[2 * c + 1][2], ds[2 * c + 1][3])});
    }
#pragma unroll
    for (int nb = 0; nb < ND; ++nb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int off0 = (32 * c + vrow) * Tile::kPitch + (16 * nb + vcol) * 2;
        const int off1 = (32 * c + 16 + vrow) * Tile::kPitch + (16 * nb + vcol) * 2;
        dv[nb] = mfma16(concat_bf16(lds_read_tr(dO + off0), lds_read_tr(dO + off1)), pf[c], dv[nb]);
        dk[nb] = mfma16(concat_bf16(lds_read_tr(Q + off0), lds_read_tr(Q + off1)), dsf[c], dk[nb]);
      }
    if (more) swrite(cur ^ 1);
    __syncthreads();
  }
  if (key < g.s) {
    const float sc = g.scale_log2 * kLn2;  // 1 / sqrt(d)
    uint16_t* krow = dqkv + (tok0 + key) * ld + (int64_t)g.n * g.d + (int64_t)j * g.d;
    uint16_t* vrow_out = krow + (int64_t)g.n * g.d;
#pragma unroll
    for (int nb = 0; nb < ND; ++nb) {
      const int col = 16 * nb + 4 * g4;
      if (col < g.d) {
        const f32x4_t a = dk[nb] * sc, b = dv[nb];
        *(u32x2_t*)(krow + col) = u32x2_t{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
        *(u32x2_t*)(vrow_out + col) = u32x2_t{pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3])};
      }
    }
  }
}

// Backward, dQ: one workgroup per (128 queries, head, sequence), 4 waves of 32
// query rows, keys 64 at a time through LDS as in the forward.  S and dP
// (= dO V^T, V rows as the first operand) come out in the forward's layout;
// dS = P * (dP - delta) stays in registers for dQ += dS K, whose first
// operand (K gathered per column) comes from transposing LDS reads.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) attn_bwd_dq_kernel(AttnGeom g, const uint16_t* __restrict__ qkv,
                                                          const uint16_t* __restrict__ dout,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ delta,
                                                          uint16_t* __restrict__ dqkv) {
  constexpr int KD = D / 32, ND = D / 16;
  using Tile = AttnTile<D>;
  __shared__ __attribute__((aligned(16))) char kt[2][Tile::kBytes];
  __shared__ __attribute__((aligned(16))) char vt[2][Tile::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, l16 = lane & 15;
  const int q0 = blockIdx.x * kAttnBM, j = blockIdx.y, bi = blockIdx.z;
  const int64_t tok0 = (int64_t)bi * g.s, T = (int64_t)g.b * g.s;
  const int64_t ld = g.ld_qkv;
  const uint16_t* Qb = qkv + tok0 * ld + (int64_t)j * g.d;
  const uint16_t* Kb = Qb + (int64_t)g.n * g.d;
  const uint16_t* Vb = Qb + 2 * (int64_t)g.n * g.d;
  const uint16_t* dOb = dout + tok0 * (int64_t)g.ld_o + (int64_t)j * g.d;
  bf16x8_t qf[2][KD], df[2][KD];
  float lq[2], dq_del[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = q0 + 32 * w + 16 * rb + l16;
    const bool in = row < g.s;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const int c = kk * 4 + g4;
      const bool ok = in && c * 8 < g.d;
      qf[rb][kk] = as_bf16x8(ok ? *(const u32x4_t*)(Qb + (int64_t)row * ld + c * 8) : u32x4_t{0u, 0u, 0u, 0u});
      df[rb][kk] =
          as_bf16x8(ok ? *(const u32x4_t*)(dOb + (int64_t)row * g.ld_o + c * 8) : u32x4_t{0u, 0u, 0u, 0u});
    }
    lq[rb] = in ? lse[(int64_t)j * T + tok0 + row] * kLog2e : 0.f;
    dq_del[rb] = in ? delta[(int64_t)j * T + tok0 + row] : 0.f;
  }
  f32x4_t dq[2][ND];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int nb = 0; nb < ND; ++nb) dq[rb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int kv_end = CAUSAL ? min(g.s, q0 + kAttnBM) : g.s;
  const int nkb = (kv_end + kAttnBN - 1) / kAttnBN;
  TileRegs<D> kr, vr;
  tile_gload<D>(kr, Kb, ld, 0, g.s, g.d, tid);
  tile_gload<D>(vr, Vb, ld, 0, g.s, g.d, tid);
  tile_swrite<D>(kt[0], kr, tid);
  tile_swrite<D>(vt[0], vr, tid);
  __syncthreads();
  const int vrow = 4 * g4 + (l16 >> 2), vcol = 4 * (l16 & 3);
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) {
      tile_gload<D>(kr, Kb, ld, (kb + 1) * kAttnBN, g.s, g.d, tid);
      tile_gload<D>(vr, Vb, ld, (kb + 1) * kAttnBN, g.s, g.d, tid);
    }
    const char* K = kt[cur];
    const char* V = vt[cur];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int q = q0 + 32 * w + 16 * rb + l16;
      float ds[4][4];
#pragma unroll
      for (int kb16 = 0; kb16 < 4; ++kb16) {
        f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f}, dpacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KD; ++kk) {
          const int off = (kb16 * 16 + l16) * Tile::kPitch + (kk * 4 + g4) * 16;
          sacc = mfma16(lds_read_b128(K + off), qf[rb][kk], sacc);
          dpacc = mfma16(lds_read_b128(V + off), df[rb][kk], dpacc);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb * kAttnBN + kb16 * 16 + 4 * g4 + r;
          const bool valid = q < g.s && key < g.s && (!CAUSAL || key <= q);
          const float p = valid ? __builtin_amdgcn_exp2f(sacc[r] * g.scale_log2 - lq[rb]) : 0.f;
          ds[kb16][r] = p * (dpacc[r] - dq_del[rb]);
        }
      }
      bf16x8_t dsf[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
        dsf[c] = as_bf16x8(u32x4_t{pack_bf16x2(ds[2 * c][0], ds[2 * c][1]), pack_bf16x2(ds[2 * c][2], ds[2 * c][3]),
                                   pack_bf16x2(ds[2 * c + 1][0], ds[2 * c + 1][1]),
                                   pack_bf16x2(ds[2 * c + 1][2], ds[2 * c + 1][3])});
#pragma unroll
      for (int nb = 0; nb < ND; ++nb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const s16x4_t lo = lds_read_tr(K + (32 * c + vrow) * Tile::kPitch + (16 * nb + vcol) * 2);
          const s16x4_t hi = lds_read_tr(K + (32 * c + 16 + vrow) * Tile::kPitch + (16 * nb + vcol) * 2);
          dq[rb][nb] = mfma16(concat_bf16(lo, hi), dsf[c], dq[rb][nb]);
        }
    }
    if (more) {
      tile_swrite<D>(kt[cur ^ 1], kr, tid);
      tile_swrite<D>(vt[cur ^ 1], vr, tid);
    }
    __syncthreads();
  }
  const float sc = g.scale_log2 * kLn2;  // 1 / sqrt(d)
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int q = q0 + 32 * w + 16 * rb + l16;
    if (q >= g.s) continue;
    uint16_t* qrow = dqkv + (tok0 + q) * ld + (int64_t)j * g.d;
#pragma unroll
    for (int nb = 0; nb < ND; ++nb) {
      const int col = 16 * nb + 4 * g4;
      if (col < g.d) {
        const f32x4_t v = dq[rb][nb] * sc;
        *(u32x2_t*)(qrow + col) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_attn_bwd_t(const AttnGeom& g, const uint16_t* qkv, const uint16_t* dout, const float* lse,
                             const float* delta, uint16_t* dqkv, hipStream_t st) {
  const dim3 gk((unsigned)((g.s + kAttnBN - 1) / kAttnBN), (unsigned)g.n, (unsigned)g.b);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL>), gk, dim3(256), 0, st, g, qkv, dout, lse, delta, dqkv);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 gq((unsigned)((g.s + kAttnBM - 1) / kAttnBM), (unsigned)g.n, (unsigned)g.b);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL>), gq, dim3(256), 0, st, g, qkv, dout, lse, delta, dqkv);
  return hipGetLastError();
}

template <int D>
hipError_t launch_attn_bwd_d(const AttnGeom& g, bool causal, const uint16_t* qkv, const uint16_t* dout,
                             const float* lse, const float* delta, uint16_t* dqkv, hipStream_t st) {
  return causal ? launch_attn_bwd_t<D, true>(g, qkv, dout, lse, delta, dqkv, st)
                : launch_attn_bwd_t<D, false>(g, qkv, dout, lse, delta, dqkv, st);
}

}  // namespace

int attn_padded_dim(int d) { return ((d + 31) / 32) * 32; }

hipError_t launch_attn_core_bwd(const AttnGeom& g, bool causal, const uint16_t* qkv, const uint16_t* out,
                                const uint16_t* dout, const float* lse, float* delta, uint16_t* dqkv,
                                hipStream_t st) {
  const int64_t rows = (int64_t)g.b * g.s * g.n;
  hipLaunchKernelGGL(attn_bwd_delta, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st, g, out, dout, delta);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  switch (attn_padded_dim(g.d)) {
    case 32: return launch_attn_bwd_d<32>(g, causal, qkv, dout, lse, delta, dqkv, st);
    case 64: return launch_attn_bwd_d<64>(g, causal, qkv, dout, lse, delta, dqkv, st);
    case 96: return launch_attn_bwd_d<96>(g, causal, qkv, dout, lse, delta, dqkv, st);
    case 128: return launch_attn_bwd_d<128>(g, causal, qkv, dout, lse, delta, dqkv, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_core_fwd(const AttnGeom& g, bool causal, const uint16_t* qkv, uint16_t* out, float* lse,
                                hipStream_t st) {
  switch (attn_padded_dim(g.d)) {
    case 32: return launch_attn_fwd_d<32>(g, causal, qkv, out, lse, st);
    case 64: return launch_attn_fwd_d<64>(g, causal, qkv, out, lse, st);
    case 96: return launch_attn_fwd_d<96>(g, causal, qkv, out, lse, st);
    case 128: return launch_attn_fwd_d<128>(g, causal, qkv, out, lse, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mshard
