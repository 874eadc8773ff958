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
//     lanes of a query row merge its max over lanes l^16 and l^32.
//   Online softmax in base 2 (scores scaled by log2(e)/sqrt(d)); the running
//     max is raised only when a scaled score exceeds it by more than 8, so most
//     steps skip the merge and the rescale of O; masks are applied only on the
//     steps that cross the causal diagonal or the sequence end.
//   O += P V: P stays in registers as the MFMA's second operand.  A lane's
//     8 keys of a 32-key step are {4g..4g+3, 16+4g..16+4g+3} (g = l/16), the
//     keys its S registers hold; the V fragment is gathered in the same key
//     order with two transposing LDS reads (ds_read_b64_tr_b16), so the
//     contraction pairs every key with itself.
// Grids put the (head, sequence) pairs on x and a sequence's row blocks on y,
// so that under a causal mask every block with the most work is dispatched
// before any block with less (the last blocks to start are the shortest).
#include <type_traits>

#include "epilogues.hpp"
#include "launch.hpp"

namespace mshard {

namespace {

constexpr int kAttnBM = 128;  // query rows per workgroup
constexpr int kAttnBN = 64;   // keys per step

// Waves per SIMD each kernel is compiled for (at most 512 / waves registers a
// lane): every head size keeps its fragments and accumulators without spills.
constexpr int attn_waves_per_simd(int d) { return d <= 32 ? 4 : d <= 64 ? 3 : 1; }
constexpr float kLn2 = 0.69314718055994530942f;

typedef short s16x8_t __attribute__((ext_vector_type(8)));

// LDS tile of 64 rows x D columns (bf16), rows padded by 16 bytes (pitch = 16
// mod 128 at every head size).  The kernels read it two ways: a 16-byte read
// per lane of one chunk from 8 consecutive rows per 128-byte bank cycle
// (ds_read_b128), which the pad spreads over 8 distinct 16-byte slots; and an
// 8-byte transposing read per lane of 32 consecutive bytes from 4 consecutive
// rows per cycle (ds_read_b64_tr_b16), where neighbouring rows share one slot.
// A layout free of both conflicts (32-byte pad, chunk pairs swapped on rows
// 4..7 of each 8) measured slower: the forward and dQ cores took 6% and 5%
// longer on the same GPU, the dK/dV core the same time.
template <int D>
struct AttnTile {
  static constexpr int kChunks = D / 8;  // 16-byte chunks per row
  static constexpr int kPitch = 2 * D + 16;
  static constexpr int kBytes = kAttnBN * kPitch;
  static constexpr int kPerThread = 64 * kChunks / 256;  // = D / 32
  // byte offset of chunk c (columns 8c .. 8c+7) of row r
  __device__ static __forceinline__ int chunk(int r, int c) { return r * kPitch + 16 * c; }
  // byte offset of columns col .. col+3 of row r (col a multiple of 4)
  __device__ static __forceinline__ int quad(int r, int col) { return chunk(r, col >> 3) + ((col & 4) << 1); }
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
    *(u32x4_t*)(lds + AttnTile<D>::chunk(row, c)) = t.v[u];
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

// The softmax step of a wave's two 16-query groups over the 64 keys whose raw
// scores sacc holds (lane l: query l%16 of group rb, keys 16kb16 + 4(l/16) + r).
// The running max m is kept in the scaled (base-2) domain and only raised when
// some row of the group sees a score more than kRescaleSlack above it (a
// wave-uniform test per group), so the common step needs no cross-lane
// merge and no rescale of O; the exponents then stay at most 2^kRescaleSlack,
// which bf16 P and the fp32 sums hold exactly as well as 1.  The row sum is kept
// per lane (the lane's 16 keys of each step) and merged over the row's four
// lanes once, after the last step.  MASK: key key0 + off of group rb is valid
// when off <= lim[rb].
constexpr float kRescaleSlack = 8.f;

template <int ND, bool MASK>
__device__ __forceinline__ void attn_softmax_step(const f32x4_t (&sacc)[2][4], f32x4_t (&o)[2][ND], float (&m)[2],
                                                  float (&nm)[2], float (&l)[2], bf16x8_t (&pf)[2][2], float scale,
                                                  const int (&lim)[2]) {
  float sv[2][4][4];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float lm = -INFINITY;
#pragma unroll
    for (int kb16 = 0; kb16 < 4; ++kb16)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[rb][kb16][r] = sacc[rb][kb16][r];
        if (MASK && kb16 * 16 + r > lim[rb]) sv[rb][kb16][r] = -INFINITY;
        lm = fmaxf(lm, sv[rb][kb16][r]);
      }
    lm *= scale;  // scale > 0, so the max commutes with it exactly
    if (__any(lm > m[rb] + kRescaleSlack)) {
      const float mnew = fmaxf(m[rb], row_max4(lm));
      const float corr = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[rb] - mnew);
      l[rb] *= corr;
#pragma unroll
      for (int nb = 0; nb < ND; ++nb) o[rb][nb] *= corr;
      m[rb] = mnew;
      nm[rb] = mnew == -INFINITY ? 0.f : -mnew;
    }
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float p[4][4];
#pragma unroll
    for (int kb16 = 0; kb16 < 4; ++kb16)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[kb16][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[rb][kb16][r], scale, nm[rb]));
        l[rb] += p[kb16][r];
      }
#pragma unroll
    for (int c = 0; c < 2; ++c)
      pf[rb][c] = as_bf16x8(u32x4_t{pack_bf16x2(p[2 * c][0], p[2 * c][1]), pack_bf16x2(p[2 * c][2], p[2 * c][3]),
                                    pack_bf16x2(p[2 * c + 1][0], p[2 * c + 1][1]),
                                    pack_bf16x2(p[2 * c + 1][2], p[2 * c + 1][3])});
  }
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(attn_waves_per_simd(D))))
attn_fwd_kernel(AttnGeom g, const uint16_t* __restrict__ qkv,
                                                       uint16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int KD = D / 32, ND = D / 16;
  using Tile = AttnTile<D>;
  __shared__ __attribute__((aligned(16))) char kt[2][Tile::kBytes];
  __shared__ __attribute__((aligned(16))) char vt[2][Tile::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so the mask test is a scalar branch
  // grid x: (head, sequence) pairs; y: query blocks, the ones that see the most keys (causal) dispatched first
  const int qblk = CAUSAL ? (int)gridDim.y - 1 - (int)blockIdx.y : (int)blockIdx.y;
  const int q0 = qblk * kAttnBM, j = (int)blockIdx.x % g.n, bi = (int)blockIdx.x / g.n;
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
  float m[2], nm[2], l[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    m[rb] = -INFINITY;
    nm[rb] = 0.f;
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
  const int vrow = 4 * g4 + (l16 >> 2), vcol = 4 * (l16 & 3);
  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    const bool more = kb + 1 < nkb;
    if (more) {  // next tile in flight while this one is consumed
      tile_gload<D>(kr, Kb, ld, (kb + 1) * kAttnBN, g.s, g.d, tid);
      tile_gload<D>(vr, Vb, ld, (kb + 1) * kAttnBN, g.s, g.d, tid);
    }
    const char* K = kt[cur];
    const char* V = vt[cur];
    const int kbase = kb * kAttnBN;
    // every K fragment is read once and serves both query groups
    f32x4_t sacc[2][4];
#pragma unroll
    for (int kb16 = 0; kb16 < 4; ++kb16) {
      sacc[0][kb16] = sacc[1][kb16] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KD; ++kk) {
        const bf16x8_t kfrag = lds_read_b128(K + Tile::chunk(kb16 * 16 + l16, kk * 4 + g4));
        sacc[0][kb16] = mfma16(kfrag, qf[0][kk], sacc[0][kb16]);
        sacc[1][kb16] = mfma16(kfrag, qf[1][kk], sacc[1][kb16]);
      }
    }
    // keys past the sequence end, or (causal) after some row of the wave, need the mask
    const int qw = q0 + 32 * w;  // the wave's first query row
    const bool masked = kbase + kAttnBN > g.s || (CAUSAL && kbase + kAttnBN - 1 > qw);
    bf16x8_t pf[2][2];
    if (masked) {
      int lim[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        lim[rb] = (CAUSAL ? min(qw + 16 * rb + l16, g.s - 1) : g.s - 1) - kbase - 4 * g4;
      attn_softmax_step<ND, true>(sacc, o, m, nm, l, pf, g.scale_log2, lim);
    } else {
      const int lim[2] = {0, 0};
      attn_softmax_step<ND, false>(sacc, o, m, nm, l, pf, g.scale_log2, lim);
    }
    // source lane 16G + s of a transposing read addresses key 4G + s/4 (+ 16 for the second half)
    // and columns 16nb + 4(s%4) .. +3; every V fragment serves both query groups
#pragma unroll
    for (int nb = 0; nb < ND; ++nb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8_t vfrag = concat_bf16(lds_read_tr(V + Tile::quad(32 * c + vrow, 16 * nb + vcol)),
                                           lds_read_tr(V + Tile::quad(32 * c + 16 + vrow, 16 * nb + vcol)));
        o[0][nb] = mfma16(vfrag, pf[0][c], o[0][nb]);
        o[1][nb] = mfma16(vfrag, pf[1][c], o[1][nb]);
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
    const float lrow = row_sum4(l[rb]);  // every lane joins the merge before the row test
    if (q >= g.s) continue;
    const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
    uint16_t* orow = out + (tok0 + q) * (int64_t)g.ld_o + (int64_t)j * g.d;
#pragma unroll
    for (int nb = 0; nb < ND; ++nb) {
      const int col = 16 * nb + 4 * g4;
      if (col < g.d) {
        const f32x4_t v = o[rb][nb] * inv;
        *(u32x2_t*)(orow + col) = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
    if (g4 == 0) lse[(int64_t)j * T + tok0 + q] = (m[rb] + __builtin_log2f(lrow)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_attn_fwd_t(const AttnGeom& g, const uint16_t* qkv, uint16_t* out, float* lse, hipStream_t st) {
  const dim3 grid((unsigned)(g.n * g.b), (unsigned)((g.s + kAttnBM - 1) / kAttnBM));
  hipLaunchKernelGGL((attn_fwd_kernel<D, CAUSAL>), grid, dim3(256), 0, st, g, qkv, out, lse);
  return hipGetLastError();
}

template <int D>
hipError_t launch_attn_fwd_d(const AttnGeom& g, bool causal, const uint16_t* qkv, uint16_t* out, float* lse,
                             hipStream_t st) {
  return causal ? launch_attn_fwd_t<D, true>(g, qkv, out, lse, st) : launch_attn_fwd_t<D, false>(g, qkv, out, lse, st);
}

// Backward, dK and dV: one workgroup per (64 keys, head, sequence); wave w owns
// keys k0 + 16w .. +15 and loops over the query blocks that see them (64
// queries per step, through LDS: the Q and dO tiles plus each query's
// -lse*log2(e) and delta).  With the Q fragment as the MFMA's first operand,
// lane l holds S[query 4(l/16) + r][key l%16] of each 16-query block: the
// transposed layout, so P^T and dS^T stay in registers as the second operand of
//   dV += P^T dO  and  dK += dS^T Q,
// whose first operands (dO and Q gathered per column) come from transposing
// LDS reads, and dP^T = V dO^T takes the wave's V rows from registers.  Only
// the steps that cross the causal diagonal or the sequence end are masked.
template <int D, bool MASK>
__device__ __forceinline__ void dkdv_group_ds(const char* Q, const char* dO, const float* nl, const float* dl,
                                              const bf16x8_t (&kf)[D / 32], const bf16x8_t (&vf)[D / 32],
                                              float scale, int lo, int hi, int l16, int g4, bf16x8_t (&pf)[2],
                                              bf16x8_t (&dsf)[2]) {
  constexpr int KD = D / 32;
  using Tile = AttnTile<D>;
  float p[4][4], ds[4][4];
#pragma unroll
  for (int qb16 = 0; qb16 < 4; ++qb16) {
    f32x4_t sacc = f32x4_t{0.f, 0.f, 0.f, 0.f}, dpacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const int off = Tile::chunk(qb16 * 16 + l16, kk * 4 + g4);
      sacc = mfma16(lds_read_b128(Q + off), kf[kk], sacc);
      dpacc = mfma16(lds_read_b128(dO + off), vf[kk], dpacc);
    }
    // the lane's four queries qb16*16 + 4(l/16) + r are consecutive: one 16-byte read each
    const f32x4_t nl4 = *(const f32x4_t*)(nl + qb16 * 16 + 4 * g4);
    const f32x4_t dl4 = *(const f32x4_t*)(dl + qb16 * 16 + 4 * g4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], scale, nl4[r]));
      if (MASK && !(qb16 * 16 + r >= lo && qb16 * 16 + r < hi)) pv = 0.f;
      p[qb16][r] = pv;
      ds[qb16][r] = pv * (dpacc[r] - dl4[r]);
    }
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    pf[c] = as_bf16x8(u32x4_t{pack_bf16x2(p[2 * c][0], p[2 * c][1]), pack_bf16x2(p[2 * c][2], p[2 * c][3]),
                              pack_bf16x2(p[2 * c + 1][0], p[2 * c + 1][1]),
                              pack_bf16x2(p[2 * c + 1][2], p[2 * c + 1][3])});
    dsf[c] = as_bf16x8(u32x4_t{pack_bf16x2(ds[2 * c][0], ds[2 * c][1]), pack_bf16x2(ds[2 * c][2], ds[2 * c][3]),
                               pack_bf16x2(ds[2 * c + 1][0], ds[2 * c + 1][1]),
                               pack_bf16x2(ds[2 * c + 1][2], ds[2 * c + 1][3])});
  }
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(attn_waves_per_simd(D))))
attn_bwd_dkdv_kernel(AttnGeom g, const uint16_t* __restrict__ qkv,
                                                            const uint16_t* __restrict__ dout,
                                                            const float* __restrict__ lse,
                                                            const float* __restrict__ delta,
                                                            uint16_t* __restrict__ dqkv) {
  constexpr int KD = D / 32, ND = D / 16;
  using Tile = AttnTile<D>;
  __shared__ __attribute__((aligned(16))) char qt[2][Tile::kBytes];
  __shared__ __attribute__((aligned(16))) char dt[2][Tile::kBytes];
  // per query of the block: -lse*log2(e) at [0, 64), delta at [64, 128)
  __shared__ __attribute__((aligned(16))) float srow[2][2 * kAttnBN];
  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so the mask test is a scalar branch
  // grid x: (head, sequence) pairs; y: key blocks, the first (causal: seen by the most queries) dispatched first
  const int k0 = (int)blockIdx.y * kAttnBN, j = (int)blockIdx.x % g.n, bi = (int)blockIdx.x / g.n;
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
  float rt = 0.f;  // threads [0, 128): their query's row term
  auto gload = [&](int qb) {
    const int r0 = qstart + qb * kAttnBN;
    tile_gload<D>(qr, Qb, ld, r0, g.s, g.d, tid);
    tile_gload<D>(dr, dOb, g.ld_o, r0, g.s, g.d, tid);
    const int q = r0 + (tid & (kAttnBN - 1));
    if (tid < 2 * kAttnBN) rt = q >= g.s ? 0.f : tid < kAttnBN ? -lseb[q] * kLog2e : delb[q];
  };
  auto swrite = [&](int buf) {
    tile_swrite<D>(qt[buf], qr, tid);
    tile_swrite<D>(dt[buf], dr, tid);
    if (tid < 2 * kAttnBN) srow[buf][tid] = rt;
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
    // query qbase + 4(l/16) + off is valid for this lane's key when lo <= off < hi
    const int lo = CAUSAL ? key - qbase - 4 * g4 : 0, hi = g.s - qbase - 4 * g4;
    const bool masked = qbase + kAttnBN > g.s || (CAUSAL && qbase < k0 + 16 * w + 15);
    bf16x8_t pf[2], dsf[2];
    if (masked)
      dkdv_group_ds<D, true>(Q, dO, srow[cur], srow[cur] + kAttnBN, kf, vf, g.scale_log2, lo, hi, l16, g4, pf,
                             dsf);
    else
      dkdv_group_ds<D, false>(Q, dO, srow[cur], srow[cur] + kAttnBN, kf, vf, g.scale_log2, lo, hi, l16, g4, pf,
                              dsf);
#pragma unroll
    for (int nb = 0; nb < ND; ++nb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int off0 = Tile::quad(32 * c + vrow, 16 * nb + vcol);
        const int off1 = Tile::quad(32 * c + 16 + vrow, 16 * nb + vcol);
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

// Backward, dQ, launched before dK/dV: one workgroup per (128 queries, head,
// sequence), 4 waves of 32 query rows, keys 64 at a time through LDS as in the
// forward.  The prologue forms each query's delta = sum over the head's
// columns of dO * O (fp32; the lane's own columns, then its row's four lanes
// in a fixed tree), the row term of dS = P * (dP - delta), and stores it for
// the dK/dV kernel.  S and dP (= dO V^T, V rows as the first operand) come out
// in the forward's layout; dS stays in registers for dQ += dS K, whose first
// operand (K gathered per column) comes from transposing LDS reads.  Only the
// steps that cross the causal diagonal or the sequence end are masked.
template <int D, bool MASK>
__device__ __forceinline__ void dq_step_ds(const char* K, const char* V, const bf16x8_t (&qf)[2][D / 32],
                                           const bf16x8_t (&df)[2][D / 32], const float (&nlq)[2],
                                           const float (&del)[2], float scale, const int (&lim)[2], int l16, int g4,
                                           bf16x8_t (&dsf)[2][2]) {
  constexpr int KD = D / 32;
  using Tile = AttnTile<D>;
  float ds[2][4][4];
#pragma unroll
  for (int kb16 = 0; kb16 < 4; ++kb16) {
    // every K and V fragment is read once and serves both query groups
    f32x4_t sacc[2], dpacc[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) sacc[rb] = dpacc[rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const int off = Tile::chunk(kb16 * 16 + l16, kk * 4 + g4);
      const bf16x8_t kfrag = lds_read_b128(K + off), vfrag = lds_read_b128(V + off);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        sacc[rb] = mfma16(kfrag, qf[rb][kk], sacc[rb]);
        dpacc[rb] = mfma16(vfrag, df[rb][kk], dpacc[rb]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[rb][r], scale, nlq[rb]));
        if (MASK && kb16 * 16 + r > lim[rb]) p = 0.f;
        ds[rb][kb16][r] = p * (dpacc[rb][r] - del[rb]);
      }
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int c = 0; c < 2; ++c)
      dsf[rb][c] = as_bf16x8(u32x4_t{pack_bf16x2(ds[rb][2 * c][0], ds[rb][2 * c][1]),
                                     pack_bf16x2(ds[rb][2 * c][2], ds[rb][2 * c][3]),
                                     pack_bf16x2(ds[rb][2 * c + 1][0], ds[rb][2 * c + 1][1]),
                                     pack_bf16x2(ds[rb][2 * c + 1][2], ds[rb][2 * c + 1][3])});
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(attn_waves_per_simd(D))))
attn_bwd_dq_kernel(AttnGeom g, const uint16_t* __restrict__ qkv,
                                                          const uint16_t* __restrict__ out,
                                                          const uint16_t* __restrict__ dout,
                                                          const float* __restrict__ lse, float* __restrict__ delta,
                                                          uint16_t* __restrict__ dqkv) {
  constexpr int KD = D / 32, ND = D / 16;
  using Tile = AttnTile<D>;
  __shared__ __attribute__((aligned(16))) char kt[2][Tile::kBytes];
  __shared__ __attribute__((aligned(16))) char vt[2][Tile::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so the mask test is a scalar branch
  // grid x: (head, sequence) pairs; y: query blocks, the ones that see the most keys (causal) dispatched first
  const int qblk = CAUSAL ? (int)gridDim.y - 1 - (int)blockIdx.y : (int)blockIdx.y;
  const int q0 = qblk * kAttnBM, j = (int)blockIdx.x % g.n, bi = (int)blockIdx.x / g.n;
  const int64_t tok0 = (int64_t)bi * g.s, T = (int64_t)g.b * g.s;
  const int64_t ld = g.ld_qkv;
  const uint16_t* Qb = qkv + tok0 * ld + (int64_t)j * g.d;
  const uint16_t* Kb = Qb + (int64_t)g.n * g.d;
  const uint16_t* Vb = Qb + 2 * (int64_t)g.n * g.d;
  const uint16_t* Ob = out + tok0 * (int64_t)g.ld_o + (int64_t)j * g.d;
  const uint16_t* dOb = dout + tok0 * (int64_t)g.ld_o + (int64_t)j * g.d;
  bf16x8_t qf[2][KD], df[2][KD];
  float nlq[2], del[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = q0 + 32 * w + 16 * rb + l16;
    const bool in = row < g.s;
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < KD; ++kk) {
      const int c = kk * 4 + g4;
      const bool ok = in && c * 8 < g.d;
      const u32x4_t zero = u32x4_t{0u, 0u, 0u, 0u};
      qf[rb][kk] = as_bf16x8(ok ? *(const u32x4_t*)(Qb + (int64_t)row * ld + c * 8) : zero);
      const u32x4_t dv = ok ? *(const u32x4_t*)(dOb + (int64_t)row * g.ld_o + c * 8) : zero;
      const u32x4_t ov = ok ? *(const u32x4_t*)(Ob + (int64_t)row * g.ld_o + c * 8) : zero;
      df[rb][kk] = as_bf16x8(dv);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        part += bf16_lo(dv[k]) * bf16_lo(ov[k]);
        part += bf16_hi(dv[k]) * bf16_hi(ov[k]);
      }
    }
    del[rb] = row_sum4(part);  // every lane joins the merge; rows past the end sum zeros
    nlq[rb] = in ? -lse[(int64_t)j * T + tok0 + row] * kLog2e : 0.f;
    if (in && g4 == 0) delta[(int64_t)j * T + tok0 + row] = del[rb];
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
    const int kbase = kb * kAttnBN;
    const int qw = q0 + 32 * w;  // the wave's first query row
    const bool masked = kbase + kAttnBN > g.s || (CAUSAL && kbase + kAttnBN - 1 > qw);
    bf16x8_t dsf[2][2];
    if (masked) {
      // key kbase + 4(l/16) + off is valid for this lane's query of group rb when off <= lim[rb]
      int lim[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        lim[rb] = (CAUSAL ? min(qw + 16 * rb + l16, g.s - 1) : g.s - 1) - kbase - 4 * g4;
      dq_step_ds<D, true>(K, V, qf, df, nlq, del, g.scale_log2, lim, l16, g4, dsf);
    } else {
      const int lim[2] = {0, 0};
      dq_step_ds<D, false>(K, V, qf, df, nlq, del, g.scale_log2, lim, l16, g4, dsf);
    }
#pragma unroll
    for (int nb = 0; nb < ND; ++nb)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8_t kfrag = concat_bf16(lds_read_tr(K + Tile::quad(32 * c + vrow, 16 * nb + vcol)),
                                           lds_read_tr(K + Tile::quad(32 * c + 16 + vrow, 16 * nb + vcol)));
        dq[0][nb] = mfma16(kfrag, dsf[0][c], dq[0][nb]);
        dq[1][nb] = mfma16(kfrag, dsf[1][c], dq[1][nb]);
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
hipError_t launch_attn_bwd_t(const AttnGeom& g, const uint16_t* qkv, const uint16_t* out, const uint16_t* dout,
                             const float* lse, float* delta, uint16_t* dqkv, hipStream_t st) {
  const dim3 gq((unsigned)(g.n * g.b), (unsigned)((g.s + kAttnBM - 1) / kAttnBM));
  hipLaunchKernelGGL((attn_bwd_dq_kernel<D, CAUSAL>), gq, dim3(256), 0, st, g, qkv, out, dout, lse, delta, dqkv);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const dim3 gk((unsigned)(g.n * g.b), (unsigned)((g.s + kAttnBN - 1) / kAttnBN));
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, CAUSAL>), gk, dim3(256), 0, st, g, qkv, dout, lse,
                     (const float*)delta, dqkv);
  return hipGetLastError();
}

template <int D>
hipError_t launch_attn_bwd_d(const AttnGeom& g, bool causal, const uint16_t* qkv, const uint16_t* out,
                             const uint16_t* dout, const float* lse, float* delta, uint16_t* dqkv, hipStream_t st) {
  return causal ? launch_attn_bwd_t<D, true>(g, qkv, out, dout, lse, delta, dqkv, st)
                : launch_attn_bwd_t<D, false>(g, qkv, out, dout, lse, delta, dqkv, st);
}

}  // namespace

int attn_padded_dim(int d) { return ((d + 31) / 32) * 32; }

hipError_t launch_attn_core_bwd(const AttnGeom& g, bool causal, const uint16_t* qkv, const uint16_t* out,
                                const uint16_t* dout, const float* lse, float* delta, uint16_t* dqkv,
                                hipStream_t st) {
  switch (attn_padded_dim(g.d)) {
    case 32: return launch_attn_bwd_d<32>(g, causal, qkv, out, dout, lse, delta, dqkv, st);
    case 64: return launch_attn_bwd_d<64>(g, causal, qkv, out, dout, lse, delta, dqkv, st);
    case 96: return launch_attn_bwd_d<96>(g, causal, qkv, out, dout, lse, delta, dqkv, st);
    case 128: return launch_attn_bwd_d<128>(g, causal, qkv, out, dout, lse, delta, dqkv, st);
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
