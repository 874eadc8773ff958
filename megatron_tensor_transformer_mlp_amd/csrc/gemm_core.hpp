// gemm_core.hpp - bf16 MFMA GEMM main loop for gfx950 (CDNA4), shared by every
// GEMM of the MLP shard and of the vocab-parallel CE shard.
//
//   C[M x N] = sum_k A(m, k) * B(k, n),  bf16 inputs, fp32 accumulation.
//
// A is stored either K-major (row-major [M x K], "A_KMAJOR") or M-major
// (row-major [K x M]); B either K-major (row-major [N x K]) or N-major
// (row-major [K x N]).  The six GEMMs of the MLP shard and the logits GEMM of
// the CE shard use three of the four combinations:
//   NN  (A K-major, B N-major):  X A_i,  Y_i B_i,  X E_i
//   NT  (A K-major, B K-major):  dZ B_i^T,  dH_i A_i^T
//   TN  (A M-major, B N-major):  Y_i^T dZ,  X^T dH_i
//
// Work decomposition
//   * One workgroup = 256 threads = 4 wave64s computes a 256 x 256 tile of C.
//     The waves form a 2 x 2 grid, each owning a 128 x 128 sub-tile held as
//     8 x 8 fp32 16x16 MFMA accumulators (256 VGPRs per lane).
//   * K advances in steps of 64.  Each step's A and B tiles are staged in LDS
//     (2 x 32 KiB), double buffered (128 KiB total), one barrier per step.
//     Global loads of step k+1 are issued before the MFMAs of step k.
//   * LDS holds both operands K-contiguous: one 128-byte row per m (or n), split
//     into eight 16-byte chunks of 8 k values.  Chunk c of row r is stored at
//     slot c ^ (r & 7), so the 16-byte fragment reads of 8 consecutive rows
//     (and the 16-byte tile writes) hit distinct bank groups.
//   * M/N-major operands are loaded as 8 x 8 bf16 blocks (8 k rows of 16 bytes)
//     and transposed in registers with v_perm before the LDS write.
//   * MFMA v_mfma_f32_16x16x32_bf16 is issued with the B fragment as its first
//     operand and the A fragment as its second, so each lane ends up holding
//     C[row = l%16][4 consecutive columns (l/16)*4 .. +3] of every 16x16
//     block: row-contiguous 16-byte (fp32) or 8-byte (bf16) output vectors,
//     and per-row reductions need only lanes l, l^16, l^32, l^48.
//   * All global accesses use buffer instructions on per-tile resources:
//     masked-off lanes get an offset beyond the resource, so edge tiles read
//     zeros and drop their stores without branches.
//   * Tiles are visited XCD-aware: consecutive block ids are dealt round-robin
//     to the 8 XCDs, so block ids are remapped to give each XCD a contiguous
//     run of tiles, walked in groups of GROUP_M tile-rows for L2 reuse.
//   * Optional split of the K range (deterministic split-K): split s of S covers
//     the k-steps [s*nk/S, (s+1)*nk/S) and its epilogue writes a private slice.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mshard {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kThreads = 256;
constexpr int kWaveM = 128, kWaveN = 128;
constexpr int kSubM = kWaveM / 16, kSubN = kWaveN / 16;
constexpr int kStageBytes = (kBM + kBN) * kBK * 2;  // 64 KiB
constexpr int kLdsBytes = 2 * kStageBytes;          // 128 KiB
constexpr int kGroupM = 8;
constexpr int kNumXcd = 8;
constexpr uint32_t kOOB = 0x80000000u;  // any offset >= every resource size
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// Buffer resource over [base, base + bytes_left), size clamped below 2^31 so
// that kOOB is always out of range.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes_left) {
  int64_t n = bytes_left < 0 ? 0 : (bytes_left > 0x7fffffff ? 0x7fffffff : bytes_left);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, (int)kRsrcWord3);
}

__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2_t buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store16(u32x4_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store8(u32x2_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store4(uint32_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

struct Operand {
  const uint16_t* ptr;  // bf16 bit patterns
  int64_t ld;           // elements between consecutive stored rows
  int64_t elems;        // total elements of the stored matrix (resource extent)
};

struct GemmGeom {
  int M, N, K;
  int tiles_m, tiles_n;
  int splits;  // >= 1
};

// Block id -> (tile_m, tile_n, split), XCD-aware and grouped along M.
__device__ __forceinline__ void map_tile(const GemmGeom& g, int& tm, int& tn, int& split) {
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int q = G / kNumXcd, r = G % kNumXcd;
  const int xcd = b % kNumXcd, idx = b / kNumXcd;
  const int lin = (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
  const int tiles = g.tiles_m * g.tiles_n;
  split = lin / tiles;
  const int t = lin - split * tiles;
  const int per_group = kGroupM * g.tiles_n;
  const int group = t / per_group;
  const int first_m = group * kGroupM;
  const int gsz = min(g.tiles_m - first_m, kGroupM);
  const int in_g = t - group * per_group;
  tm = first_m + in_g % gsz;
  tn = in_g / gsz;
}

// ---------------------------------------------------------------------------
// Tile loaders: global -> registers (16-byte buffer loads) and registers -> LDS.
// LDS row r (of m or n) holds 64 k values; chunk c (k = 8c .. 8c+7) sits at
// byte r*128 + ((c ^ (r & 7)) << 4).

// K-major tile: 256 stored rows (row0 ..), 64 k values from k0.
// Thread t loads chunk c = t & 7 of rows (t >> 3) + 32 i, i = 0..7.
__device__ __forceinline__ void load_kmajor(u32x4_t (&v)[8], const Operand& op, int row0, int nrows,
                                            int k0, int K) {
  const int t = threadIdx.x;
  const int c = t & 7, r = t >> 3;
  const int64_t base_elem = (int64_t)row0 * op.ld + k0;
  const rsrc_t rs = make_rsrc(op.ptr + base_elem, (op.elems - base_elem) * 2);
  const bool kok = (k0 + c * 8) < K;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r + 32 * i;
    const bool ok = kok && (row0 + row) < nrows;
    const uint32_t off = ok ? (uint32_t)(((int64_t)row * op.ld + c * 8) * 2) : kOOB;
    v[i] = buf_load16(rs, off);
  }
}

__device__ __forceinline__ void store_kmajor(const u32x4_t (&v)[8], char* lds) {
  const int t = threadIdx.x;
  const int c = t & 7, r = t >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = r + 32 * i;
    *(u32x4_t*)(lds + row * 128 + ((c ^ (row & 7)) << 4)) = v[i];
  }
}

// M/N-major tile: 64 stored rows (k = k0 ..), 256 contiguous columns from col0.
// Thread t owns the 8 x 8 block k = 8*(t & 7) .. +7, col = 8*(t >> 3) .. +7.
__device__ __forceinline__ void load_mnmajor(u32x4_t (&v)[8], const Operand& op, int col0, int ncols,
                                             int k0, int K) {
  const int t = threadIdx.x;
  const int kb = t & 7, mb = t >> 3;
  const int64_t base_elem = (int64_t)k0 * op.ld + col0;
  const rsrc_t rs = make_rsrc(op.ptr + base_elem, (op.elems - base_elem) * 2);
  const bool cok = (col0 + mb * 8) < ncols;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = kb * 8 + i;
    const bool ok = cok && (k0 + k) < K;
    const uint32_t off = ok ? (uint32_t)(((int64_t)k * op.ld + mb * 8) * 2) : kOOB;
    v[i] = buf_load16(rs, off);
  }
}

// in[i] = 8 columns of k row i; out[j] = 8 k values of column j.
__device__ __forceinline__ void transpose8x8(const u32x4_t (&in)[8], u32x4_t (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      out[j][p] = __builtin_amdgcn_perm(in[2 * p + 1][j >> 1], in[2 * p][j >> 1], sel);
    }
  }
}

__device__ __forceinline__ void store_mnmajor(const u32x4_t (&v)[8], char* lds) {
  const int t = threadIdx.x;
  const int kb = t & 7, mb = t >> 3;
  u32x4_t tr[8];
  transpose8x8(v, tr);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = mb * 8 + j;
    *(u32x4_t*)(lds + row * 128 + ((kb ^ j) << 4)) = tr[j];
  }
}

template <bool KMAJOR>
__device__ __forceinline__ void load_tile(u32x4_t (&v)[8], const Operand& op, int mn0, int nmn, int k0, int K) {
  if constexpr (KMAJOR) load_kmajor(v, op, mn0, nmn, k0, K);
  else load_mnmajor(v, op, mn0, nmn, k0, K);
}
template <bool KMAJOR>
__device__ __forceinline__ void store_tile(const u32x4_t (&v)[8], char* lds) {
  if constexpr (KMAJOR) store_kmajor(v, lds);
  else store_mnmajor(v, lds);
}

// One 64-deep K step from an LDS stage into the wave's 8 x 8 accumulators.
__device__ __forceinline__ void mfma_stage(f32x4_t (&acc)[kSubM][kSubN], const char* As, const char* Bs,
                                           int wm, int wn, int lane) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int c = ks * 4 + (lane >> 4);
    bf16x8_t af[kSubM], bfr[kSubN];
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi) {
      const int row = wm * kWaveM + mi * 16 + (lane & 15);
      af[mi] = *(const bf16x8_t*)(As + row * 128 + ((c ^ (row & 7)) << 4));
    }
#pragma unroll
    for (int ni = 0; ni < kSubN; ++ni) {
      const int row = wn * kWaveN + ni * 16 + (lane & 15);
      bfr[ni] = *(const bf16x8_t*)(Bs + row * 128 + ((c ^ (row & 7)) << 4));
    }
#pragma unroll
    for (int mi = 0; mi < kSubM; ++mi)
#pragma unroll
      for (int ni = 0; ni < kSubN; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[ni], af[mi], acc[mi][ni], 0, 0, 0);
  }
}

// Position of accumulator element acc[mi][ni][r] inside the 256 x 256 tile:
//   row = wm*128 + mi*16 + (lane & 15),  col = wn*128 + ni*16 + (lane >> 4)*4 + r.
struct EpiCtx {
  int m0, n0;   // tile origin in C
  int tm, tn;   // tile coordinates
  int split;    // K split index
  int wm, wn;   // wave coordinates in the tile
  int lane;
  char* lds;    // 128 KiB, free for the epilogue after the main loop
};

template <bool A_KMAJOR, bool B_KMAJOR, class Epi>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
gemm_kernel(GemmGeom g, Operand a, Operand b, Epi epi) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  int tm, tn, split;
  map_tile(g, tm, tn, split);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int nk = (g.K + kBK - 1) / kBK;
  const int kt_beg = (int)(((int64_t)split * nk) / g.splits);
  const int kt_end = (int)(((int64_t)(split + 1) * nk) / g.splits);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x4_t acc[kSubM][kSubN];
#pragma unroll
  for (int mi = 0; mi < kSubM; ++mi)
#pragma unroll
    for (int ni = 0; ni < kSubN; ++ni) acc[mi][ni] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (kt_beg < kt_end) {
    u32x4_t ra[8], rb[8];
    load_tile<A_KMAJOR>(ra, a, m0, g.M, kt_beg * kBK, g.K);
    load_tile<B_KMAJOR>(rb, b, n0, g.N, kt_beg * kBK, g.K);
    store_tile<A_KMAJOR>(ra, lds);
    store_tile<B_KMAJOR>(rb, lds + kBM * 128);
    __syncthreads();
    for (int kt = kt_beg; kt < kt_end; ++kt) {
      const int stage = (kt - kt_beg) & 1;
      const bool more = kt + 1 < kt_end;
      if (more) {
        load_tile<A_KMAJOR>(ra, a, m0, g.M, (kt + 1) * kBK, g.K);
        load_tile<B_KMAJOR>(rb, b, n0, g.N, (kt + 1) * kBK, g.K);
      }
      const char* As = lds + stage * kStageBytes;
      mfma_stage(acc, As, As + kBM * 128, wm, wn, lane);
      if (more) {
        char* nxt = lds + (stage ^ 1) * kStageBytes;
        store_tile<A_KMAJOR>(ra, nxt);
        store_tile<B_KMAJOR>(rb, nxt + kBM * 128);
      }
      __syncthreads();
    }
  }
  EpiCtx ctx{m0, n0, tm, tn, split, wm, wn, lane, lds};
  epi(acc, ctx);
}

}  // namespace mshard
