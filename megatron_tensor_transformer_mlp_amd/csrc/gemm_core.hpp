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
//     4 x 4 fp32 32x32 MFMA accumulators (256 accumulation registers per lane).
//   * K advances in steps of 32.  A ring of 4 LDS stages (32 KiB each: the A
//     and B tiles of one step) holds step kt being consumed, kt+1 and kt+2
//     resident or landing, and kt+3 being loaded; the loads of kt+3 are
//     interleaved with the MFMAs of kt.  One barrier per step.
//   * Global -> LDS moves use direct-to-LDS buffer loads (no staging
//     registers); the layouts (see below) make every fragment read
//     conflict-free: K-major tiles are read with ds_read_b128, M/N-major tiles
//     with the transposing ds_read_b64_tr_b16.
//   * MFMA v_mfma_f32_32x32x16_bf16 (16 k per instruction; 2 k steps per LDS
//     stage).  The fragments of k step s+1 are read from LDS while the 16
//     MFMAs of step s run (two fragment register sets).
//   * The MFMA is issued with the B fragment as its first operand and the A
//     fragment as its second, so each lane ends up holding, for every 32x32
//     block, row l%32 and the four 4-column groups 8g + 4*(l/32) .. +3
//     (g = 0..3): row-contiguous 16-byte (fp32) or 8-byte (bf16) output
//     vectors, and per-row reductions need only lanes l and l^32.
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

#include <type_traits>

namespace mshard {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kBM = 256, kBN = 256, kBK = 32;
constexpr int kStages = 4;  // LDS ring: tiles kt+1..kt+3 in flight while kt is consumed
constexpr int kThreads = 256;
constexpr int kWaveM = 128, kWaveN = 128;
constexpr int kSubM = kWaveM / 32, kSubN = kWaveN / 32;  // 32x32 MFMA blocks per wave
constexpr int kStageBytes = (kBM + kBN) * kBK * 2;  // 32 KiB
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
// Global -> LDS: direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds), no
// staging registers.  One instruction moves 64 x 16 bytes into 1 KiB of
// contiguous LDS (lane l -> byte 16*l); each lane chooses which 16-byte global
// chunk lands in its slot, so the LDS layout is free at 16-byte granularity.
// Out-of-range lanes (edge tiles) get an offset beyond the resource and write
// zeros.  A 16 KiB operand tile = 1024 slots = 16 instructions, 4 per wave.
//
// Layouts (16-byte slots; a K-major tile is [256 m/n rows][32 k], an
// M/N-major tile is [32 k rows][256 m/n columns]):
//   K-major : slot(r, c) = (r/16)*64 + c*16 + r%16       c = k/8 (8 k values)
//   MN-major: slot(k, j) = (k/4)*128 + j*4 + k%4         j = col/8 (8 columns)
// LDS serves 16 lanes x 16 bytes (all 64 banks) per cycle.  The K-major layout
// puts 16 consecutive rows of one k chunk in 256 contiguous bytes, so a 16-lane
// ds_read_b128 fragment read is conflict-free; the MN-major layout puts 4
// consecutive k rows of a chunk pair in 128 contiguous bytes (a 16-lane
// ds_read_b64_tr_b16 read is conflict-free).  In both, the fragment address is
// one per-lane base plus compile-time offsets.

typedef __attribute__((address_space(3))) char lds_char;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
constexpr int kTileBytes = kBM * kBK * 2;  // 16 KiB per operand tile
constexpr int kDmaPerWave = kTileBytes / 1024 / 4;

// One buffer_load_dwordx4 ... lds: 64 lanes x 16 bytes from the buffer
// described by `desc` at per-lane byte offsets `off` into 1 KiB of LDS at
// `lds_addr` (wave-uniform; passed in M0).  Issued as inline assembly so the
// compiler's wait-count pass neither tracks nor waits for it: the main loop
// accounts for these loads itself with explicit vmcnt waits (vector-memory
// operations retire in issue order, so the compiler's own waits stay correct).
__device__ __forceinline__ void dma16(u32x4_t desc, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(desc), "s"(lds_addr)
               : "memory", "m0");
}

// Buffer descriptor over [base, base + bytes_left), size clamped below 2^31.
__device__ __forceinline__ u32x4_t make_desc(const void* base, int64_t bytes_left) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t n = bytes_left < 0 ? 0u : (bytes_left > 0x7fffffff ? 0x7fffffffu : (uint32_t)bytes_left);
  return u32x4_t{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, n, kRsrcWord3};
}

// Descriptor of the k tile at k0 of an operand (scalar work, once per tile).
template <bool KMAJOR>
__device__ __forceinline__ u32x4_t tile_desc(const Operand& op, int mn0, int k0) {
  int64_t base_elem;
  if constexpr (KMAJOR) base_elem = (int64_t)mn0 * op.ld + k0;
  else base_elem = (int64_t)k0 * op.ld + mn0;
  return make_desc(op.ptr + base_elem, (op.elems - base_elem) * 2);
}

// Direct-to-LDS instruction i (0 .. kDmaPerWave-1) of this wave's share of one
// operand tile.  The per-lane offset is recomputed each time (a few VALU ops
// that co-issue with the MFMAs) rather than hoisted into long-lived registers.
template <bool KMAJOR>
__device__ __forceinline__ void dma_one(const Operand& op, u32x4_t desc, int mn0, int nmn, int k0, int K,
                                        lds_char* tile, int wave, int lane, int i) {
  asm volatile("" : "+v"(lane));
  const int inst = wave * kDmaPerWave + i;
  uint32_t off;
  if constexpr (KMAJOR) {
    // one 16-row group per instruction: slot l -> row l%16, chunk l/16
    const int r = inst * 16 + (lane & 15), c = lane >> 4;
    const bool ok = (mn0 + r) < nmn && (k0 + c * 8) < K;
    off = ok ? (uint32_t)(((int64_t)r * op.ld + c * 8) * 2) : kOOB;
  } else {
    const int k = (inst >> 1) * 4 + (lane & 3), j = (inst & 1) * 16 + (lane >> 2);
    const bool ok = (k0 + k) < K && (mn0 + j * 8) < nmn;
    off = ok ? (uint32_t)(((int64_t)k * op.ld + j * 8) * 2) : kOOB;
  }
  dma16(desc, off, __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(tile + inst * 1024)));
}

// Direct-to-LDS copy of this wave's share of one operand tile.
template <bool KMAJOR>
__device__ __forceinline__ void dma_tile(const Operand& op, int mn0, int nmn, int k0, int K, lds_char* tile,
                                         int wave, int lane) {
  const u32x4_t desc = tile_desc<KMAJOR>(op, mn0, k0);
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) dma_one<KMAJOR>(op, desc, mn0, nmn, k0, K, tile, wave, lane, i);
}

// Per-lane byte offset of this lane's fragment piece inside a tile (k step 0,
// block 0, wave coordinate 0); the rest of the address is compile-time.
template <bool KMAJOR>
__device__ __forceinline__ int frag_lane_base(int lane) {
  if constexpr (KMAJOR) {
    // row = blk*32 + l%32 -> (row/16)*1024 + (row%16)*16; chunk = 2*ks + l/32 -> chunk*256
    return ((lane & 31) >> 4) * 1024 + (lane >> 5) * 256 + (lane & 15) * 16;
  } else {
    // group g = l/16 (k half g/2, column half g%2); in-group i: q = i%4 (column quad), e = i/4 (k row)
    const int g = lane >> 4, i = lane & 15, q = i & 3, e = i >> 2;
    return e * 16 + (q >> 1) * 64 + (q & 1) * 8 + (g & 1) * 128 + (g >> 1) * 4096;
  }
}

// Fragment of k step ks (16 k) of block blk (32 rows/columns) for wave
// coordinate w: 8 bf16 k values of row/column l%32 at k = 16ks + 8(l/32) + e.
template <bool KMAJOR>
__device__ __forceinline__ bf16x8_t load_frag(const lds_char* tile, int lane_base, int w, int blk, int ks) {
  if constexpr (KMAJOR) {
    return *(const bf16x8_t*)(tile + lane_base + w * 8192 + blk * 2048 + ks * 512);
  } else {
    const lds_char* p = tile + lane_base + w * 1024 + blk * 256 + ks * 8192;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
    const s16x4_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p + 2048));
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
}

struct Frags {
  bf16x8_t a[kSubM];
  bf16x8_t b[kSubN];
};

template <bool AK, bool BK>
__device__ __forceinline__ void load_frags(Frags& f, const lds_char* stage, int ks, int wm, int wn, int la, int lb) {
#pragma unroll
  for (int mi = 0; mi < kSubM; ++mi) f.a[mi] = load_frag<AK>(stage, la, wm, mi, ks);
#pragma unroll
  for (int ni = 0; ni < kSubN; ++ni) f.b[ni] = load_frag<BK>(stage + kTileBytes, lb, wn, ni, ks);
}

// The MFMA is written as inline assembly with accumulation-register operands so
// that the 256 accumulators are pinned to the accumulation registers for their
// whole life (compiler-selected forms end up copying them between register
// files every iteration).  Hazards: a given accumulator is re-used only after
// the 15 other MFMAs of the k step; fragment registers come from LDS loads,
// which the wait-count pass tracks through the asm operands; the first read
// after the loop is fenced with explicit wait states.
template <bool FIRST>
__device__ __forceinline__ void mfma_32x32x16(f32x16_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  if constexpr (FIRST)  // the first k step starts from C = 0 (inline constant): no zero fill
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// The 16 MFMAs of one k step; after each group of 4 (one A row block), calls
// between(mi) so that other work (direct-to-LDS issue) interleaves with them.
template <bool FIRST, class Between>
__device__ __forceinline__ void mfma_frags(f32x16_t (&acc)[kSubM][kSubN], const Frags& f, Between&& between) {
#pragma unroll
  for (int mi = 0; mi < kSubM; ++mi) {
#pragma unroll
    for (int ni = 0; ni < kSubN; ++ni) mfma_32x32x16<FIRST>(acc[mi][ni], f.b[ni], f.a[mi]);
    between(mi);
  }
}

// Position of accumulator element acc[mi][ni][4g + r] inside the 256 x 256 tile:
//   row = wm*128 + mi*32 + (lane & 31),
//   col = wn*128 + ni*32 + 8g + 4*(lane >> 5) + r        (g, r = 0..3).
// LDS store of 4 accumulators straight from their accumulation registers.
// Every non-MFMA use of the accumulators is this or a buffer store, so they
// stay in the accumulation registers for the whole main loop.  LDS operations
// of a wave complete in order, so later LDS reads of the same bytes see the data.
__device__ __forceinline__ void acc_store_lds(char* p, f32x4_t a) {
  // generic (flat) pointer the compiler cannot narrow to LDS: a flat store, whose
  // data operand may be an accumulation register, like a buffer store's
  asm volatile("" : "+v"(p));
  *(f32x4_t*)p = a;
}

// Wait states between the last MFMA and the first explicit accumulator read
// (covers the longest MFMA result latency).
__device__ __forceinline__ void acc_settle() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n s_nop 7\n s_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

struct EpiCtx {
  int m0, n0;   // tile origin in C
  int tm, tn;   // tile coordinates
  int split;    // K split index
  int wm, wn;   // wave coordinates in the tile
  int lane;
  char* lds0;   // the four 32 KiB LDS stages, free for the epilogue after the main loop
  char* lds1;
  char* lds2;
  char* lds3;
};

// s_waitcnt with only the vector-memory count: wait until at most n of this
// wave's vector memory operations (here: direct-to-LDS loads) are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  static_assert(kDmaPerWave == kSubM, "one DMA instruction per A row block of MFMAs");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Make every 32-bit word of a kernel-argument struct live in scalar registers
// here.  Scalar memory loads complete out of order, so one left outstanding
// across the main loop (the compiler likes to hoist the epilogue's argument
// loads) would turn every LDS wait in the loop into a full drain.
template <class T>
__device__ __forceinline__ void args_to_sgprs(const T& t) {
  static_assert(sizeof(T) % 4 == 0, "word-sized argument struct");
  const uint32_t* w = (const uint32_t*)&t;
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" ::"s"(w[i]));
}

template <bool A_KMAJOR, bool B_KMAJOR, class Epi>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
gemm_kernel(GemmGeom g, Operand a, Operand b, Epi epi) {
  args_to_sgprs(g);
  args_to_sgprs(a);
  args_to_sgprs(b);
  args_to_sgprs(epi);
  // Four LDS stages (A tile then B tile in each), kept as separate objects so
  // that the direct-to-LDS writes into one stage are known not to alias the
  // fragment reads of another.
  __shared__ __attribute__((aligned(1024))) char lds0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds1[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds2[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char lds3[kStageBytes];
  lds_char* st[kStages] = {(lds_char*)lds0, (lds_char*)lds1, (lds_char*)lds2, (lds_char*)lds3};
  int tm, tn, split;
  map_tile(g, tm, tn, split);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int nk = (g.K + kBK - 1) / kBK;
  const int kt_beg = (int)(((int64_t)split * nk) / g.splits);
  const int kt_end = (int)(((int64_t)(split + 1) * nk) / g.splits);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int la = frag_lane_base<A_KMAJOR>(lane), lb = frag_lane_base<B_KMAJOR>(lane);

  f32x16_t acc[kSubM][kSubN];

  auto dma = [&](int kt, lds_char* stage) {
    dma_tile<A_KMAJOR>(a, m0, g.M, kt * kBK, g.K, stage, wave, lane);
    dma_tile<B_KMAJOR>(b, n0, g.N, kt * kBK, g.K, stage + kTileBytes, wave, lane);
  };
  constexpr int kPerTile = 2 * kDmaPerWave;  // direct-to-LDS instructions per wave per tile

  // One k tile from stage `cur` (2 k steps of 16).  Invariant at entry: tiles
  // kt and kt+1 are published (complete in LDS for every wave) and the first
  // k step's fragments of tile kt are in f[0].  The DMA of tile kt+3 goes into
  // the stage consumed at kt-1; the second k step's fragments of tile kt are
  // read under the first step's MFMAs, and the first step's fragments of tile
  // kt+1 under the second step's.  Then this wave waits for its share of tile
  // kt+2 (tile kt+3 may stay in flight) and the barrier publishes it; that
  // barrier also orders every read of stage kt before its reuse at kt+1.
  // The host guarantees kt_beg < kt_end.
  auto step = [&](auto first, const lds_char* cur, const lds_char* nxt, lds_char* far, int kt, Frags (&f)[2]) {
    constexpr bool kFirst = decltype(first)::value;
    const bool issue = kt + 3 < kt_end;
    const int k3 = (kt + 3) * kBK;
    const u32x4_t da = tile_desc<A_KMAJOR>(a, m0, k3);
    const u32x4_t db = tile_desc<B_KMAJOR>(b, n0, k3);
    // one direct-to-LDS instruction after every 4 MFMAs: A's share under the
    // first k step, B's under the second
    auto dma_a = [&](int q) {
      if (issue) dma_one<A_KMAJOR>(a, da, m0, g.M, k3, g.K, far, wave, lane, q);
    };
    auto dma_b = [&](int q) {
      if (issue) dma_one<B_KMAJOR>(b, db, n0, g.N, k3, g.K, far + kTileBytes, wave, lane, q);
    };
    load_frags<A_KMAJOR, B_KMAJOR>(f[1], cur, 1, wm, wn, la, lb);
    if constexpr (kFirst) mfma_frags<true>(acc, f[0], dma_a);
    else mfma_frags<false>(acc, f[0], dma_a);
    if (kt + 1 < kt_end) load_frags<A_KMAJOR, B_KMAJOR>(f[0], nxt, 0, wm, wn, la, lb);
    mfma_frags<false>(acc, f[1], dma_b);
    if (issue) wait_vmcnt<kPerTile>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };
  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;

  dma(kt_beg, st[0]);
  if (kt_beg + 1 < kt_end) dma(kt_beg + 1, st[1]);
  if (kt_beg + 2 < kt_end) dma(kt_beg + 2, st[2]);
  if (kt_beg + 2 < kt_end) wait_vmcnt<kPerTile>();  // tiles kt_beg, kt_beg+1 done
  else wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  Frags f[2];
  load_frags<A_KMAJOR, B_KMAJOR>(f[0], st[0], 0, wm, wn, la, lb);
  step(True{}, st[0], st[1], st[3], kt_beg, f);
  for (int kt = kt_beg + 1; kt < kt_end; kt += 4) {
    step(False{}, st[1], st[2], st[0], kt, f);
    if (kt + 1 < kt_end) step(False{}, st[2], st[3], st[1], kt + 1, f);
    if (kt + 2 < kt_end) step(False{}, st[3], st[0], st[2], kt + 2, f);
    if (kt + 3 < kt_end) step(False{}, st[0], st[1], st[3], kt + 3, f);
  }
  EpiCtx ctx{m0, n0, tm, tn, split, wm, wn, lane, lds0, lds1, lds2, lds3};
  epi(acc, ctx);
}

}  // namespace mshard
