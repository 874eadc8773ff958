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
//     8 x 8 fp32 16x16 MFMA accumulators (256 accumulation registers per lane).
//   * K advances in steps of 32.  Each operand has a ring in LDS (128 KiB in
//     all): an M/N-major operand four 16 KiB stages, one k tile each; a
//     K-major operand two 32 KiB pair slots, two k tiles each, so that its
//     loads read whole 128-byte rows.  Step kt consumes tile kt while kt+1 and
//     kt+2 are resident or landing and the loads of kt+3 (M/N-major), or on
//     every other step of the pair kt+3, kt+4 (K-major), run interleaved with
//     its MFMAs.  One barrier per step.
//   * Global -> LDS moves use direct-to-LDS buffer loads (no staging
//     registers); the layouts (see below) make every fragment read
//     conflict-free: K-major tiles are read with ds_read_b128, M/N-major tiles
//     with the transposing ds_read_b64_tr_b16.
//   * MFMA v_mfma_f32_16x16x32_bf16 (32 k per instruction: one per LDS
//     stage and 16x16 block).  The fragments of k tile kt+1 are read from LDS
//     while the 64 MFMAs of tile kt run (two fragment register sets).
//   * The MFMA is issued with the B fragment as its first operand and the A
//     fragment as its second, so each lane ends up holding, for every 16x16
//     block, row l%16 and the 4 columns 4*(l/16) .. +3: row-contiguous
//     16-byte (fp32) or 8-byte (bf16) output vectors.  The four lanes
//     l%16 + 16g share a row, so per-row reductions exchange over lanes l^16
//     and l^32.
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
#include <utility>

namespace mshard {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kBM = 256, kBN = 256, kBK = 32;
// Wave grid of a workgroup: kWavesM x kWavesN waves, each owning a
// kWaveM x kWaveN sub-tile of the 256 x 256 tile.
constexpr int kWavesM = 2, kWavesN = 2;
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kThreads = 64 * kWaves;
constexpr int kWavesPerSimd = kWaves / 4;  // a CU has 4 SIMDs
constexpr int kWaveM = kBM / kWavesM, kWaveN = kBN / kWavesN;
constexpr int kSubM = kWaveM / 16, kSubN = kWaveN / 16;  // 16x16 MFMA blocks per wave
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

// Buffer loads and stores with cache-policy bits POLICY (0: default;
// kNonTemporal: the non-temporal hint).  Outputs that the next kernel does not
// read back from the caches (the fp32 partials Z and dX, the weight gradients,
// split-K slices, the CE backward's logit gradient, which is larger than the
// MALL) are stored non-temporally, and data read exactly once (H in the GeLU'
// epilogue, the split-K slices and CE tile partials in the reductions) is
// loaded non-temporally: measured 1.0-3.6% faster steps at the rank-shard
// workloads, 0.8% on the GPT-2 MLP and 2% on the CE backward.  H, Y and dH,
// which the next GEMM reads while they are still cached, are stored with the
// default (non-temporal there was 1% slower).
constexpr int kNonTemporal = 2;  // the nt bit of a buffer access's cache policy on gfx950
template <int POLICY = 0>
__device__ __forceinline__ u32x2_t buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, POLICY);
}
template <int POLICY = 0>
__device__ __forceinline__ void buf_store16(u32x4_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, POLICY);
}
template <int POLICY = 0>
__device__ __forceinline__ void buf_store8(u32x2_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, POLICY);
}
template <int POLICY = 0>
__device__ __forceinline__ void buf_store4(uint32_t v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, POLICY);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even
// (one v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
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
// `b` and `G` are the block's index and the block count of this GEMM within
// the launch; the first block of each GEMM sits on XCD 0 (callers keep every
// GEMM's first block index a multiple of 8).
__device__ __forceinline__ void map_tile(const GemmGeom& g, int b, int G, int& tm, int& tn, int& split) {
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
// zeros.
//
// An operand stored K-major is loaded two k tiles at a time: a pair of k
// tiles is [256 m/n rows][64 k], whose 128-byte rows are whole cache lines
// (one k tile's 64-byte rows would each be half a line, fetched twice, and
// the memory path pays per request, not per byte: loading whole lines made
// the CE GEMM about 5% faster).  Pairs live in two 32 KiB pair slots.  An
// operand stored M/N-major is loaded one k tile ([32 k rows][256 m/n]) per
// step into four 16 KiB stages; its 512-byte k rows are whole lines already.
// The four 32 KiB LDS arrays hold, in order, the pair slots of each K-major
// operand (A first) and then the stages of each M/N-major one, two 16 KiB
// stages per array; with both operands M/N-major, array s holds stage s of A
// then stage s of B.
//
// Layouts (16-byte slots):
//   K-major pair : slot(r, c) = r*8 + (c ^ (r % 8))     c = k/8 (0..7 over the pair's 64 k)
//   MN-major tile: slot(k, j) = k*32 + (j ^ 2*((k%4) | 4*((k/8)%2)))
//                                                       j = col/8 (8 columns)
// Rows (K-major) and k rows (M/N-major) are contiguous, so each load
// instruction's 64 lanes read 8 whole 128-byte rows or 2 whole 512-byte k
// rows.  The XOR terms only permute slots within a row; they make the
// fragment reads conflict-free.  A ds_read_b128 is served 8 lanes at a time,
// whose 16-byte chunks must lie in different 16-byte slots of a 128-byte
// window: a K-major fragment reads one chunk of 8 consecutive rows, which the
// XOR with r % 8 spreads over the 8 slots of the window (with two rows per
// slot the read runs at half rate: measured on gfx950, 128 versus 250 bytes
// per clock per CU).  The 8 k rows x 32 bytes that 32 lanes of an M/N-major
// transposing read touch fall in 8 different 32-byte windows.

typedef __attribute__((address_space(3))) char lds_char;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
constexpr int kTileBytes = kBM * kBK * 2;  // 16 KiB per operand tile
constexpr int kPairBytes = 2 * kTileBytes;  // a K-major operand's pair slot: two k tiles
constexpr int kDmaPerWave = kTileBytes / 1024 / kWaves;  // direct-to-LDS instructions per wave per operand tile
static_assert(kDmaPerWave == 1 || kDmaPerWave == 2 || kDmaPerWave == 4, "layout offsets assume 1, 2 or 4");

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
// Resource for one operand tile whose origin is (mn0, k0): it starts at the
// tile origin and ends at the end of the stored matrix.  A K-major tile's rows
// past M and an M/N-major tile's k rows past K therefore lie beyond the end and
// read as zeros without any lane mask.
template <bool KMAJOR>
__device__ __forceinline__ u32x4_t tile_desc(const Operand& op, int mn0, int k0) {
  int64_t base_elem;
  if constexpr (KMAJOR) base_elem = (int64_t)mn0 * op.ld + k0;
  else base_elem = (int64_t)k0 * op.ld + mn0;
  // every operand is smaller than 2^31 bytes and the origin lies inside it
  const uint64_t p = (uint64_t)(uintptr_t)(op.ptr + base_elem);
  return u32x4_t{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, (uint32_t)((op.elems - base_elem) * 2), kRsrcWord3};
}

// Loop-invariant per-lane byte offsets of one operand's direct-to-LDS loads,
// relative to the tile (K-major: pair) origin:
//   K-major:   instruction i of this wave (0 .. 2*kDmaPerWave-1) at offset
//              v[0] + i * step, or kOOB when the lane's k chunk (k offset v[1]
//              within the pair) lies past K;
//   M/N-major: instruction i at v[i % 2] + i * step    (columns past M/N masked).
// The host keeps every leading dimension below 2^22 elements, so no offset of
// a 256-row tile wraps 32 bits and a masked offset (kOOB + up to 7 steps)
// stays out of range.
struct DmaLanes {
  uint32_t v[2];
  uint32_t step;
};

template <bool KMAJOR>
__device__ __forceinline__ DmaLanes dma_lanes(const Operand& op, int mn0, int nmn, int K, int wave, int lane) {
  DmaLanes d;
  const uint32_t ldb = (uint32_t)op.ld * 2u;
  if constexpr (KMAJOR) {
    // instruction 2D*w + i (D = kDmaPerWave) writes slots (2D*w + i)*64 + l:
    // row (2D*w + i)*8 + l/8, chunk (l%8) ^ (l/8)  (the row's index mod 8 is l/8)
    const uint32_t r = (uint32_t)wave * (16u * kDmaPerWave) + (uint32_t)(lane >> 3);
    const int c = (lane & 7) ^ (lane >> 3);
    d.v[0] = r * ldb + (uint32_t)c * 16u;
    d.v[1] = (uint32_t)c * 8u;
    d.step = 8u * ldb;
  } else {
    // instruction D*w + i (D = kDmaPerWave) writes slots (D*w + i)*64 + l:
    // k row 2Dw + 2i + l/32 and column group (l%32) ^ 2F with
    // F = ((2i + l/32) % 4) | 4*((2Dw/8) % 2); F depends on i only through i%2
    const uint32_t k = (uint32_t)wave * (2u * kDmaPerWave) + (uint32_t)(lane >> 5);
    const int k8 = ((wave * 2 * kDmaPerWave) >> 3) & 1;
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int F = ((2 * par + (lane >> 5)) & 3) | (k8 << 2);
      const int j = (lane & 31) ^ (2 * F);
      d.v[par] = (mn0 + j * 8 < nmn) ? k * ldb + (uint32_t)j * 16u : kOOB;
    }
    d.step = 2u * ldb;
  }
  return d;
}

// K-major: the lane's base offset for the pair whose first k is k0 (masked when
// its chunk lies past K).  Computed once per pair.
__device__ __forceinline__ uint32_t dma_pair_base(const DmaLanes& d, int k0, int K) {
  return (int)d.v[1] < K - k0 ? d.v[0] : kOOB;
}

// Direct-to-LDS instruction i of this wave's share of one pair (K-major, `base`
// from dma_pair_base) or one tile (M/N-major).  `dst` is the pair slot's or the
// stage's LDS address; `wave_s` the wave index (uniform).
template <bool KMAJOR>
__device__ __forceinline__ void dma_one(const DmaLanes& d, u32x4_t desc, uint32_t base, uint32_t dst, int wave_s,
                                        int i) {
  if constexpr (KMAJOR)
    dma16(desc, base + (uint32_t)i * d.step, dst + (uint32_t)wave_s * (2 * kDmaPerWave * 1024u) + (uint32_t)i * 1024u);
  else
    dma16(desc, d.v[i & 1] + (uint32_t)i * d.step, dst + (uint32_t)wave_s * (kDmaPerWave * 1024u) + (uint32_t)i * 1024u);
}

// All of this wave's loads of one pair (K-major, first k at k0) or one tile.
template <bool KMAJOR>
__device__ __forceinline__ void dma_unit(const Operand& op, const DmaLanes& d, int mn0, int k0, int K, uint32_t dst,
                                         int wave_s) {
  const u32x4_t desc = tile_desc<KMAJOR>(op, mn0, k0);
  const uint32_t base = KMAJOR ? dma_pair_base(d, k0, K) : 0u;
#pragma unroll
  for (int i = 0; i < (KMAJOR ? 2 : 1) * kDmaPerWave; ++i) dma_one<KMAJOR>(d, desc, base, dst, wave_s, i);
}

// Fragments for v_mfma_f32_16x16x32_bf16.  Lane l holds 8 bf16 values of one
// row (A) or column (B) of a 16-wide block: row/column l%16, k = 8*(l/16) + e
// for e = 0..7, as two 4-value halves (k 8g..8g+3 and 8g+4..8g+7, g = l/16).
// Both operands use the same lane -> k assignment, which is all the product
// over k requires.
//   K-major pair: a block's fragment for one k tile of the pair is its 16
//     rows x 4 chunks (chunks 4h..4h+3 of each row for k tile h of the pair):
//     one ds_read_b128 per fragment.
//   M/N-major tile: each half is one ds_read_b64_tr_b16.  Within a 16-lane
//     group, lane x = 4e + q supplies the address of k row 8g + 4h + e,
//     columns 4q..4q+3 of the block, and the instruction hands lane i the
//     values of column i for the four k rows.
struct Frag {
  s16x4_t lo, hi;
};

__device__ __forceinline__ bf16x8_t frag_value(const Frag& f) {
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(f.lo, f.hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// SUB: the 16-wide blocks of this operand one wave covers (kSubM for A, kSubN for B).
template <bool KMAJOR, int SUB>
struct FragBase {
  int x[KMAJOR ? 2 : SUB];  // K-major: a lane base per k tile of the pair; M/N-major: one per 16-column block
};

template <bool KMAJOR, int SUB>
__device__ __forceinline__ FragBase<KMAJOR, SUB> frag_lane_base(int lane) {
  FragBase<KMAJOR, SUB> fb;
  if constexpr (KMAJOR) {
    // row l%16 of the block (its index mod 8 is (l%16)%8), chunk 4h + l/16 of the pair
#pragma unroll
    for (int h = 0; h < 2; ++h)
      fb.x[h] = (lane & 15) * 128 + ((4 * h + (lane >> 4)) ^ (lane & 7)) * 16;
  } else {
    // lane x = 4e + q of group g: k row 8g + e (+ 4h), columns 4q..4q+3 of the
    // block; the layout's XOR moves block b to position b ^ F within the row
    const int g = lane >> 4, x = lane & 15, e = x >> 2, q = x & 3;
    const int F = e | ((g & 1) << 2);
    const int base = (8 * g + e) * 512 + F * 32 + (q >> 1) * 16 + (q & 1) * 8;
#pragma unroll
    for (int blk = 0; blk < SUB; ++blk) fb.x[blk] = base ^ (blk * 32);
  }
  return fb;
}

// Pieces (LDS read instructions) per fragment.
template <bool KMAJOR>
constexpr int kPieces = KMAJOR ? 1 : 2;

// Read piece h of the fragment of block blk (0..SUB-1) for wave coordinate w;
// `half` (K-major): which k tile of the pair in `tile` (a pair slot).
// M/N-major: the wave's first block is block w*SUB of the 16 in a k row, and
// the layout's XOR acts on the block index (bits 5-8 of the byte offset), so
// the wave offset is XORed in too.
template <bool KMAJOR, int SUB>
__device__ __forceinline__ void read_piece(Frag& f, const lds_char* tile, int half, const FragBase<KMAJOR, SUB>& fb,
                                           int w, int blk, int h) {
  if constexpr (KMAJOR) {
    const s16x8_t v = *(const s16x8_t*)(tile + fb.x[half] + (w * SUB + blk) * 2048);
    f.lo = __builtin_shufflevector(v, v, 0, 1, 2, 3);
    f.hi = __builtin_shufflevector(v, v, 4, 5, 6, 7);
  } else {
    const lds_char* p = tile + (fb.x[blk] ^ (w * SUB * 32)) + h * 2048;
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)p);
    if (h == 0) f.lo = v;
    else f.hi = v;
  }
}

struct Frags {
  Frag a[kSubM];
  Frag b[kSubN];
};

// Order in which the fragments of a tile are read: A block 0, then every B
// block, then A blocks 1.. -- the order in which the MFMA sequence (A block
// outer, B block inner) first needs them.
template <bool AK, bool BK>
struct ReadOrder {
  static constexpr int PA = kPieces<AK>, PB = kPieces<BK>;
  static constexpr int P = PA * kSubM + PB * kSubN;
  static constexpr int kMfma = kSubM * kSubN;
  // piece p is issued right after MFMA number slot(p) (spread over the first 3/4 of them)
  static constexpr int slot(int p) { return (p * (3 * kMfma / 4)) / P; }
  static constexpr int piece_at(int j) {
    for (int p = 0; p < P; ++p)
      if (slot(p) == j) return p;
    return -1;
  }
};

// Where one k tile of each operand sits in LDS: the pair slot and half
// (K-major) or the stage (M/N-major, half 0).
struct TileSrc {
  const lds_char* a;
  const lds_char* b;
  int ha, hb;
};

template <bool AK, bool BK, int p>
__device__ __forceinline__ void read_piece_p(Frags& f, const TileSrc& t, const FragBase<AK, kSubM>& fa,
                                             const FragBase<BK, kSubN>& fb, int wm, int wn) {
  using R = ReadOrder<AK, BK>;
  if constexpr (p < R::PA) {
    read_piece<AK, kSubM>(f.a[0], t.a, t.ha, fa, wm, 0, p);
  } else if constexpr (p < R::PA + kSubN * R::PB) {
    constexpr int q = p - R::PA;
    read_piece<BK, kSubN>(f.b[q / R::PB], t.b, t.hb, fb, wn, q / R::PB, q % R::PB);
  } else {
    constexpr int q = p - R::PA - kSubN * R::PB;
    read_piece<AK, kSubM>(f.a[1 + q / R::PA], t.a, t.ha, fa, wm, 1 + q / R::PA, q % R::PA);
  }
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <bool AK, bool BK>
__device__ __forceinline__ void read_all(Frags& f, const TileSrc& t, const FragBase<AK, kSubM>& fa,
                                         const FragBase<BK, kSubN>& fb, int wm, int wn) {
  static_for<ReadOrder<AK, BK>::P>([&](auto pc) { read_piece_p<AK, BK, decltype(pc)::value>(f, t, fa, fb, wm, wn); });
}

// The MFMA is written as inline assembly with accumulation-register operands so
// that the 256 accumulators are pinned to the accumulation registers for their
// whole life (compiler-selected forms end up copying them between register
// files every iteration).  A given accumulator is re-used only after the
// kSubM*kSubN - 1 other MFMAs of the tile; fragment registers come from LDS loads, which the
// wait-count pass tracks through the asm operands; the first read of the
// accumulators after the loop is fenced with explicit wait states.
template <bool FIRST>
__device__ __forceinline__ void mfma_16x16x32(f32x4_t& acc, const bf16x8_t& a, const bf16x8_t& b) {
  if constexpr (FIRST)  // the first k tile starts from C = 0 (inline constant): no zero fill
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

typedef f32x4_t AccTile[kSubM][kSubN];

// Position of accumulator element acc[mi][ni][r] inside the 256 x 256 tile
// (the MFMA takes the B fragment as its first operand, so the hardware's row
// index is the tile's column):
//   row = wm*128 + mi*16 + (lane & 15),
//   col = wn*128 + ni*16 + 4*(lane >> 4) + r        (r = 0..3).
// LDS store of 4 accumulators straight from their accumulation registers: a
// ds_write_b128 whose data operand is the accumulation-register quad, so the
// accumulators stay in the accumulation registers for the whole main loop and
// no copy to ordinary registers is made.  Written as inline assembly, it is
// not tracked by the compiler's wait-count pass: callers wait for lgkmcnt(0)
// before the staged bytes are read.
__device__ __forceinline__ void acc_store_lds(char* p, const f32x4_t& a) {
  const uint32_t addr = (uint32_t)(uintptr_t)(lds_char*)p;
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "a"(a) : "memory");
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
  char* xch;    // small cross-wave exchange buffer (lds0 unless the kernel gives one of its own)
};

// s_waitcnt with only the vector-memory count: wait until at most n of this
// wave's vector memory operations (here: direct-to-LDS loads) are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
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

// The LDS homes of the two operands (see the layout notes above): K-major
// operands have two 32 KiB pair slots p[0..1], M/N-major ones four 16 KiB
// stages p[0..3].
template <bool AK, bool BK>
struct LdsRing {
  lds_char* a[4];
  lds_char* b[4];
};

template <bool AK, bool BK>
__device__ __forceinline__ LdsRing<AK, BK> lds_ring(char* lds0, char* lds1, char* lds2, char* lds3) {
  lds_char* l[4] = {(lds_char*)lds0, (lds_char*)lds1, (lds_char*)lds2, (lds_char*)lds3};
  LdsRing<AK, BK> r;
  if constexpr (!AK && !BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.a[i] = l[i];
      r.b[i] = l[i] + kTileBytes;
    }
  } else {
    // pair slots of the K-major operand(s) first, then the stages of an M/N-major one
    lds_char** kop = AK ? r.a : r.b;  // A if it is K-major, else B
    kop[0] = l[0];
    kop[1] = l[1];
    kop[2] = kop[3] = nullptr;
    lds_char** other = AK ? r.b : r.a;
    if constexpr (AK && BK) {
      other[0] = l[2];
      other[1] = l[3];
      other[2] = other[3] = nullptr;
    } else {
      other[0] = l[2];
      other[1] = l[2] + kTileBytes;
      other[2] = l[3];
      other[3] = l[3] + kTileBytes;
    }
  }
  return r;
}

// Direct-to-LDS instructions per wave one operand issues at a k step of the
// given parity (of the step's index counted from the tile's first k step):
// a K-major operand loads a pair on odd steps, an M/N-major one a tile on every step.
template <bool KMAJOR>
constexpr int dma_count(bool odd) { return KMAJOR ? (odd ? 2 * kDmaPerWave : 0) : kDmaPerWave; }

// The q-th of cnt direct-to-LDS instructions of a step is issued after MFMA
// number ((q + 1) * 64) / cnt - 1; returns the q issued after MFMA j, or -1.
constexpr int dma_at(int j, int cnt, int nmfma) {
  for (int q = 0; q < cnt; ++q)
    if (((q + 1) * nmfma) / cnt - 1 == j) return q;
  return -1;
}

// The k loop of one tile (or K split), shared by the per-tile and the
// persistent kernels: local k step i = 0 .. n-1 (global kt_beg + i).
//
// Ring: local k tile t sits in pair slot (t/2)%2, half t%2 (K-major operand)
// or stage t%4 (M/N-major).  Step i runs the 64 MFMAs of tile i on fragments
// fc, reads the fragments of tile i+1 into fn, and issues the loads of tile
// i+3 (M/N-major) and, on odd i, of the pair of tiles i+3 and i+4 (K-major).
// Each slot or stage it loads into was last read in step i-2 or earlier (as
// fragments of tiles i-1 or i).  It then waits until only its own loads are
// outstanding, so tile i+2 has landed, and the barrier publishes it; the
// barrier also orders every read of a slot or stage before the step that
// loads into it again.  At entry: tiles 0 and 1 are published and tile 2
// (with the rest of its pair) may be landing.
template <bool AK, bool BK>
__device__ __forceinline__ void tile_k_loop(AccTile& acc, const GemmGeom& g, const Operand& a, const Operand& b,
                                            int m0, int n0, int kt_beg, int n, const DmaLanes& dla,
                                            const DmaLanes& dlb, const LdsRing<AK, BK>& R, int wave_s, int wm, int wn,
                                            int lane) {
  const FragBase<AK, kSubM> fra = frag_lane_base<AK, kSubM>(lane);
  const FragBase<BK, kSubN> frb = frag_lane_base<BK, kSubN>(lane);
  using RO = ReadOrder<AK, BK>;
  constexpr int kMfma = kSubM * kSubN;
  auto lds_addr = [](const lds_char* q) { return (uint32_t)(uintptr_t)q; };
  // LDS home of local tile t, for t with t % 4 == T4 (compile time)
  auto src = [&](auto t4) {
    constexpr int T4 = decltype(t4)::value;
    TileSrc ts;
    ts.a = AK ? R.a[(T4 >> 1) & 1] : R.a[T4 & 3];
    ts.b = BK ? R.b[(T4 >> 1) & 1] : R.b[T4 & 3];
    ts.ha = AK ? (T4 & 1) : 0;
    ts.hb = BK ? (T4 & 1) : 0;
    return ts;
  };
  // step i with i % 4 == POS (compile time)
  auto step = [&](auto first, auto checked, auto posc, int i, Frags& fc, Frags& fn) {
    constexpr bool kFirst = decltype(first)::value;
    constexpr bool kChecked = decltype(checked)::value;
    constexpr int POS = decltype(posc)::value;
    constexpr bool kOdd = (POS & 1) != 0;
    constexpr int cA = dma_count<AK>(kOdd), cB = dma_count<BK>(kOdd), cnt = cA + cB;
    const bool issue = !kChecked || i + 3 < n;
    const bool next = !kChecked || i + 1 < n;
    const TileSrc nx = src(std::integral_constant<int, (POS + 1) & 3>{});
    const int k3 = (kt_beg + i + 3) * kBK;
    u32x4_t da = {0u, 0u, 0u, 0u}, db = {0u, 0u, 0u, 0u};
    uint32_t baseA = 0u, baseB = 0u, dstA = 0u, dstB = 0u;
    if constexpr (cA > 0) {
      da = tile_desc<AK>(a, m0, k3);
      if constexpr (AK) baseA = dma_pair_base(dla, k3, g.K);
      dstA = lds_addr(AK ? R.a[((POS + 3) >> 1) & 1] : R.a[(POS + 3) & 3]);
    }
    if constexpr (cB > 0) {
      db = tile_desc<BK>(b, n0, k3);
      if constexpr (BK) baseB = dma_pair_base(dlb, k3, g.K);
      dstB = lds_addr(BK ? R.b[((POS + 3) >> 1) & 1] : R.b[(POS + 3) & 3]);
    }
    static_for<kMfma>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int mi = j / kSubN, ni = j % kSubN;
      mfma_16x16x32<kFirst>(acc[mi][ni], frag_value(fc.b[ni]), frag_value(fc.a[mi]));
      constexpr int p = RO::piece_at(j);
      if constexpr (p >= 0) {
        if (next) read_piece_p<AK, BK, p>(fn, nx, fra, frb, wm, wn);
      }
      constexpr int q = dma_at(j, cnt, kMfma);
      if constexpr (q >= 0) {
        if (issue) {
          if constexpr (q < cA) dma_one<AK>(dla, da, baseA, dstA, wave_s, q);
          else dma_one<BK>(dlb, db, baseB, dstB, wave_s, q - cA);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if (issue) wait_vmcnt<cnt>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
  };
  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  using P2 = std::integral_constant<int, 2>;
  using P3 = std::integral_constant<int, 3>;

  Frags f0, f1;
  read_all<AK, BK>(f0, src(P0{}), fra, frb, wm, wn);
  step(True{}, True{}, P0{}, 0, f0, f1);
  int i = 1;
  // steady state: every step of the group reads its next tile and issues its loads
  for (; i + 6 < n; i += 4) {
    step(False{}, False{}, P1{}, i, f1, f0);
    step(False{}, False{}, P2{}, i + 1, f0, f1);
    step(False{}, False{}, P3{}, i + 2, f1, f0);
    step(False{}, False{}, P0{}, i + 3, f0, f1);
  }
  for (; i < n; i += 4) {
    step(False{}, True{}, P1{}, i, f1, f0);
    if (i + 1 < n) step(False{}, True{}, P2{}, i + 1, f0, f1);
    if (i + 2 < n) step(False{}, True{}, P3{}, i + 2, f1, f0);
    if (i + 3 < n) step(False{}, True{}, P0{}, i + 3, f0, f1);
  }
}

// The loads of local k tiles 0, 1 and 2 (K-major: pairs 0 and 1), in an order
// that lets the caller wait for tiles 0 and 1 alone: tile 2's loads
// (dma_count<AK>(true) + dma_count<BK>(true) per wave when n > 2) are last.
template <bool AK, bool BK>
__device__ __forceinline__ void tile_first_loads(const GemmGeom& g, const Operand& a, const Operand& b, int m0, int n0,
                                                 int kt_beg, int n, const DmaLanes& dla, const DmaLanes& dlb,
                                                 const LdsRing<AK, BK>& R, int wave_s) {
  auto lds_addr = [](const lds_char* q) { return (uint32_t)(uintptr_t)q; };
  const int k0 = kt_beg * kBK;
  dma_unit<AK>(a, dla, m0, k0, g.K, lds_addr(R.a[0]), wave_s);
  dma_unit<BK>(b, dlb, n0, k0, g.K, lds_addr(R.b[0]), wave_s);
  if (n > 1) {
    if constexpr (!AK) dma_unit<false>(a, dla, m0, k0 + kBK, g.K, lds_addr(R.a[1]), wave_s);
    if constexpr (!BK) dma_unit<false>(b, dlb, n0, k0 + kBK, g.K, lds_addr(R.b[1]), wave_s);
  }
  if (n > 2) {
    // K-major: the pair of tiles 2 and 3 into slot 1; M/N-major: tile 2 into stage 2
    dma_unit<AK>(a, dla, m0, k0 + 2 * kBK, g.K, lds_addr(R.a[AK ? 1 : 2]), wave_s);
    dma_unit<BK>(b, dlb, n0, k0 + 2 * kBK, g.K, lds_addr(R.b[BK ? 1 : 2]), wave_s);
  }
}

// One 256 x 256 output tile (or one K split of it): block `vb` of the `vg`
// blocks this GEMM has in the launch.  lds0..lds3 are the kernel's four
// 32 KiB LDS arrays (the operands' pair slots and stages).
template <bool A_KMAJOR, bool B_KMAJOR, class Epi>
__device__ __forceinline__ void gemm_tile(const GemmGeom& g, const Operand& a, const Operand& b, const Epi& epi,
                                          int vb, int vg, char* lds0, char* lds1, char* lds2, char* lds3) {
  args_to_sgprs(g);
  args_to_sgprs(a);
  args_to_sgprs(b);
  args_to_sgprs(epi);
  const LdsRing<A_KMAJOR, B_KMAJOR> R = lds_ring<A_KMAJOR, B_KMAJOR>(lds0, lds1, lds2, lds3);
  int tm, tn, split;
  map_tile(g, vb, vg, tm, tn, split);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int nk = (g.K + kBK - 1) / kBK;
  const int kt_beg = (int)(((int64_t)split * nk) / g.splits);
  const int kt_end = (int)(((int64_t)(split + 1) * nk) / g.splits);
  const int n = kt_end - kt_beg;  // >= 1 (the host guarantees kt_beg < kt_end)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // uniform copy for scalar address math
  const int wm = wave / kWavesN, wn = wave % kWavesN;
  const DmaLanes dla = dma_lanes<A_KMAJOR>(a, m0, g.M, g.K, wave_s, lane);
  const DmaLanes dlb = dma_lanes<B_KMAJOR>(b, n0, g.N, g.K, wave_s, lane);

  AccTile acc;
  tile_first_loads<A_KMAJOR, B_KMAJOR>(g, a, b, m0, n0, kt_beg, n, dla, dlb, R, wave_s);
  constexpr int kLate = dma_count<A_KMAJOR>(true) + dma_count<B_KMAJOR>(true);
  if (n > 2) wait_vmcnt<kLate>();  // tiles 0 and 1 landed; tile 2 may still be in flight
  else wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  tile_k_loop<A_KMAJOR, B_KMAJOR>(acc, g, a, b, m0, n0, kt_beg, n, dla, dlb, R, wave_s, wm, wn, lane);
  EpiCtx ctx{m0, n0, tm, tn, split, wm, wn, lane, lds0, lds1, lds2, lds3, lds0};
  epi(acc, ctx);
}

// Persistent form for epilogues that leave the four LDS arrays alone
// (Epi::kKeepsStages): workgroup p of P walks the blocks p, p + P, p + 2P, ...
// (P a multiple of 8, so every tile stays on the XCD map_tile gives it).
// After the last k step of a tile, whose closing barrier ends every read of
// the slots and stages, the first k tiles of the next tile (0, 1 and 2, with 3
// for a K-major operand's second pair) are loaded, and only then does the
// epilogue run: the loads land while it computes.  The next k loop starts by
// waiting for every outstanding load (count-based, in program order: the
// epilogue's own loads and stores issued after them only make it wait longer)
// and a barrier.  The k steps are those of gemm_tile, in the same order of
// reads, loads, waits and barriers, so the accumulators, and the results, are
// the same bits.
template <bool A_KMAJOR, bool B_KMAJOR, class Epi>
__device__ __forceinline__ void gemm_tiles_persistent(const GemmGeom& g, const Operand& a, const Operand& b,
                                                      const Epi& epi, int p, int P, int vg, char* lds0, char* lds1,
                                                      char* lds2, char* lds3, char* xch) {
  static_assert(Epi::kKeepsStages, "the persistent form needs an epilogue that leaves the LDS stages alone");
  args_to_sgprs(g);
  args_to_sgprs(a);
  args_to_sgprs(b);
  args_to_sgprs(epi);
  const LdsRing<A_KMAJOR, B_KMAJOR> R = lds_ring<A_KMAJOR, B_KMAJOR>(lds0, lds1, lds2, lds3);
  const int nk = (g.K + kBK - 1) / kBK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave / kWavesN, wn = wave % kWavesN;

  struct TileState {
    int tm, tn, split, m0, n0, kt_beg, n;
    DmaLanes dla, dlb;
  };
  auto setup = [&](int vb) {
    TileState t;
    map_tile(g, vb, vg, t.tm, t.tn, t.split);
    t.m0 = t.tm * kBM;
    t.n0 = t.tn * kBN;
    t.kt_beg = (int)(((int64_t)t.split * nk) / g.splits);
    t.n = (int)(((int64_t)(t.split + 1) * nk) / g.splits) - t.kt_beg;
    t.dla = dma_lanes<A_KMAJOR>(a, t.m0, g.M, g.K, wave_s, lane);
    t.dlb = dma_lanes<B_KMAJOR>(b, t.n0, g.N, g.K, wave_s, lane);
    return t;
  };
  auto first_loads = [&](const TileState& t) {
    tile_first_loads<A_KMAJOR, B_KMAJOR>(g, a, b, t.m0, t.n0, t.kt_beg, t.n, t.dla, t.dlb, R, wave_s);
  };

  AccTile acc;
  // Tile state is rebuilt from the block index where it is needed (a few
  // instructions) rather than kept live across the epilogue, which needs
  // every register it can get.
  int vb = p;
  if (vb >= vg) return;
  first_loads(setup(vb));
  while (true) {
    {
      const TileState cur = setup(vb);
      wait_vmcnt<0>();  // the first loads (and anything issued after them)
      __builtin_amdgcn_s_barrier();
      tile_k_loop<A_KMAJOR, B_KMAJOR>(acc, g, a, b, cur.m0, cur.n0, cur.kt_beg, cur.n, cur.dla, cur.dlb, R, wave_s,
                                      wm, wn, lane);
    }
    const int nvb = vb + P;
    const bool more = nvb < vg;
    if (more) first_loads(setup(nvb));
    int tm, tn, split;
    map_tile(g, vb, vg, tm, tn, split);
    const EpiCtx ctx{tm * kBM, tn * kBN, tm, tn, split, wm, wn, lane, lds0, lds1, lds2, lds3, xch};
    epi(acc, ctx);
    if (!more) break;
    vb = nvb;
  }
}

#define MS_DECLARE_LDS_STAGES                                 \
  __shared__ __attribute__((aligned(1024))) char lds0[kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) char lds1[kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) char lds2[kStageBytes]; \
  __shared__ __attribute__((aligned(1024))) char lds3[kStageBytes]

// Persistent launch of gemm_tiles_persistent: gridDim.x workgroups (a multiple
// of 8, at most one per CU) share the vg tiles.
template <bool A_KMAJOR, bool B_KMAJOR, class Epi>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd)))
gemm_persistent_kernel(GemmGeom g, Operand a, Operand b, Epi epi, int vg) {
  MS_DECLARE_LDS_STAGES;
  __shared__ __attribute__((aligned(16))) char xch[Epi::kXchBytes];
  gemm_tiles_persistent<A_KMAJOR, B_KMAJOR, Epi>(g, a, b, epi, (int)blockIdx.x, (int)gridDim.x, vg, lds0, lds1, lds2,
                                                 lds3, xch);
}

template <bool A_KMAJOR, bool B_KMAJOR, class Epi>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd)))
gemm_kernel(GemmGeom g, Operand a, Operand b, Epi epi) {
  MS_DECLARE_LDS_STAGES;
  gemm_tile<A_KMAJOR, B_KMAJOR, Epi>(g, a, b, epi, (int)blockIdx.x, (int)gridDim.x, lds0, lds1, lds2, lds3);
}

// Two independent GEMMs in one launch, so that the blocks of one fill the CUs
// the other leaves idle.  The hardware hands blocks to free CUs in index
// order, and the host puts the GEMM with the longer blocks first: when
// `second_first` is set, GEMM 2 takes the leading block range.  The leading
// GEMM's range is its block count rounded up to a multiple of 8 (the extra
// blocks exit at once), which keeps the trailing GEMM's first block on XCD 0.
template <bool AK1, bool BK1, class E1, bool AK2, bool BK2, class E2>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(kWavesPerSimd, kWavesPerSimd)))
gemm_pair_kernel(GemmGeom g1, Operand a1, Operand b1, E1 e1, int blocks1, GemmGeom g2, Operand a2, Operand b2,
                 E2 e2, int blocks2, int second_first) {
  MS_DECLARE_LDS_STAGES;
  const int bid = (int)blockIdx.x;
  const int lead = second_first ? blocks2 : blocks1;
  const int lead_pad = (lead + 7) & ~7;
  const bool in_lead = bid < lead_pad;
  if (in_lead && bid >= lead) return;
  const int vb = in_lead ? bid : bid - lead_pad;
  if (in_lead != (second_first != 0)) {
    gemm_tile<AK1, BK1, E1>(g1, a1, b1, e1, vb, blocks1, lds0, lds1, lds2, lds3);
  } else {
    gemm_tile<AK2, BK2, E2>(g2, a2, b2, e2, vb, blocks2, lds0, lds1, lds2, lds3);
  }
}

}  // namespace mshard
