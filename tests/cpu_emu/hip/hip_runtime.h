// Host emulation of the HIP subset that the attention and fingerprint kernels
// use, for running their unmodified sources on the CPU in tests: a workgroup
// runs as one OS thread per lane, workgroups run one after another, barriers
// are std::barrier, and cross-lane operations exchange values through per-wave
// slots (see epilogues.hpp here for their lane semantics).
#pragma once
#include <barrier>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <deque>
#include <functional>
#include <thread>
#include <vector>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define amdgpu_flat_work_group_size(...) unused
#define amdgpu_waves_per_eu(...) unused
#define __shared__ static

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
typedef void* hipStream_t;
inline hipError_t hipGetLastError() { return hipSuccess; }

struct dim3 {
  unsigned x, y, z;
  dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
struct emu_idx { unsigned x, y, z; };
inline thread_local emu_idx threadIdx, blockIdx;
inline dim3 gridDim, blockDim;

inline int min(int a, int b) { return a < b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }
inline float __int_as_float(int x) { float f; std::memcpy(&f, &x, 4); return f; }
inline float __uint_as_float(unsigned x) { float f; std::memcpy(&f, &x, 4); return f; }

namespace emu {
struct Block {
  explicit Block(int threads) : all(threads) {}
  std::barrier<> all;
  std::barrier<> wave[4] = {std::barrier<>{64}, std::barrier<>{64}, std::barrier<>{64}, std::barrier<>{64}};
  alignas(64) unsigned char slot[4][64][64];  // per wave, per lane: up to 64 bytes of exchange data
};
inline Block* g_block = nullptr;

template <class T>
inline void deposit(const T& v) {
  static_assert(sizeof(T) <= 64, "slot size");
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  std::memcpy(g_block->slot[w][l], &v, sizeof(T));
}
template <class T>
inline T fetch(int lane) {
  T v;
  std::memcpy(&v, g_block->slot[threadIdx.x / 64][lane], sizeof(T));
  return v;
}
inline void wave_sync() { g_block->wave[threadIdx.x / 64].arrive_and_wait(); }

template <class F, class... A>
inline void launch(dim3 grid, dim3 block, F kernel, A... args) {
  gridDim = grid;
  blockDim = block;
  for (unsigned bz = 0; bz < grid.z; ++bz)
    for (unsigned by = 0; by < grid.y; ++by)
      for (unsigned bx = 0; bx < grid.x; ++bx) {
        Block blk((int)block.x);
        g_block = &blk;
        std::vector<std::thread> th;
        th.reserve(block.x);
        for (unsigned t = 0; t < block.x; ++t)
          th.emplace_back([=] {
            threadIdx = emu_idx{t, 0, 0};
            blockIdx = emu_idx{bx, by, bz};
            kernel(args...);
          });
        for (auto& x : th) x.join();
        g_block = nullptr;
      }
}
}  // namespace emu

#define hipLaunchKernelGGL(K, GRID, BLOCK, SHMEM, STREAM, ...) emu::launch(GRID, BLOCK, K, __VA_ARGS__)
inline void __syncthreads() { emu::g_block->all.arrive_and_wait(); }

// ---- builtins of the GEMM core and the epilogues
namespace emu {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
struct Rsrc {
  char* base;
  int64_t bytes;
};
inline Rsrc make_rsrc(const void* base, int n) { return Rsrc{(char*)base, n}; }
template <class V>
inline V rload(Rsrc r, int off) {
  V v{};
  if (off >= 0 && (int64_t)off + (int64_t)sizeof(V) <= r.bytes) std::memcpy(&v, r.base + off, sizeof(V));
  return v;
}
template <class V>
inline void rstore(V v, Rsrc r, int off) {
  if (off >= 0 && (int64_t)off + (int64_t)sizeof(V) <= r.bytes) std::memcpy(r.base + off, &v, sizeof(V));
}
// Both lanes of each pair (l, l^m) receive (lower lane's value, upper lane's value).
struct Pair {
  uint32_t v[2];
  uint32_t operator[](int i) const { return v[i]; }
};
inline Pair permlane_swap(uint32_t x, int m) {
  deposit(x);
  wave_sync();
  const int l = threadIdx.x % 64, o = l ^ m;
  Pair r{{fetch<uint32_t>(l < o ? l : o), fetch<uint32_t>(l < o ? o : l)}};
  wave_sync();
  return r;
}
inline float shfl_xor(float x, int m) {
  deposit(x);
  wave_sync();
  const float v = fetch<float>((threadIdx.x % 64) ^ m);
  wave_sync();
  return v;
}
inline bool any(bool x) {
  deposit((int)x);
  wave_sync();
  int r = 0;
  for (int l = 0; l < 64; ++l) r |= fetch<int>(l);
  wave_sync();
  return r != 0;
}
// buffer_load_dwordx4 ... lds: lane l's 16 bytes from the buffer the descriptor
// {base low, base high (16 bits), bytes, flags} describes, at byte offset off,
// go to LDS byte 16*l of the 1 KiB at lds_addr; past the buffer they are zero.
// The LDS write is held back until an s_waitcnt whose vector-memory count
// leaves fewer of this lane's loads outstanding, the latest the hardware may
// land it (other vector-memory operations would only make a wait stricter), so
// a missing or too-loose wait leaves stale LDS bytes for the readers to see.
struct PendingDma {
  char* dst;
  unsigned char data[16];
};
inline thread_local std::deque<PendingDma> t_dma;  // this lane's loads not yet landed, oldest first
inline void dma16(u32x4 desc, uint32_t off, uint32_t lds_addr) {
  const char* base = (const char*)(uintptr_t)((uint64_t)desc[0] | ((uint64_t)(desc[1] & 0xffffu) << 32));
  PendingDma p;
  p.dst = (char*)(uintptr_t)lds_addr + 16 * (threadIdx.x % 64);
  if ((uint64_t)off + 16 <= (uint64_t)desc[2]) std::memcpy(p.data, base + off, 16);
  else std::memset(p.data, 0, 16);
  t_dma.push_back(p);
}
inline void wait_vmcnt(unsigned n) {
  while (t_dma.size() > n) {
    std::memcpy(t_dma.front().dst, t_dma.front().data, 16);
    t_dma.pop_front();
  }
}

inline float bf16f(unsigned short u) {
  uint32_t x = (uint32_t)u << 16;
  float v;
  std::memcpy(&v, &x, 4);
  return v;
}
// fp32 -> bf16 bits, round to nearest even, NaN kept quiet.
inline uint32_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
inline uint32_t pack_bf16x2_rne(float lo, float hi) { return bf16_rne(lo) | (bf16_rne(hi) << 16); }

// v_mfma_f32_16x16x32_bf16 on any 16-byte operand type holding bf16 bit
// patterns: lane l supplies row l%16, k = 8(l/16) .. +7 of the first operand and
// column l%16 of the second; it receives D[4(l/16) + r][l%16].
template <class V, class A>
inline A mfma16x16x32(const V& a, const V& b, const A& c) {
  typedef unsigned short us8 __attribute__((ext_vector_type(8)));
  struct Ops { us8 a, b; };
  deposit(Ops{__builtin_bit_cast(us8, a), __builtin_bit_cast(us8, b)});
  wave_sync();
  const int l = threadIdx.x % 64, g = l / 16, col = l % 16;
  float av[4][32], bv[32];
  for (int q = 0; q < 4; ++q) {
    const us8 bq = fetch<Ops>(col + 16 * q).b;
    for (int e = 0; e < 8; ++e) bv[8 * q + e] = bf16f(bq[e]);
    for (int r = 0; r < 4; ++r) {
      const us8 aq = fetch<Ops>(4 * g + r + 16 * q).a;
      for (int e = 0; e < 8; ++e) av[r][8 * q + e] = bf16f(aq[e]);
    }
  }
  wave_sync();
  A out = c;
  for (int r = 0; r < 4; ++r) {
    float acc = 0.f;
    for (int k = 0; k < 32; ++k) acc += av[r][k] * bv[k];
    out[r] += acc;
  }
  return out;
}

// ds_read_b64_tr_b16: within each group of 16 lanes, result lane i, element e is
// element i%4 of the 8 bytes source lane i/4 + 4e addressed.
typedef short s16x4 __attribute__((ext_vector_type(4)));
inline s16x4 ds_read_tr16(const char* p) {
  deposit(p);
  wave_sync();
  const int l = threadIdx.x % 64, G = l / 16, i = l % 16;
  s16x4 out;
  for (int e = 0; e < 4; ++e) {
    const char* src = fetch<const char*>(16 * G + i / 4 + 4 * e);
    short v;
    std::memcpy(&v, src + 2 * (i % 4), 2);
    out[e] = v;
  }
  wave_sync();
  return out;
}
}  // namespace emu

typedef emu::Rsrc __amdgpu_buffer_rsrc_t;
#define __builtin_amdgcn_make_buffer_rsrc(P, S, N, F) emu::make_rsrc(P, N)
#define __builtin_amdgcn_raw_buffer_load_b128(R, O, S, A) emu::rload<emu::u32x4>(R, O)
#define __builtin_amdgcn_raw_buffer_load_b64(R, O, S, A) emu::rload<emu::u32x2>(R, O)
#define __builtin_amdgcn_raw_buffer_store_b128(V, R, O, S, A) emu::rstore<emu::u32x4>(V, R, O)
#define __builtin_amdgcn_raw_buffer_store_b64(V, R, O, S, A) emu::rstore<emu::u32x2>(V, R, O)
#define __builtin_amdgcn_raw_buffer_store_b32(V, R, O, S, A) emu::rstore<uint32_t>(V, R, O)
#define __builtin_amdgcn_s_waitcnt(x) emu::wait_vmcnt(((x) & 15) | ((((x) >> 14) & 3) << 4))
#define __builtin_amdgcn_sched_barrier(x) ((void)0)
#define __builtin_amdgcn_s_barrier() __syncthreads()
#define __builtin_amdgcn_readfirstlane(x) (x)
#define __builtin_amdgcn_wave_barrier() emu::wave_sync()
#define __builtin_amdgcn_rcpf(x) (1.0f / (x))
#define __builtin_amdgcn_permlane16_swap(A, B, C, D) emu::permlane_swap(A, 16)
#define __builtin_amdgcn_permlane32_swap(A, B, C, D) emu::permlane_swap(A, 32)
inline uint32_t __float_as_uint(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
inline float __shfl_xor(float x, int m, int) { return emu::shfl_xor(x, m); }
inline bool __any(bool x) { return emu::any(x); }

#define __builtin_amdgcn_exp2f(x) exp2f(x)
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, C, X, Y, Z) emu::mfma16x16x32(A, B, C)
#define __builtin_amdgcn_ds_read_tr16_b64_v4i16(P) emu::ds_read_tr16((const char*)(P))
