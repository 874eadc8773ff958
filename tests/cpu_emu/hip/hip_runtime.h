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
#include <functional>
#include <thread>
#include <vector>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
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

#define __builtin_amdgcn_exp2f(x) exp2f(x)
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, C, X, Y, Z) emu::mfma16x16x32(A, B, C)
#define __builtin_amdgcn_ds_read_tr16_b64_v4i16(P) emu::ds_read_tr16((const char*)(P))
