// Stand-in for the library's epilogues.hpp / gemm_core.hpp when the attention
// kernels are compiled for the host on their own: the vector types (as bit
// containers), the bf16 helpers with round-to-nearest-even, and the lane-pair
// exchanges through the per-wave slots of hip/hip_runtime.h (which also holds
// the emulated MFMA and transposing LDS read).
#pragma once
#include <hip/hip_runtime.h>

namespace mshard {

typedef unsigned short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef char lds_char;

constexpr float kLog2e = 1.44269504088896340736f;

inline uint32_t f32_to_bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
inline uint32_t pack_bf16x2(float lo, float hi) { return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16); }
inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Both lanes of each pair (l, l^16) / (l, l^32) receive (lower lane's value, upper lane's value).
inline void xswap_n(float x, float& lo, float& hi, int m) {
  emu::deposit(x);
  emu::wave_sync();
  const int l = threadIdx.x % 64, o = l ^ m;
  const float a = emu::fetch<float>(l < o ? l : o), b = emu::fetch<float>(l < o ? o : l);
  emu::wave_sync();
  lo = a;
  hi = b;
}
inline void xswap16(float x, float& lo, float& hi) { xswap_n(x, lo, hi, 16); }
inline void xswap32(float x, float& lo, float& hi) { xswap_n(x, lo, hi, 32); }

}  // namespace mshard
