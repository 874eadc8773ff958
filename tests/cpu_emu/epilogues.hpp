// Stand-in for the library's epilogues.hpp / gemm_core.hpp when a kernel source
// is compiled for the host: the vector types (as bit containers), the bf16
// helpers with round-to-nearest-even, and the cross-lane operations emulated
// through the per-wave exchange of hip/hip_runtime.h.
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

namespace emu {
inline float bf16f(unsigned short u) { return __uint_as_float((uint32_t)u << 16); }

// v_mfma_f32_16x16x32_bf16: lane l supplies row l%16, k = 8(l/16) .. +7 of the
// first operand and column l%16 of the second; it receives D[4(l/16) + r][l%16].
inline mshard::f32x4_t mfma16x16x32(const mshard::bf16x8_t& a, const mshard::bf16x8_t& b, const mshard::f32x4_t& c) {
  struct Ops { mshard::bf16x8_t a, b; };
  deposit(Ops{a, b});
  wave_sync();
  Ops all[64];
  for (int l = 0; l < 64; ++l) all[l] = fetch<Ops>(l);
  wave_sync();
  const int l = threadIdx.x % 64, g = l / 16, col = l % 16;
  mshard::f32x4_t out = c;
  for (int r = 0; r < 4; ++r) {
    const int i = 4 * g + r;
    float acc = 0.f;
    for (int k = 0; k < 32; ++k) acc += bf16f(all[i + 16 * (k / 8)].a[k % 8]) * bf16f(all[col + 16 * (k / 8)].b[k % 8]);
    out[r] += acc;
  }
  return out;
}

// ds_read_b64_tr_b16: within each group of 16 lanes, result lane i, element e is
// element i%4 of the 8 bytes source lane i/4 + 4e addressed.
inline mshard::s16x4_t ds_read_tr16(const char* p) {
  deposit(p);
  wave_sync();
  const int l = threadIdx.x % 64, G = l / 16, i = l % 16;
  mshard::s16x4_t out;
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
