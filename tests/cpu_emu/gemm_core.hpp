// Stand-in for the GEMM core when epilogues.hpp is compiled for the host: the
// types, tile constants and accumulator layout of the core, buffer resources
// with the hardware's out-of-range behaviour (loads past the resource read
// zero, stores past it are dropped), the accumulator staging store, and the
// cross-lane exchanges through hip/hip_runtime.h's per-wave slots.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>

namespace mshard {

typedef unsigned short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef char lds_char;

constexpr int kBM = 256, kBN = 256, kBK = 32;
constexpr int kWavesM = 2, kWavesN = 2;
constexpr int kWaves = kWavesM * kWavesN;
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveM = kBM / kWavesM, kWaveN = kBN / kWavesN;
constexpr int kSubM = kWaveM / 16, kSubN = kWaveN / 16;
constexpr int kStageBytes = (kBM + kBN) * kBK * 2;
constexpr uint32_t kOOB = 0x80000000u;

struct rsrc_t {
  char* base;
  int64_t bytes;
};
inline rsrc_t make_rsrc(const void* base, int64_t bytes_left) {
  return rsrc_t{(char*)base, bytes_left < 0 ? 0 : (bytes_left > 0x7fffffff ? 0x7fffffff : bytes_left)};
}
template <class V>
inline V buf_load(rsrc_t r, uint32_t off) {
  V v{};
  if ((int64_t)off + (int64_t)sizeof(V) <= r.bytes) std::memcpy(&v, r.base + off, sizeof(V));
  return v;
}
template <class V>
inline void buf_store(V v, rsrc_t r, uint32_t off) {
  if ((int64_t)off + (int64_t)sizeof(V) <= r.bytes) std::memcpy(r.base + off, &v, sizeof(V));
}
inline u32x4_t buf_load16(rsrc_t r, uint32_t off) { return buf_load<u32x4_t>(r, off); }
template <int POLICY = 0>
inline u32x2_t buf_load8(rsrc_t r, uint32_t off) { return buf_load<u32x2_t>(r, off); }
// the cache-policy argument of the real helpers changes nothing on the host
constexpr int kNonTemporal = 2;
template <int POLICY = 0>
inline void buf_store16(u32x4_t v, rsrc_t r, uint32_t off) { buf_store(v, r, off); }
template <int POLICY = 0>
inline void buf_store8(u32x2_t v, rsrc_t r, uint32_t off) { buf_store(v, r, off); }

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

// acc[mi][ni][r] of wave (wm, wn) holds C[wm*kWaveM + mi*16 + (lane & 15)][wn*kWaveN + ni*16 + 4*(lane >> 4) + r]
typedef f32x4_t AccTile[kSubM][kSubN];
inline void acc_store_lds(char* p, const f32x4_t& a) { std::memcpy(p, &a, 16); }
inline void acc_settle() {}

struct EpiCtx {
  int m0, n0;
  int tm, tn;
  int split;
  int wm, wn;
  int lane;
  char* lds0;
  char* lds1;
  char* lds2;
  char* lds3;
  char* xch;
};

}  // namespace mshard
