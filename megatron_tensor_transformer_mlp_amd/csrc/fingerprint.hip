// fingerprint.hip - chunk-wise fingerprints of device buffers, for tracking
// down non-determinism (Megatron Core bitwise-determinism news item,
// news.hamidun.com, "debugging methodology": tensors are fingerprinted on the
// GPU, chunk-wise where the order of the data matters, and two runs are
// compared call by call to find the first one that differs).
//
// The hash is XXH64 with seed 0, from its published specification (xxHash,
// "XXH64 algorithm description").  A buffer of n bytes in chunks of c bytes
// has ceil(n / c) chunks (one empty chunk when n = 0); out[1 + k] is XXH64 of
// chunk k and out[0] is XXH64 of out[1 ..] as little-endian 64-bit words.
// One thread hashes one chunk from start to end; a second launch hashes the
// chunk hashes.  This is a debugging aid, not a hot-path kernel.
#include "launch.hpp"

namespace mshard {

namespace {

constexpr uint64_t kP1 = 0x9E3779B185EBCA87ull;
constexpr uint64_t kP2 = 0xC2B2AE3D27D4EB4Full;
constexpr uint64_t kP3 = 0x165667B19E3779F9ull;
constexpr uint64_t kP4 = 0x85EBCA77C2B2AE63ull;
constexpr uint64_t kP5 = 0x27D4EB2F165667C5ull;

__device__ __forceinline__ uint64_t rotl64(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }

__device__ __forceinline__ uint64_t xxh_round(uint64_t acc, uint64_t lane) {
  acc += lane * kP2;
  return rotl64(acc, 31) * kP1;
}

__device__ __forceinline__ uint64_t xxh_merge(uint64_t h, uint64_t acc) {
  h ^= xxh_round(0, acc);
  return h * kP1 + kP4;
}

// XXH64 (seed 0) of the n bytes at p; p is 8-byte aligned.
__device__ uint64_t xxh64_aligned(const uint8_t* __restrict__ p, uint64_t n) {
  const uint64_t* w = (const uint64_t*)p;
  uint64_t i = 0;
  uint64_t h;
  if (n >= 32) {
    uint64_t v1 = kP1 + kP2, v2 = kP2, v3 = 0, v4 = 0 - kP1;
    for (; i + 32 <= n; i += 32) {
      v1 = xxh_round(v1, w[i / 8]);
      v2 = xxh_round(v2, w[i / 8 + 1]);
      v3 = xxh_round(v3, w[i / 8 + 2]);
      v4 = xxh_round(v4, w[i / 8 + 3]);
    }
    h = rotl64(v1, 1) + rotl64(v2, 7) + rotl64(v3, 12) + rotl64(v4, 18);
    h = xxh_merge(h, v1);
    h = xxh_merge(h, v2);
    h = xxh_merge(h, v3);
    h = xxh_merge(h, v4);
  } else {
    h = kP5;
  }
  h += n;
  for (; i + 8 <= n; i += 8) {
    h ^= xxh_round(0, w[i / 8]);
    h = rotl64(h, 27) * kP1 + kP4;
  }
  if (i + 4 <= n) {
    h ^= (uint64_t)(*(const uint32_t*)(p + i)) * kP1;
    h = rotl64(h, 23) * kP2 + kP3;
    i += 4;
  }
  for (; i < n; ++i) {
    h ^= (uint64_t)p[i] * kP5;
    h = rotl64(h, 11) * kP1;
  }
  h ^= h >> 33;
  h *= kP2;
  h ^= h >> 29;
  h *= kP3;
  h ^= h >> 32;
  return h;
}

// out[1 + k] = XXH64 of chunk k (bytes [k*chunk, min(bytes, (k+1)*chunk))), k < n.
__global__ void __launch_bounds__(256) fingerprint_chunks(const uint8_t* __restrict__ buf, uint64_t bytes,
                                                          uint64_t chunk, uint64_t n, uint64_t* __restrict__ out) {
  const uint64_t k = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= n) return;
  const uint64_t b0 = k * chunk;
  const uint64_t len = bytes > b0 ? (bytes - b0 < chunk ? bytes - b0 : chunk) : 0;
  out[1 + k] = xxh64_aligned(buf + b0, len);
}

// out[0] = XXH64 of the n chunk hashes out[1 .. n] (one thread).
__global__ void __launch_bounds__(64) fingerprint_combine(uint64_t* __restrict__ out, uint64_t n) {
  if (threadIdx.x == 0) out[0] = xxh64_aligned((const uint8_t*)(out + 1), n * 8);
}

}  // namespace

uint64_t fingerprint_chunk_count(uint64_t bytes, uint64_t chunk) {
  return bytes == 0 ? 1 : (bytes + chunk - 1) / chunk;
}

hipError_t launch_fingerprint(const void* buf, uint64_t bytes, uint64_t chunk, uint64_t* out, hipStream_t st) {
  const uint64_t n = fingerprint_chunk_count(bytes, chunk);
  hipLaunchKernelGGL(fingerprint_chunks, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const uint8_t*)buf,
                     bytes, chunk, n, out);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(fingerprint_combine, dim3(1), dim3(64), 0, st, out, n);
  return hipGetLastError();
}

}  // namespace mshard
