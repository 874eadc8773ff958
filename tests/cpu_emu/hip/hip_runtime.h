// Host emulation of the HIP subset that the library's kernels use, for running
// their sources on the CPU in tests.  A workgroup's lanes run as cooperative
// fibers on one OS thread, workgroups one after another.  A lane runs until it
// reaches a barrier: the wave-wide one that every emulated cross-lane
// operation passes through (values are exchanged in per-wave slots), or the
// workgroup's.  A barrier opens once every lane it covers has arrived or has
// finished (as on the hardware, finished lanes no longer hold a barrier); no
// lane can pass one early, and a schedule in which no lane can move is
// reported and aborts.  Under ThreadSanitizer or AddressSanitizer the fibers
// are announced to the sanitizer, and a barrier is the only ordering between
// lanes that ThreadSanitizer sees.
#pragma once
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <functional>
#include <vector>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define amdgpu_flat_work_group_size(...) unused
#define amdgpu_waves_per_eu(...) unused
#define __shared__ static

#if defined(__has_feature)
#if __has_feature(thread_sanitizer)
#define EMU_TSAN 1
#endif
#if __has_feature(address_sanitizer)
#define EMU_ASAN 1
#endif
#endif
#ifdef EMU_TSAN
extern "C" void* __tsan_get_current_fiber(void);
extern "C" void* __tsan_create_fiber(unsigned flags);
extern "C" void __tsan_destroy_fiber(void* fiber);
extern "C" void __tsan_switch_to_fiber(void* fiber, unsigned flags);
extern "C" void __tsan_acquire(void* addr);
extern "C" void __tsan_release(void* addr);
extern "C" void AnnotateIgnoreReadsBegin(const char* file, int line);
extern "C" void AnnotateIgnoreReadsEnd(const char* file, int line);
extern "C" void AnnotateIgnoreWritesBegin(const char* file, int line);
extern "C" void AnnotateIgnoreWritesEnd(const char* file, int line);
#endif
#ifdef EMU_ASAN
extern "C" void __sanitizer_start_switch_fiber(void** fake_stack_save, const void* bottom, size_t size);
extern "C" void __sanitizer_finish_switch_fiber(void* fake_stack_save, const void** bottom_old, size_t* size_old);
#endif

typedef int hipError_t;
enum { hipSuccess = 0, hipErrorInvalidValue = 1 };
typedef void* hipStream_t;
inline hipError_t hipGetLastError() { return hipSuccess; }
inline hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
// Device attributes a launcher may size a grid by: the compute-unit count is
// EMU_CUS (default 8), small enough that a grid sized by it leaves each
// workgroup several tiles on the small shapes emulated here.
enum hipDeviceAttribute_t { hipDeviceAttributeMultiprocessorCount = 0 };
inline hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int) {
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  const char* e = std::getenv("EMU_CUS");
  *value = e ? std::atoi(e) : 8;
  return hipSuccess;
}

// Static device arrays: the host array stands for the device one, and a
// symbol's device address is the host array's own address.
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(s) (&(s))
inline hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) {
  *ptr = const_cast<void*>(symbol);
  return hipSuccess;
}

struct dim3 {
  unsigned x, y, z;
  dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {}
};
struct emu_idx { unsigned x, y, z; };
inline dim3 gridDim, blockDim;

inline int min(int a, int b) { return a < b ? a : b; }
inline int max(int a, int b) { return a > b ? a : b; }
inline float __int_as_float(int x) { float f; std::memcpy(&f, &x, 4); return f; }
inline float __uint_as_float(unsigned x) { float f; std::memcpy(&f, &x, 4); return f; }

// Saves the callee-saved registers on the current stack, stores its pointer at
// *save and continues on the stack at next (System V x86-64).
extern "C" void emu_swap_context(void** save, void* next);
asm(R"(
  .text
  .weak emu_swap_context
  .type emu_swap_context, @function
emu_swap_context:
  pushq %rbp
  pushq %rbx
  pushq %r12
  pushq %r13
  pushq %r14
  pushq %r15
  movq %rsp, (%rdi)
  movq %rsi, %rsp
  popq %r15
  popq %r14
  popq %r13
  popq %r12
  popq %rbx
  popq %rbp
  ret
  .size emu_swap_context, .-emu_swap_context
)");

namespace emu {
struct PendingDma {
  char* dst;
  unsigned char data[16];
};
struct Fiber {
  void* sp = nullptr;
  void* first_sp = nullptr;  // sp until the lane first runs
  char* stack = nullptr;
  emu_idx tid{0, 0, 0};
  int state = 0;  // 0 runnable, 1 waiting at a barrier, 2 finished
  int bar = -1;   // barrier waited at
  unsigned gen = 0;
  std::deque<PendingDma> dma;  // this lane's direct-to-LDS loads not yet landed, oldest first
  void* tsan = nullptr;
  void* asan_fake = nullptr;
};
struct Bar {
  int participants = 0, arrived = 0;
  unsigned gen = 0;
};
constexpr size_t kStack = 256 << 10;
struct Block {
  int n = 0, waves = 0;
  std::vector<Bar> bars;  // one per wave, then the workgroup's
  std::vector<unsigned char> slots;  // per wave, per lane: up to 64 bytes of exchange data
  std::vector<float> results;        // per wave: one 16 x 16 MFMA result block
  std::function<void()> body;
};
inline Block* g_block = nullptr;
inline Fiber* g_cur = nullptr;
inline std::vector<Fiber> g_fibers;
inline std::vector<char*> g_stacks;
inline void* g_sched_sp = nullptr;
inline void* g_sched_tsan = nullptr;
inline void* g_sched_fake = nullptr;
inline const void* g_sched_bottom = nullptr;
inline size_t g_sched_size = 0;
}  // namespace emu

namespace emu {
inline Fiber* cur() { return __atomic_load_n(&g_cur, __ATOMIC_RELAXED); }
inline char g_join;  // ThreadSanitizer: a finished workgroup's lanes release here, the scheduler acquires
// ThreadSanitizer: the scheduler's bookkeeping is not kernel data; no race is reported on it
inline void ignore_begin() {
#ifdef EMU_TSAN
  AnnotateIgnoreReadsBegin(__FILE__, __LINE__);
  AnnotateIgnoreWritesBegin(__FILE__, __LINE__);
#endif
}
inline void ignore_end() {
#ifdef EMU_TSAN
  AnnotateIgnoreWritesEnd(__FILE__, __LINE__);
  AnnotateIgnoreReadsEnd(__FILE__, __LINE__);
#endif
}
inline void tsan_release(void* p) {
#ifdef EMU_TSAN
  __tsan_release(p);
#endif
  (void)p;
}
inline void tsan_acquire(void* p) {
#ifdef EMU_TSAN
  __tsan_acquire(p);
#endif
  (void)p;
}
}  // namespace emu

// threadIdx and blockIdx of the running lane
#define threadIdx (emu::cur()->tid)
inline emu_idx blockIdx;

namespace emu {
// scheduler -> fiber f, and back when it blocks or finishes; the first entry
// into a lane orders the workgroup's set-up before it
inline void enter(Fiber& f, bool first) {
  __atomic_store_n(&g_cur, &f, __ATOMIC_RELAXED);
#ifdef EMU_TSAN
  __tsan_switch_to_fiber(f.tsan, first ? 0 : 1);
#endif
  (void)first;
#ifdef EMU_ASAN
  __sanitizer_start_switch_fiber(&g_sched_fake, f.stack, kStack);
#endif
  emu_swap_context(&g_sched_sp, f.sp);
#ifdef EMU_ASAN
  __sanitizer_finish_switch_fiber(g_sched_fake, nullptr, nullptr);
#endif
}
inline void leave(bool finished) {
  Fiber& f = *cur();
#ifdef EMU_TSAN
  __tsan_switch_to_fiber(__atomic_load_n(&g_sched_tsan, __ATOMIC_RELAXED), 1);
#endif
#ifdef EMU_ASAN
  __sanitizer_start_switch_fiber(finished ? nullptr : &f.asan_fake, g_sched_bottom, g_sched_size);
#endif
  emu_swap_context(&f.sp, g_sched_sp);
#ifdef EMU_ASAN
  __sanitizer_finish_switch_fiber(f.asan_fake, nullptr, nullptr);
#endif
}
inline void open_if_complete(Bar& b) {
  if (b.arrived > 0 && b.arrived == b.participants) {
    b.arrived = 0;
    ++b.gen;
  }
}
inline void arrive(int i) {
  Bar& b = g_block->bars[i];
  tsan_release(&b);
  ignore_begin();
  const bool last = ++b.arrived == b.participants;
  if (last) {
    open_if_complete(b);
  } else {
    Fiber& f = *cur();
    f.state = 1;
    f.bar = i;
    f.gen = b.gen;
  }
  ignore_end();
  if (!last) leave(false);
  tsan_acquire(&b);
}
[[noreturn]] inline void fiber_main() {
#ifdef EMU_ASAN
  __sanitizer_finish_switch_fiber(nullptr, &g_sched_bottom, &g_sched_size);
#endif
  g_block->body();
  Fiber& f = *cur();
  for (int i : {(int)(f.tid.x / 64), g_block->waves}) tsan_release(&g_block->bars[i]);
  tsan_release(&g_join);
  ignore_begin();
  f.state = 2;
  f.dma.clear();  // loads never waited for: nothing reads them
  for (int i : {(int)(f.tid.x / 64), g_block->waves}) {
    Bar& b = g_block->bars[i];
    --b.participants;
    open_if_complete(b);
  }
  ignore_end();
  leave(true);
  std::abort();
}

template <class T>
inline void deposit(const T& v) {
  static_assert(sizeof(T) <= 64, "slot size");
  std::memcpy(&g_block->slots[(size_t)threadIdx.x * 64], &v, sizeof(T));
}
template <class T>
inline T fetch(int lane) {
  T v;
  std::memcpy(&v, &g_block->slots[(size_t)((threadIdx.x / 64) * 64 + lane) * 64], sizeof(T));
  return v;
}
inline void wave_sync() { arrive((int)(threadIdx.x / 64)); }
inline float* wave_result() { return &g_block->results[(size_t)(threadIdx.x / 64) * 256]; }

template <class F, class... A>
inline void launch(dim3 grid, dim3 block, F kernel, A... args) {
  gridDim = grid;
  blockDim = block;
  const int n = (int)block.x;
  while ((int)g_stacks.size() < n) g_stacks.push_back((char*)std::aligned_alloc(64, kStack));
#ifdef EMU_TSAN
  __atomic_store_n(&g_sched_tsan, __tsan_get_current_fiber(), __ATOMIC_RELAXED);
#endif
  ignore_begin();
  g_fibers.resize(n);
  // EMU_SAMPLE=k: a GEMM launch (a kernel taking a GemmGeom) or a launch over a
  // 2-D or 3-D grid (the attention cores) of more than 16k workgroups runs only
  // k at each end of its linear workgroup order and k spread evenly between:
  // full-size shapes checked on a sample, the outputs of the others left as
  // they were.  Every other launch (the small per-token and reduction
  // kernels) runs in full.
  const uint64_t G = (uint64_t)grid.x * grid.y * grid.z;
  const char* env = std::getenv("EMU_SAMPLE");
  const bool may_sample = grid.y * grid.z > 1 || std::strstr(__PRETTY_FUNCTION__, "GemmGeom");
  const uint64_t k = env && may_sample ? std::strtoull(env, nullptr, 10) : 0;
  auto sampled = [&](uint64_t lin) {
    if (k == 0 || G <= 16 * k) return true;
    if (lin < k || lin >= G - k) return true;
    for (uint64_t i = 1; i <= k; ++i)
      if (lin == i * G / (k + 1)) return true;
    return false;
  };
  for (unsigned bz = 0; bz < grid.z; ++bz)
    for (unsigned by = 0; by < grid.y; ++by)
      for (unsigned bx = 0; bx < grid.x; ++bx) {
        if (!sampled(bx + (uint64_t)grid.x * (by + (uint64_t)grid.y * bz))) continue;
        Block blk;
        blk.n = n;
        blk.waves = (n + 63) / 64;
        blk.bars.resize(blk.waves + 1);
        for (int w = 0; w < blk.waves; ++w) blk.bars[w].participants = min(64, n - 64 * w);
        blk.bars[blk.waves].participants = n;
        blk.slots.assign((size_t)blk.waves * 64 * 64, 0);
        blk.results.assign((size_t)blk.waves * 256, 0.f);
        blk.body = [&] { kernel(args...); };
        g_block = &blk;
        blockIdx = emu_idx{bx, by, bz};
        for (int t = 0; t < n; ++t) {
          Fiber& f = g_fibers[t];
          f = Fiber{};
          f.stack = g_stacks[t];
          f.tid = emu_idx{(unsigned)t, 0, 0};
          // initial frame: six zero registers, then fiber_main as the return address,
          // then a zero return slot so that fiber_main starts with the ABI's alignment
          uintptr_t top = ((uintptr_t)f.stack + kStack) & ~(uintptr_t)15;
          void** sp = (void**)top;
          *--sp = nullptr;
          *--sp = (void*)&fiber_main;
          for (int r = 0; r < 6; ++r) *--sp = nullptr;
          f.sp = f.first_sp = sp;
#ifdef EMU_TSAN
          f.tsan = __tsan_create_fiber(0);
#endif
        }
        int done = 0;
        while (done < n) {
          bool moved = false;
          done = 0;
          for (int t = 0; t < n; ++t) {
            Fiber& f = g_fibers[t];
            if (f.state == 1 && blk.bars[f.bar].gen != f.gen) f.state = 0;
            if (f.state == 0) {
              enter(f, f.sp == f.first_sp);
              moved = true;
            }
            done += f.state == 2;
          }
          if (!moved && done < n) {
            std::fprintf(stderr, "emulation: no lane can move (block %u,%u,%u)\n", bx, by, bz);
            std::abort();
          }
        }
        tsan_acquire(&g_join);
#ifdef EMU_TSAN
        for (int t = 0; t < n; ++t) __tsan_destroy_fiber(g_fibers[t].tsan);
#endif
        g_block = nullptr;
        __atomic_store_n(&g_cur, (Fiber*)nullptr, __ATOMIC_RELAXED);
      }
  ignore_end();
}
}  // namespace emu

#define hipLaunchKernelGGL(K, GRID, BLOCK, SHMEM, STREAM, ...) emu::launch(GRID, BLOCK, K, __VA_ARGS__)
inline void __syncthreads() { emu::arrive(emu::g_block->waves); }

// ---- builtins of the GEMM core and the epilogues
namespace emu {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
struct Rsrc {
  char* base;
  int64_t bytes;
};
inline Rsrc make_rsrc(const void* base, int n) { return Rsrc{(char*)base, n}; }
// The hardware range-checks a multi-dword buffer access dword by dword; an
// access that straddles the end of its resource would need that, and the
// kernels never make one, so it is reported instead of emulated.
inline bool in_range(int64_t off, int64_t size, int64_t bytes) {
  if (off < 0 || off >= bytes) return false;
  if (off + size > bytes) {
    std::fprintf(stderr, "emulation: buffer access straddles the end of its resource\n");
    std::abort();
  }
  return true;
}
template <class V>
inline V rload(Rsrc r, int off) {
  V v{};
  if (in_range(off, sizeof(V), r.bytes)) std::memcpy(&v, r.base + off, sizeof(V));
  return v;
}
template <class V>
inline void rstore(V v, Rsrc r, int off) {
  if (in_range(off, sizeof(V), r.bytes)) std::memcpy(r.base + off, &v, sizeof(V));
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
inline void dma16(u32x4 desc, uint32_t off, uint32_t lds_addr) {
  const char* base = (const char*)(uintptr_t)((uint64_t)desc[0] | ((uint64_t)(desc[1] & 0xffffu) << 32));
  PendingDma p;
  p.dst = (char*)(uintptr_t)lds_addr + 16 * (threadIdx.x % 64);
  if (in_range(off, 16, desc[2])) std::memcpy(p.data, base + off, 16);
  else std::memset(p.data, 0, 16);
  cur()->dma.push_back(p);
}
inline void wait_vmcnt(unsigned n) {
  auto& q = cur()->dma;
  while (q.size() > n) {
    std::memcpy(q.front().dst, q.front().data, 16);
    q.pop_front();
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
// column l%16 of the second; it receives C[r] + D[4(l/16) + r][l%16], with D's
// sum over k formed in k order.  The wave's lane 0 forms its 16 x 16 block D once.
// (ThreadSanitizer leaves this function's accesses, which are the emulation's
// own exchange data, unchecked: the operands come from registers.)
template <class V, class A>
__attribute__((no_sanitize("thread"))) inline A mfma16x16x32(const V& a, const V& b, const A& c) {
  typedef unsigned short us8 __attribute__((ext_vector_type(8)));
  struct Ops { us8 a, b; };
  deposit(Ops{__builtin_bit_cast(us8, a), __builtin_bit_cast(us8, b)});
  wave_sync();
  const int l = threadIdx.x % 64;
  if (l == 0) {
    // bf16 products are exact in fp32, so only the order of the additions matters:
    // each of the 16 columns j (one vector lane each) adds its 32 products in k order
    typedef float f32x16 __attribute__((ext_vector_type(16)));
    float av[16][32];
    f32x16 bk[32];
    for (int src = 0; src < 64; ++src) {
      const Ops o = fetch<Ops>(src);
      for (int e = 0; e < 8; ++e) {
        av[src % 16][8 * (src / 16) + e] = bf16f(o.a[e]);
        bk[8 * (src / 16) + e][src % 16] = bf16f(o.b[e]);
      }
    }
    float* d = wave_result();
    for (int i = 0; i < 16; ++i) {
      f32x16 acc = 0.f;
      for (int k = 0; k < 32; ++k) acc += av[i][k] * bk[k];
      std::memcpy(d + 16 * i, &acc, sizeof(acc));
    }
  }
  wave_sync();
  const float* d = wave_result();
  A out = c;
  for (int r = 0; r < 4; ++r) out[r] += d[16 * (4 * (l / 16) + r) + l % 16];
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
