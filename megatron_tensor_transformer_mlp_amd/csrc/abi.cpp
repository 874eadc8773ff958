// abi.cpp - the extern "C" entry points of libmshard.so declared in mshard.h:
// host-side validation (no device access), workspace sizing, a one-time check
// that the current device is a gfx950, then the launch sequences.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "launch.hpp"
#include "mshard.h"

namespace {

thread_local std::string g_last_error;

// Events armed by ms_arm_kernel_events, per kernel id, on this thread.
struct ArmedPair {
  hipEvent_t before = nullptr, after = nullptr;
};
thread_local ArmedPair g_armed[mshard::kTkCount];

// Disarms the listed kernels when an entry point returns, whatever the path.
struct DisarmOnReturn {
  int first, last;  // kernel ids [first, last] belong to one entry point
  ~DisarmOnReturn() {
    for (int id = first; id <= last; ++id) g_armed[id] = ArmedPair{};
  }
};

ms_status fail(ms_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

struct Buf {
  const void* p;
  size_t bytes;
  const char* name;
  bool output;
  bool whole_below_2g31 = true;  // false for a workspace: its regions are checked one by one
};

constexpr int64_t kMaxBytes = (int64_t)1 << 31;  // every buffer must be smaller than 2^31 bytes

// a * b * esize in bytes, saturated at 2^62 (dimensions are at most 2^31 - 1 each).
size_t nbytes(int64_t a, int64_t b, int64_t esize) {
  const int64_t cap = (int64_t)1 << 62;
  if (a <= 0 || b <= 0) return 0;
  if (a > cap / b) return (size_t)cap;
  const int64_t ab = a * b;
  if (ab > cap / esize) return (size_t)cap;
  return (size_t)(ab * esize);
}

// h, f_i and v_i are the leading dimensions of the GEMM operands; keeping them
// below 2^22 elements keeps every per-lane load offset of a 256-row tile, and
// every masked one, inside 32 bits (the kernels rely on it).
constexpr int64_t kMaxLd = (int64_t)1 << 22;

ms_status check_dims(int64_t T, std::initializer_list<std::pair<const char*, int64_t>> dims) {
  if (T < 1) return fail(MS_ERR_SHAPE, "T must be >= 1 (got %lld)", (long long)T);
  if (T > INT32_MAX) return fail(MS_ERR_SHAPE, "T too large (%lld)", (long long)T);
  for (auto& d : dims) {
    if (d.second < 8 || d.second % 8 != 0)
      return fail(MS_ERR_SHAPE, "%s must be a positive multiple of 8 (got %lld)", d.first, (long long)d.second);
    if (d.second >= kMaxLd)
      return fail(MS_ERR_SHAPE, "%s must be < 2^22 (got %lld)", d.first, (long long)d.second);
  }
  return MS_OK;
}

ms_status check_bufs(const std::vector<Buf>& bufs) {
  for (const Buf& b : bufs) {
    if (!b.p) return fail(MS_ERR_NULL, "%s is NULL", b.name);
    if (b.whole_below_2g31 && (int64_t)b.bytes >= kMaxBytes)
      return fail(MS_ERR_SHAPE, "%s is %zu bytes; each buffer must be < 2^31 bytes", b.name, b.bytes);
    if (((uintptr_t)b.p & 15) != 0) return fail(MS_ERR_ALIGN, "%s is not 16-byte aligned", b.name);
  }
  for (size_t i = 0; i < bufs.size(); ++i) {
    for (size_t j = i + 1; j < bufs.size(); ++j) {
      const Buf& a = bufs[i];
      const Buf& b = bufs[j];
      if (!a.output && !b.output) continue;  // inputs may share memory
      const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
      const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
      if (a0 < b1 && b0 < a1) return fail(MS_ERR_ALIAS, "%s overlaps %s", a.name, b.name);
    }
  }
  return MS_OK;
}

// The workspace as a whole may exceed 2^31 bytes: the kernels address each of
// its regions (and each split-K slice) through a resource of its own, so it is
// the largest region that must stay below 2^31 bytes.
ms_status check_workspace(const void* ws, size_t have, size_t need, size_t max_region, std::vector<Buf>& bufs) {
  if (need == 0) return MS_OK;
  if ((int64_t)max_region >= kMaxBytes)
    return fail(MS_ERR_SHAPE, "a workspace region would be %zu bytes; each must be < 2^31 bytes", max_region);
  if (!ws) return fail(MS_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (have < need) return fail(MS_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  bufs.push_back(Buf{ws, need, "workspace", true, false});
  return MS_OK;
}

template <class Layout>
ms_status check_workspace_layout(const void* ws, size_t have, const Layout& w, std::vector<Buf>& bufs) {
  return check_workspace(ws, have, w.bytes, w.max_region, bufs);
}

// One-time (per device) check that the current device is a gfx950.
ms_status check_device() {
  static std::mutex mu;
  static std::vector<int> ok_devices;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  for (int d : ok_devices)
    if (d == dev) return MS_OK;
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return fail(MS_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(MS_ERR_HIP, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
  ok_devices.push_back(dev);
  return MS_OK;
}

ms_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MS_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  g_last_error.clear();
  return MS_OK;
}

#define MS_TRY(x)                   \
  do {                              \
    ms_status _st = (x);            \
    if (_st != MS_OK) return _st;   \
  } while (0)

// Attention shard sizes: b, s >= 1 (b*s tokens), h as the other entry points,
// n >= 1 heads of size d (a multiple of 16, 16..128).  The core kernels' grids
// put the (head, sequence) pairs on x and the 64-row blocks of a sequence on y,
// so n*b < 2^31 and s <= 65535 * 64.
ms_status check_attn(int64_t b, int64_t s, int64_t h, int64_t n, int64_t d, int32_t causal) {
  if (b < 1 || s < 1 || n < 1) return fail(MS_ERR_SHAPE, "b, s and n must be >= 1 (got %lld, %lld, %lld)",
                                           (long long)b, (long long)s, (long long)n);
  if (n > INT32_MAX / b) return fail(MS_ERR_SHAPE, "n*b too large");
  if (s > (int64_t)65535 * 64) return fail(MS_ERR_SHAPE, "s must be <= 4194240 (got %lld)", (long long)s);
  if (s > INT32_MAX / b) return fail(MS_ERR_SHAPE, "b*s too large");
  if (d < 16 || d > 128 || d % 16 != 0)
    return fail(MS_ERR_SHAPE, "d must be a multiple of 16 in [16, 128] (got %lld)", (long long)d);
  if (causal != 0 && causal != 1) return fail(MS_ERR_ENUM, "causal must be 0 or 1 (got %d)", (int)causal);
  MS_TRY(check_dims(b * s, {{"h", h}, {"3nd", 3 * n * d}}));
  return MS_OK;
}

}  // namespace

namespace mshard {
void record_armed_event(int id, bool after, hipStream_t st) {
  const hipEvent_t ev = after ? g_armed[id].after : g_armed[id].before;
  if (ev) (void)hipEventRecord(ev, st);
}
}  // namespace mshard

extern "C" {

size_t mlp_shard_workspace_bytes(int64_t T, int64_t h, int64_t f_i) {
  if (check_dims(T, {{"h", h}, {"f_i", f_i}}) != MS_OK) return 0;
  return mshard::mlp_workspace_layout(T, h, f_i).bytes;
}

size_t mlp_shard_fwd_workspace_bytes(int64_t T, int64_t h, int64_t f_i) {
  if (check_dims(T, {{"h", h}, {"f_i", f_i}}) != MS_OK) return 0;
  const mshard::MlpWorkspace w = mshard::mlp_workspace_layout(T, h, f_i);
  return (w.fwd.tail_n > 0 || w.fwd.z_tail_n > 0) ? w.bytes : 0;
}

ms_status mlp_shard_fwd(const ms_bf16* X, const ms_bf16* A_i, const ms_bf16* b1_i, const ms_bf16* B_i,
                        int64_t T, int64_t h, int64_t f_i, ms_gelu gelu, ms_bf16* H_i, ms_bf16* Y_i, float* Z_i,
                        void* workspace, size_t workspace_bytes, void* stream) {
  const DisarmOnReturn disarm{mshard::kTkFwdH, mshard::kTkFwdZ};
  MS_TRY(check_dims(T, {{"h", h}, {"f_i", f_i}}));
  if (gelu != MS_GELU_ERF && gelu != MS_GELU_TANH) return fail(MS_ERR_ENUM, "unknown gelu form %d", (int)gelu);
  std::vector<Buf> bufs = {
      {X, nbytes(T, h, 2), "X", false},         {A_i, nbytes(h, f_i, 2), "A_i", false},
      {B_i, nbytes(f_i, h, 2), "B_i", false},   {H_i, nbytes(T, f_i, 2), "H_i", true},
      {Y_i, nbytes(T, f_i, 2), "Y_i", true},    {Z_i, nbytes(T, h, 4), "Z_i", true}};
  if (b1_i) bufs.push_back({b1_i, nbytes(f_i, 1, 2), "b1_i", false});
  // the workspace is used only when the plan splits the last tile columns of a GEMM
  const mshard::MlpWorkspace layout = mshard::mlp_workspace_layout(T, h, f_i);
  if (layout.fwd.tail_n > 0 || layout.fwd.z_tail_n > 0)
    MS_TRY(check_workspace_layout(workspace, workspace_bytes, layout, bufs));
  MS_TRY(check_bufs(bufs));
  MS_TRY(check_device());
  return launched(mshard::launch_mlp_fwd(X, A_i, b1_i, B_i, T, h, f_i, (int)gelu, H_i, Y_i, Z_i, workspace,
                                         (hipStream_t)stream),
                  "mlp_shard_fwd");
}

ms_status mlp_shard_bwd(const ms_bf16* X, const ms_bf16* A_i, const ms_bf16* B_i, const ms_bf16* H_i,
                        const ms_bf16* Y_i, const ms_bf16* dZ, int64_t T, int64_t h, int64_t f_i, ms_gelu gelu,
                        float* dX_i, ms_bf16* dA_i, ms_bf16* dB_i, ms_bf16* db1_i, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const DisarmOnReturn disarm{mshard::kTkBwdDH, mshard::kTkBwdDX};
  MS_TRY(check_dims(T, {{"h", h}, {"f_i", f_i}}));
  if (gelu != MS_GELU_ERF && gelu != MS_GELU_TANH) return fail(MS_ERR_ENUM, "unknown gelu form %d", (int)gelu);
  std::vector<Buf> bufs = {
      {X, nbytes(T, h, 2), "X", false},          {A_i, nbytes(h, f_i, 2), "A_i", false},
      {B_i, nbytes(f_i, h, 2), "B_i", false},    {H_i, nbytes(T, f_i, 2), "H_i", false},
      {Y_i, nbytes(T, f_i, 2), "Y_i", false},    {dZ, nbytes(T, h, 2), "dZ", false},
      {dX_i, nbytes(T, h, 4), "dX_i", true},     {dA_i, nbytes(h, f_i, 2), "dA_i", true},
      {dB_i, nbytes(f_i, h, 2), "dB_i", true}};
  if (db1_i) bufs.push_back({db1_i, nbytes(f_i, 1, 2), "db1_i", true});
  MS_TRY(check_workspace_layout(workspace, workspace_bytes, mshard::mlp_workspace_layout(T, h, f_i), bufs));
  MS_TRY(check_bufs(bufs));
  MS_TRY(check_device());
  return launched(mshard::launch_mlp_bwd(X, A_i, B_i, H_i, Y_i, dZ, T, h, f_i, (int)gelu, dX_i, dA_i, dB_i,
                                         db1_i, workspace, (hipStream_t)stream),
                  "mlp_shard_bwd");
}

size_t vocab_ce_workspace_bytes(int64_t T, int64_t h, int64_t v_i) {
  if (check_dims(T, {{"h", h}, {"v_i", v_i}}) != MS_OK) return 0;
  return mshard::ce_workspace_layout(T, v_i).bytes;
}

ms_status vocab_ce_shard_fwd(const ms_bf16* X, const ms_bf16* E_i, const int64_t* target, int64_t T, int64_t h,
                             int64_t v_i, int64_t vocab_start, float* m_i, float* s_i, float* z_i,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const DisarmOnReturn disarm{mshard::kTkCeGemm, mshard::kTkCeGemm};
  MS_TRY(check_dims(T, {{"h", h}, {"v_i", v_i}}));
  if (vocab_start < 0) return fail(MS_ERR_SHAPE, "vocab_start must be >= 0 (got %lld)", (long long)vocab_start);
  std::vector<Buf> bufs = {{X, nbytes(T, h, 2), "X", false},     {E_i, nbytes(h, v_i, 2), "E_i", false},
                           {target, nbytes(T, 1, 8), "target", false}, {m_i, nbytes(T, 1, 4), "m_i", true},
                           {s_i, nbytes(T, 1, 4), "s_i", true},       {z_i, nbytes(T, 1, 4), "z_i", true}};
  MS_TRY(check_workspace_layout(workspace, workspace_bytes, mshard::ce_workspace_layout(T, v_i), bufs));
  MS_TRY(check_bufs(bufs));
  MS_TRY(check_device());
  return launched(mshard::launch_vocab_ce(X, E_i, target, T, h, v_i, vocab_start, m_i, s_i, z_i, workspace,
                                          (hipStream_t)stream),
                  "vocab_ce_shard_fwd");
}

size_t attn_shard_workspace_bytes(int64_t b, int64_t s, int64_t h, int64_t n, int64_t d) {
  if (check_attn(b, s, h, n, d, 0) != MS_OK) return 0;
  return mshard::attn_workspace_layout(b, s, h, n, d).bytes;
}

ms_status attn_shard_fwd(const ms_bf16* X, const ms_bf16* Wqkv_i, const ms_bf16* Wo_i, int64_t b, int64_t s,
                         int64_t h, int64_t n, int64_t d, int32_t causal, ms_bf16* QKV, ms_bf16* O, float* lse,
                         float* Z_i, void* workspace, size_t workspace_bytes, void* stream) {
  const DisarmOnReturn disarm{mshard::kTkAttnQkv, mshard::kTkAttnOut};
  (void)workspace;
  (void)workspace_bytes;  // the forward needs no workspace
  MS_TRY(check_attn(b, s, h, n, d, causal));
  const int64_t T = b * s, nd = n * d;
  std::vector<Buf> bufs = {{X, nbytes(T, h, 2), "X", false},          {Wqkv_i, nbytes(h, 3 * nd, 2), "Wqkv_i", false},
                           {Wo_i, nbytes(nd, h, 2), "Wo_i", false},   {QKV, nbytes(T, 3 * nd, 2), "QKV", true},
                           {O, nbytes(T, nd, 2), "O", true},          {lse, nbytes(n, T, 4), "lse", true},
                           {Z_i, nbytes(T, h, 4), "Z_i", true}};
  MS_TRY(check_bufs(bufs));
  MS_TRY(check_device());
  return launched(mshard::launch_attn_fwd(X, Wqkv_i, Wo_i, b, s, h, n, d, causal == 1, QKV, O, lse, Z_i,
                                          (hipStream_t)stream),
                  "attn_shard_fwd");
}

ms_status attn_shard_bwd(const ms_bf16* X, const ms_bf16* Wqkv_i, const ms_bf16* Wo_i, const ms_bf16* QKV,
                         const ms_bf16* O, const float* lse, const ms_bf16* dZ, int64_t b, int64_t s, int64_t h,
                         int64_t n, int64_t d, int32_t causal, float* dX_i, ms_bf16* dWqkv_i, ms_bf16* dWo_i,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const DisarmOnReturn disarm{mshard::kTkAttnBwdDO, mshard::kTkAttnBwdDX};
  MS_TRY(check_attn(b, s, h, n, d, causal));
  const int64_t T = b * s, nd = n * d;
  std::vector<Buf> bufs = {{X, nbytes(T, h, 2), "X", false},          {Wqkv_i, nbytes(h, 3 * nd, 2), "Wqkv_i", false},
                           {Wo_i, nbytes(nd, h, 2), "Wo_i", false},   {QKV, nbytes(T, 3 * nd, 2), "QKV", false},
                           {O, nbytes(T, nd, 2), "O", false},         {lse, nbytes(n, T, 4), "lse", false},
                           {dZ, nbytes(T, h, 2), "dZ", false},        {dX_i, nbytes(T, h, 4), "dX_i", true},
                           {dWqkv_i, nbytes(h, 3 * nd, 2), "dWqkv_i", true},
                           {dWo_i, nbytes(nd, h, 2), "dWo_i", true}};
  MS_TRY(check_workspace_layout(workspace, workspace_bytes, mshard::attn_workspace_layout(b, s, h, n, d), bufs));
  MS_TRY(check_bufs(bufs));
  MS_TRY(check_device());
  return launched(mshard::launch_attn_bwd(X, Wqkv_i, Wo_i, QKV, O, lse, dZ, b, s, h, n, d, causal == 1, dX_i,
                                          dWqkv_i, dWo_i, workspace, (hipStream_t)stream),
                  "attn_shard_bwd");
}

size_t vocab_ce_bwd_workspace_bytes(int64_t T, int64_t h, int64_t v_i) {
  if (check_dims(T, {{"h", h}, {"v_i", v_i}}) != MS_OK) return 0;
  return mshard::ce_bwd_workspace_layout(T, h, v_i).bytes;
}

ms_status vocab_ce_shard_bwd(const ms_bf16* X, const ms_bf16* E_i, const int64_t* target, const float* m,
                             const float* s, int32_t t, const float* dloss, float grad_scale, int64_t T, int64_t h,
                             int64_t v_i, int64_t vocab_start, float* dX_i, ms_bf16* dE_i, void* workspace,
                             size_t workspace_bytes, void* stream) {
  const DisarmOnReturn disarm{mshard::kTkCeBwdL, mshard::kTkCeBwdDE};
  MS_TRY(check_dims(T, {{"h", h}, {"v_i", v_i}}));
  if (t < 1) return fail(MS_ERR_SHAPE, "t must be >= 1 (got %d)", (int)t);
  if (vocab_start < 0) return fail(MS_ERR_SHAPE, "vocab_start must be >= 0 (got %lld)", (long long)vocab_start);
  std::vector<Buf> bufs = {{X, nbytes(T, h, 2), "X", false},          {E_i, nbytes(h, v_i, 2), "E_i", false},
                           {target, nbytes(T, 1, 8), "target", false},  {m, nbytes(t, T, 4), "m", false},
                           {s, nbytes(t, T, 4), "s", false},            {dX_i, nbytes(T, h, 4), "dX_i", true},
                           {dE_i, nbytes(h, v_i, 2), "dE_i", true}};
  if (dloss) bufs.push_back({dloss, nbytes(T, 1, 4), "dloss", false});
  MS_TRY(check_workspace_layout(workspace, workspace_bytes, mshard::ce_bwd_workspace_layout(T, h, v_i), bufs));
  MS_TRY(check_bufs(bufs));
  MS_TRY(check_device());
  return launched(mshard::launch_vocab_ce_bwd(X, E_i, target, m, s, (int)t, dloss, grad_scale, T, h, v_i,
                                              vocab_start, dX_i, dE_i, workspace, (hipStream_t)stream),
                  "vocab_ce_shard_bwd");
}

ms_status vocab_ce_shard_fwd_noalloc(const ms_bf16* X, const ms_bf16* E_i, const int64_t* target, int64_t T,
                                     int64_t h, int64_t v_i, int64_t vocab_start, float* m_i, float* s_i, float* z_i,
                                     void* stream) {
  const DisarmOnReturn disarm{mshard::kTkCeGemm, mshard::kTkCeGemm};
  MS_TRY(check_dims(T, {{"h", h}, {"v_i", v_i}}));
  if (vocab_start < 0) return fail(MS_ERR_SHAPE, "vocab_start must be >= 0 (got %lld)", (long long)vocab_start);
  const size_t need = mshard::ce_workspace_layout(T, v_i).bytes;
  if (need > mshard::kNoAllocScratchBytes)
    return fail(MS_ERR_WORKSPACE,
                "vocab_ce_shard_fwd_noalloc: these sizes need %zu bytes of scratch, more than its fixed %zu",
                need, mshard::kNoAllocScratchBytes);
  std::vector<Buf> bufs = {{X, nbytes(T, h, 2), "X", false},           {E_i, nbytes(h, v_i, 2), "E_i", false},
                           {target, nbytes(T, 1, 8), "target", false}, {m_i, nbytes(T, 1, 4), "m_i", true},
                           {s_i, nbytes(T, 1, 4), "s_i", true},        {z_i, nbytes(T, 1, 4), "z_i", true}};
  MS_TRY(check_bufs(bufs));
  MS_TRY(check_device());
  void* scratch = nullptr;
  const hipError_t e = mshard::noalloc_scratch(&scratch);
  if (e != hipSuccess) return fail(MS_ERR_HIP, "scratch address lookup: %s", hipGetErrorString(e));
  return launched(mshard::launch_vocab_ce(X, E_i, target, T, h, v_i, vocab_start, m_i, s_i, z_i, scratch,
                                          (hipStream_t)stream),
                  "vocab_ce_shard_fwd_noalloc");
}

size_t ce_combine_workspace_bytes(int32_t t, int64_t T) {
  (void)t;
  (void)T;
  return 0;
}

ms_status ce_combine(const float* m, const float* s, const float* z, int32_t t, int64_t T, float* loss,
                     float* loss_mean, void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (t < 1) return fail(MS_ERR_SHAPE, "t must be >= 1 (got %d)", (int)t);
  if (T < 1 || T > INT32_MAX) return fail(MS_ERR_SHAPE, "T out of range (%lld)", (long long)T);
  std::vector<Buf> bufs = {{m, nbytes(t, T, 4), "m", false},
                           {s, nbytes(t, T, 4), "s", false},
                           {z, nbytes(t, T, 4), "z", false},
                           {loss, nbytes(T, 1, 4), "loss", true}};
  if (loss_mean) bufs.push_back({loss_mean, 4, "loss_mean", true});
  MS_TRY(check_bufs(bufs));
  MS_TRY(check_device());
  return launched(mshard::launch_ce_combine(m, s, z, t, T, loss, loss_mean, (hipStream_t)stream), "ce_combine");
}

size_t ms_fingerprint_words(size_t bytes, size_t chunk_bytes) {
  if (chunk_bytes < 8 || chunk_bytes % 8 != 0 || chunk_bytes > ((size_t)1 << 40)) return 0;
  if (bytes >= ((size_t)1 << 48)) return 0;
  const uint64_t n = mshard::fingerprint_chunk_count(bytes, chunk_bytes);
  if (n > (uint64_t)INT32_MAX) return 0;
  return (size_t)(1 + n);
}

ms_status ms_fingerprint(const void* buf, size_t bytes, size_t chunk_bytes, uint64_t* out, void* stream) {
  const size_t words = ms_fingerprint_words(bytes, chunk_bytes);
  if (words == 0)
    return fail(MS_ERR_SHAPE, "chunk_bytes must be a positive multiple of 8 (<= 2^40), bytes < 2^48 and at most "
                "2^31 - 1 chunks (got bytes %zu, chunk_bytes %zu)", bytes, chunk_bytes);
  if (!buf) return fail(MS_ERR_NULL, "buf is NULL");
  if (!out) return fail(MS_ERR_NULL, "out is NULL");
  if (((uintptr_t)buf & 7) != 0) return fail(MS_ERR_ALIGN, "buf is not 8-byte aligned");
  if (((uintptr_t)out & 7) != 0) return fail(MS_ERR_ALIGN, "out is not 8-byte aligned");
  const uintptr_t b0 = (uintptr_t)buf, b1 = b0 + bytes, o0 = (uintptr_t)out, o1 = o0 + words * 8;
  if (b0 < o1 && o0 < b1) return fail(MS_ERR_ALIAS, "out overlaps buf");
  MS_TRY(check_device());
  return launched(mshard::launch_fingerprint(buf, bytes, chunk_bytes, out, (hipStream_t)stream), "ms_fingerprint");
}

ms_status ms_arm_kernel_events(ms_kernel k, void* before, void* after) {
  if ((int)k < 0 || (int)k >= mshard::kTkCount) return fail(MS_ERR_ENUM, "unknown kernel id %d", (int)k);
  if ((before == nullptr) != (after == nullptr))
    return fail(MS_ERR_NULL, "ms_arm_kernel_events: give both events or neither");
  g_armed[k].before = (hipEvent_t)before;
  g_armed[k].after = (hipEvent_t)after;
  return MS_OK;
}

const char* ms_last_error(void) { return g_last_error.c_str(); }

const char* ms_version(void) { return "mshard 0.1.0 (gfx950)"; }

ms_status ms_device_info(int32_t device, int32_t* compute_units, int32_t* clock_khz) {
  if (!compute_units || !clock_khz) return fail(MS_ERR_NULL, "an output pointer is NULL");
  int cus = 0, khz = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, device);
  if (e != hipSuccess) return fail(MS_ERR_HIP, "hipDeviceGetAttribute(device %d): %s", (int)device, hipGetErrorString(e));
  *compute_units = cus;
  *clock_khz = khz;
  g_last_error.clear();
  return MS_OK;
}

}  // extern "C"
