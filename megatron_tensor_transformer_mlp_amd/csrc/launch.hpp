// launch.hpp - host-side interface between the C ABI layer (abi.cpp) and the
// kernel launch sequences (kernels.hip).  Arguments reaching these functions
// have been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mshard {

// Launch plan of the backward: the four GEMMs form two independent pairs,
// (dB, dH) and (dA, dX); each pair runs as two launches or one paired launch.
struct BwdPlan {
  int splits_dB, splits_dA;  // K splits of the weight gradients (1 = none)
  bool pair_bh, pair_ax;     // (dB, dH) / (dA, dX) share one launch
  bool dh_first, dx_first;   // in a paired launch, the partner's blocks lead
};

// Launch plan of the forward's two GEMMs: when a GEMM's tiles leave the last
// round of workgroups mostly idle, its last tile columns are computed apart,
// their contraction split into workspace slices that a second kernel sums, in
// slice order.  X A_i with GeLU: tail_n columns split tail_splits ways, summed
// before the bias and GeLU.  Z = Y B_i: z_tail_n columns split z_tail_splits
// ways, summed into Z.  A tail of 0 columns: one plain launch.
struct FwdPlan {
  int tail_n;
  int tail_splits;
  int z_tail_n;
  int z_tail_splits;
};

struct MlpWorkspace {
  size_t off_dH;      // bf16 [T x f]: dH, consumed by the dA and dX GEMMs
  size_t off_db1;     // fp32 [db1_parts x f]: per-writer bias-gradient column sums
  size_t off_splitk;  // fp32 [S x h*f]: weight-gradient split-K slices
  size_t off_fwd_tail;  // fp32 [tail_splits x T x tail_n], then [z_tail_splits x T x z_tail_n]: the
                        // forward's tail slices, one GEMM's after the other's (the forward and the
                        // backward never use one workspace at the same time)
  size_t bytes;
  size_t max_region;  // largest piece one kernel addresses through one resource (a region or one slice)
  int db1_parts;
  BwdPlan plan;
  FwdPlan fwd;
};

struct CeWorkspace {
  size_t off_m, off_s, off_z;  // fp32 [parts x T] each
  size_t bytes;
  size_t max_region;
  int parts;
};

struct CeBwdWorkspace {
  size_t off_stats;   // [T] 16-byte per-token records
  size_t off_dL;      // bf16 [T x v]: the logit gradient
  size_t off_splitk;  // fp32 [S x h*v]: split-K slices of dE
  size_t bytes;
  size_t max_region;
  int splits_dE;      // K split of dE (1 = none)
  bool paired;        // dE and dX share one launch
  bool dx_first;      // in the paired launch, dX's blocks lead
};

// One rank's attention core: b sequences of s tokens, n heads of size d.
struct AttnGeom {
  int b, s, n, d;
  int ld_qkv;        // 3 n d: row stride of QKV
  int ld_o;          // n d: row stride of O (and dO)
  float scale_log2;  // log2(e) / sqrt(d)
};

// Attention shard backward workspace: dO, delta, dQKV and the split-K slices
// of the two weight gradients; each weight gradient is planned with its
// independent partner GEMM (dW_O with dO, dWqkv with dX).
struct AttnWorkspace {
  size_t off_dO;      // bf16 [T x nd]
  size_t off_delta;   // fp32 [n x T]
  size_t off_dqkv;    // bf16 [T x 3nd]
  size_t off_splitk;  // fp32 slices
  size_t bytes;
  size_t max_region;
  int splits_wo, splits_wqkv;
  bool pair_o, o_first;   // dW_O with dO in one launch; dO's blocks lead
  bool pair_x, x_first;   // dWqkv with dX in one launch; dX's blocks lead
};

// Kernel ids for the measurement hook (same values as ms_kernel in mshard.h).
enum TimedKernel {
  kTkCeGemm = 0, kTkFwdH, kTkFwdZ, kTkBwdDH, kTkBwdDB, kTkBwdDA, kTkBwdDX, kTkCeBwdL, kTkCeBwdDX, kTkCeBwdDE,
  kTkAttnQkv, kTkAttnCoreFwd, kTkAttnOut, kTkAttnBwdDO, kTkAttnBwdDWo, kTkAttnCoreBwd, kTkAttnBwdDWqkv,
  kTkAttnBwdDX, kTkCount
};

// Records the armed event (if any) of kernel `id` on `st`; `after` picks which
// of the pair.  Defined by the ABI layer, which owns the per-thread arming.
void record_armed_event(int id, bool after, hipStream_t st);

BwdPlan plan_backward(int64_t T, int64_t h, int64_t f);
FwdPlan plan_forward(int64_t T, int64_t h, int64_t f);
MlpWorkspace mlp_workspace_layout(int64_t T, int64_t h, int64_t f);
CeWorkspace ce_workspace_layout(int64_t T, int64_t v);
CeBwdWorkspace ce_bwd_workspace_layout(int64_t T, int64_t h, int64_t v);
AttnWorkspace attn_workspace_layout(int64_t b, int64_t s, int64_t h, int64_t n, int64_t d);

hipError_t launch_mlp_fwd(const uint16_t* X, const uint16_t* A, const uint16_t* b1, const uint16_t* B,
                          int64_t T, int64_t h, int64_t f, int gelu, uint16_t* H, uint16_t* Y, float* Z, void* ws,
                          hipStream_t st);
hipError_t launch_mlp_bwd(const uint16_t* X, const uint16_t* A, const uint16_t* B, const uint16_t* H,
                          const uint16_t* Y, const uint16_t* dZ, int64_t T, int64_t h, int64_t f, int gelu,
                          float* dX, uint16_t* dA, uint16_t* dB, uint16_t* db1, void* ws, hipStream_t st);
hipError_t launch_vocab_ce(const uint16_t* X, const uint16_t* E, const int64_t* target, int64_t T, int64_t h,
                           int64_t v, int64_t vocab_start, float* m, float* s, float* z, void* ws,
                           hipStream_t st);
hipError_t launch_vocab_ce_bwd(const uint16_t* X, const uint16_t* E, const int64_t* target, const float* m,
                               const float* s, int t, const float* dloss, float scale, int64_t T, int64_t h,
                               int64_t v, int64_t vocab_start, float* dX, uint16_t* dE, void* ws, hipStream_t st);
int attn_padded_dim(int d);
hipError_t launch_attn_core_fwd(const AttnGeom& g, bool causal, const uint16_t* qkv, uint16_t* out, float* lse,
                                hipStream_t st);
hipError_t launch_attn_core_bwd(const AttnGeom& g, bool causal, const uint16_t* qkv, const uint16_t* out,
                                const uint16_t* dout, const float* lse, float* delta, uint16_t* dqkv,
                                hipStream_t st);
hipError_t launch_attn_fwd(const uint16_t* X, const uint16_t* Wqkv, const uint16_t* Wo, int64_t b, int64_t s,
                           int64_t h, int64_t n, int64_t d, bool causal, uint16_t* QKV, uint16_t* O, float* lse,
                           float* Z, hipStream_t st);
hipError_t launch_attn_bwd(const uint16_t* X, const uint16_t* Wqkv, const uint16_t* Wo, const uint16_t* QKV,
                           const uint16_t* O, const float* lse, const uint16_t* dZ, int64_t b, int64_t s, int64_t h,
                           int64_t n, int64_t d, bool causal, float* dX, uint16_t* dWqkv, uint16_t* dWo, void* ws,
                           hipStream_t st);
// Scratch of the allocation-free CE entry point: one static device array per
// GPU, sized for the per-tile partials of every workload shape in use.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
// Device address of this GPU's scratch array (looked up once per device, with
// that device current).
hipError_t noalloc_scratch(void** ptr);
uint64_t fingerprint_chunk_count(uint64_t bytes, uint64_t chunk);
hipError_t launch_fingerprint(const void* buf, uint64_t bytes, uint64_t chunk, uint64_t* out, hipStream_t st);
hipError_t launch_ce_combine(const float* m, const float* s, const float* z, int t, int64_t T, float* loss,
                             float* loss_mean, hipStream_t st);

}  // namespace mshard
