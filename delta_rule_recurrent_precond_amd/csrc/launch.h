// Internal launchers behind the C ABI (not exported).  Arguments are
// validated by the caller (osdn_api.hip) before any of these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace osdn {

// Bits of the flags the kernels take: q, k arrive unnormalised; beta, r arrive
// as logits; (internal) the given write keys are the unnormalised keys
// themselves; alpha holds one gate per key dimension; (internal) the write
// keys kt are fp32 whatever the data type (the two-phase forward keeps them
// in its scratch at full precision: rounded to bf16 they would cost up to
// 2^-9 relative per element, which near-orthogonal q . kt products amplify).
constexpr unsigned kNormQK = 2u, kGateLogits = 4u, kNormKt = 8u, kGateChannels = 16u,
                   kKtF32 = 32u;

struct ScanArgs {
  const void *k;
  const float *beta, *r, *d0;
  float eta;
  int B, H, T, dk, dtype;
  int mode_off;          // 1: plain delta rule (only the residual-ratio sums are produced)
  void *k_tilde;         // [B,H,T,dk] dtype (unused when mode_off)
  float *d_final, *d_all, *log_ratio, *log_ratio_sum;  // optional
  unsigned xf;           // input transforms (kNormQK: k unnormalised; kGateLogits: beta, r logits);
                         // kKtF32: k_tilde is fp32
};

struct ChunkArgs {
  const void *q, *k, *k_tilde, *v;
  const float *beta, *alpha, *S0;  // alpha: optional state gate
  int B, H, T, dk, dv, chunk, dtype;
  void *o;
  float *S_final;
  unsigned xf;  // input transforms of q, k and beta (kNormQK, kGateLogits); kKtF32: k_tilde fp32
};

struct FusedArgs {
  const void *q, *k, *v;
  const float *beta, *r, *alpha, *d0, *S0;  // alpha: optional state gate
  float eta;
  int B, H, T, dk, dv, chunk, dtype;
  int precond_off;
  void *o;
  float *S_final, *d_final, *log_ratio_sum;
  unsigned xf;  // input transforms (kNormQK, kGateLogits)
};

struct StepArgs {
  const void *q, *k, *v;
  const float *beta, *r, *alpha;  // alpha: optional state gate
  float eta;
  int B, H, dk, dv, dtype;
  float *S, *d;   // updated in place
  void *o;
  float *log_ratio;  // optional
  unsigned xf;       // input transforms (kNormQK, kGateLogits)
};

// One decoding step with persistent (S, d), one workgroup per (b,h).
hipError_t launch_step(const StepArgs &a, hipStream_t s);

// Token-serial preconditioner walk, one wave per (b,h).
hipError_t launch_precond_scan_serial(const ScanArgs &a, hipStream_t s);

// Chunkwise state pass with fp32 vector arithmetic; any supported shape/dtype.
hipError_t launch_chunk_generic(const ChunkArgs &a, hipStream_t s);

// Fused single-kernel forward on matrix cores (bf16, dk = dv = 128, chunk = 64).
bool fused_supported(int dk, int dv, int chunk, int dtype);
hipError_t launch_fused_forward(const FusedArgs &a, hipStream_t s);
// The same kernel with the write keys read from memory (phase 2 alone).
hipError_t launch_fused_chunk(const ChunkArgs &a, hipStream_t s);
// Two-kernel chunkwise pass (bf16, dk = dv = 128, chunk 64): a chunk-parallel
// prep kernel writes per-chunk operands into `ws` (split_workspace_bytes), a
// state kernel runs the sequential pass.  given: kt from a.k_tilde, else kt = k.
size_t split_workspace_bytes(int B, int H, int T, bool gate_channels);
hipError_t launch_split_chunk(const ChunkArgs &a, bool given, void *ws, hipStream_t s);
// The same kernel's chunked preconditioner walk alone (bf16, dk = 128).
bool fused_scan_supported(int dk, int dtype);
hipError_t launch_fused_scan(const ScanArgs &a, hipStream_t s);

// The walk in three launches (bf16 keys, dk = 128, chunk 64; walk.hip):
// walk_prep + walk write per-chunk records (wrec, WREC bytes each) and the
// entry d and c of every chunk (wout, WOUT floats each), plus d_final,
// log_ratio and log_ratio_sum of `a`; launch_walk_scan adds walk_keys, which
// writes a.k_tilde and a.d_all, with wrec and wout carved from ws (at least
// walk_workspace_min_bytes; with walk_workspace_bytes two flags per chunk
// follow them, and the three may run as one launch, walk_scan_pipe).
// The record of (b h, chunk c) lies at wrec + (bh NC + c) rstride (rstride >=
// WREC).  flags: if given (words flags[(bh NC + c) fstride], any contents),
// walk_prep and the walk may run as one launch (walk_pipe) in which the
// records are announced through these flags.
bool walk_supported(int dk, int dtype);
size_t walk_workspace_bytes(int B, int H, int T);
size_t walk_workspace_min_bytes(int B, int H, int T);
hipError_t launch_walk(const ScanArgs &a, unsigned char *wrec, size_t rstride, float *wout,
                       hipStream_t s, unsigned long long *flags = nullptr, int fstride = 1);
// compute units of the current device; a value no earlier one-launch walk of
// this process used (for its flags)
int device_cus();
unsigned long long next_epoch();
hipError_t launch_walk_scan(const ScanArgs &a, void *ws, size_t ws_bytes, hipStream_t s);

// The forward in four launches (bf16, dk = dv = 128, chunk 64): the walk, then
// the chunk-parallel pass forming the write keys from the walk's results, then
// the state kernel; ws of split_forward_workspace_bytes.
// (larger with the per-channel gate, whose chunk records carry K (.) G and Q (.) G)
size_t split_forward_workspace_bytes(int B, int H, int T, bool gate_channels);
hipError_t launch_split_forward(const FusedArgs &a, void *ws, hipStream_t s);

}  // namespace osdn
