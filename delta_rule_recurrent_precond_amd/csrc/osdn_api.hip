// C ABI of libosdn.so: argument checks, path selection and launches.
// Declarations and the meaning of every argument: include/osdn.h.
#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "../../include/osdn.h"
#include "launch.h"

#define OSDN_EXPORT extern "C" __attribute__((visibility("default")))

// Scratch of osdn_forward_noalloc: one fixed array in device memory, in place
// of a workspace argument.  Every GPU the library runs on holds its own copy
// for the life of the process.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): it uses the device
// address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = OSDN_NOALLOC_MAX_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool chunk_ok(int c) { return c == 16 || c == 32 || c == 64; }

// Sizes common to every entry point.
int check_sizes(int B, int H, int T, int dk, int dv, int chunk, int dtype, bool need_dv,
                bool need_chunk) {
  if (B < 0 || H < 0 || T < 0) return OSDN_ERR_SHAPE;
  if (dtype != OSDN_BF16 && dtype != OSDN_F32) return OSDN_ERR_UNSUPPORTED;
  if (!dim_ok(dk)) return OSDN_ERR_UNSUPPORTED;
  if (need_dv && !dim_ok(dv)) return OSDN_ERR_UNSUPPORTED;
  if (need_chunk && !chunk_ok(chunk)) return OSDN_ERR_UNSUPPORTED;
  const long long heads = (long long)B * H;
  if (heads > INT_MAX / 8) return OSDN_ERR_SHAPE;  // grid size; also bounds the products below
  const long long per_head = (long long)T * 128;
  if (heads > 0 && per_head > (LLONG_MAX / 8) / heads) return OSDN_ERR_SHAPE;
  return OSDN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? OSDN_OK : OSDN_ERR_HIP; }

// The device address of `scratch` on the current device, resolved with
// hipGetSymbolAddress the first time a call runs on that device and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_addr[kMaxDevices];

hipError_t scratch_address(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

bool use_fused(int dk, int dv, int chunk, int dtype) {
  return osdn::fused_supported(dk, dv, chunk, dtype);
}

// Scratch of the two-launch path: kt between the walk and the chunk pass, in
// fp32 whatever the data type, then (bf16 keys, dk = 128) the chunked walk's
// records.
size_t two_phase_kt_bytes(int B, int H, int T, int dk) {
  const size_t n = (size_t)B * H * T * dk * sizeof(float);
  return (n + 255) & ~(size_t)255;
}
size_t two_phase_bytes(int B, int H, int T, int dk, int dtype, unsigned flags) {
  if (flags & OSDN_PRECOND_OFF) return 0;
  return two_phase_kt_bytes(B, H, T, dk) +
         (osdn::walk_supported(dk, dtype) ? osdn::walk_workspace_bytes(B, H, T) : 0);
}

// Scratch that selects the fastest path: the split pipeline on the shapes of
// the matrix-core kernels, else what the two-launch path needs.
size_t ws_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype, unsigned flags) {
  if (use_fused(dk, dv, chunk, dtype))
    return osdn::split_forward_workspace_bytes(B, H, T, (flags & OSDN_GATE_PER_CHANNEL) != 0);
  return two_phase_bytes(B, H, T, dk, dtype, flags);
}

constexpr unsigned kFlags =
    OSDN_PRECOND_OFF | OSDN_NORM_QK | OSDN_GATE_LOGITS | OSDN_GATE_PER_CHANNEL;
// the kernels' bits from the ABI flags
unsigned transforms(unsigned flags) {
  return (flags & OSDN_NORM_QK ? osdn::kNormQK : 0u) |
         (flags & OSDN_GATE_LOGITS ? osdn::kGateLogits : 0u) |
         (flags & OSDN_GATE_PER_CHANNEL ? osdn::kGateChannels : 0u);
}

bool split_ok(int B, int H, int T, int dk, int dv, int chunk, int dtype, unsigned flags,
              size_t workspace_bytes, const void *workspace) {
  return use_fused(dk, dv, chunk, dtype) && workspace &&
         workspace_bytes >= osdn::split_forward_workspace_bytes(
                                B, H, T, (flags & OSDN_GATE_PER_CHANNEL) != 0);
}

// the single fused kernel takes the call: its shapes, not enough scratch for
// the split pipeline, and no per-channel gate (which then runs on the
// two-phase path)
bool fused_ok(int B, int H, int T, int dk, int dv, int chunk, int dtype, unsigned flags,
              size_t workspace_bytes, const void *workspace) {
  return use_fused(dk, dv, chunk, dtype) && !(flags & OSDN_GATE_PER_CHANNEL) &&
         !split_ok(B, H, T, dk, dv, chunk, dtype, flags, workspace_bytes, workspace);
}

}  // namespace

OSDN_EXPORT const char *osdn_status_str(int status) {
  switch (status) {
    case OSDN_OK: return "ok";
    case OSDN_ERR_NULL: return "a required pointer is NULL";
    case OSDN_ERR_SHAPE: return "a size is negative or the sizes overflow";
    case OSDN_ERR_UNSUPPORTED: return "dtype, dk, dv or chunk outside the supported set";
    case OSDN_ERR_WORKSPACE: return "workspace is NULL or smaller than required";
    case OSDN_ERR_HIP: return "the HIP runtime rejected a launch";
    case OSDN_ERR_TOO_LARGE: return "the call needs more scratch than the library's fixed array holds";
    default: return "unknown status";
  }
}

OSDN_EXPORT size_t osdn_precond_scan_workspace_bytes(int B, int H, int T, int dk, int dtype) {
  if (check_sizes(B, H, T, dk, 16, 16, dtype, false, false) != OSDN_OK) return (size_t)-1;
  return osdn::walk_supported(dk, dtype) ? osdn::walk_workspace_bytes(B, H, T) : 0;
}

OSDN_EXPORT int osdn_precond_scan(const void *k, const float *beta, const float *r,
                                  const float *d0, float eta, int B, int H, int T, int dk,
                                  int dtype, void *k_tilde, float *d_final, float *d_all,
                                  float *log_ratio, void *workspace, size_t workspace_bytes,
                                  void *stream) {
  int st = check_sizes(B, H, T, dk, 16, 16, dtype, false, false);
  if (st != OSDN_OK) return st;
  if ((long long)B * H == 0) return OSDN_OK;
  if (T > 0 && (!k || !beta || !k_tilde)) return OSDN_ERR_NULL;
  osdn::ScanArgs a{k, beta, r, d0, eta, B, H, T, dk, dtype, 0, k_tilde,
                   d_final, d_all, log_ratio, nullptr};
  if (osdn::walk_supported(dk, dtype) && workspace &&
      workspace_bytes >= osdn::walk_workspace_min_bytes(B, H, T))
    return hip_status(osdn::launch_walk_scan(a, workspace, workspace_bytes, (hipStream_t)stream));
  if (osdn::fused_scan_supported(dk, dtype))
    return hip_status(osdn::launch_fused_scan(a, (hipStream_t)stream));
  return hip_status(osdn::launch_precond_scan_serial(a, (hipStream_t)stream));
}

OSDN_EXPORT int osdn_step(const void *q, const void *k, const void *v, const float *beta,
                          const float *r, const float *alpha, float eta, int B, int H, int dk,
                          int dv, int dtype, unsigned flags, float *S, float *d, void *o,
                          float *log_ratio, void *stream) {
  int st = check_sizes(B, H, 1, dk, dv, 16, dtype, true, false);
  if (st != OSDN_OK) return st;
  if (flags & ~(OSDN_NORM_QK | OSDN_GATE_LOGITS | OSDN_GATE_PER_CHANNEL))
    return OSDN_ERR_UNSUPPORTED;
  if ((long long)B * H == 0) return OSDN_OK;
  if (!q || !k || !v || !beta || !S || !d || !o) return OSDN_ERR_NULL;
  if ((flags & OSDN_GATE_PER_CHANNEL) && !alpha) return OSDN_ERR_NULL;
  osdn::StepArgs a{q, k, v, beta, r, alpha, eta, B, H, dk, dv, dtype, S, d, o, log_ratio,
                   transforms(flags)};
  return hip_status(osdn::launch_step(a, (hipStream_t)stream));
}

OSDN_EXPORT size_t osdn_chunk_fwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk,
                                                  int dtype, unsigned flags) {
  if (check_sizes(B, H, T, dk, dv, chunk, dtype, true, true) != OSDN_OK) return (size_t)-1;
  if (flags & ~OSDN_GATE_PER_CHANNEL) return (size_t)-1;
  return use_fused(dk, dv, chunk, dtype)
             ? osdn::split_workspace_bytes(B, H, T, (flags & OSDN_GATE_PER_CHANNEL) != 0)
             : 0;
}

OSDN_EXPORT int osdn_chunk_fwd(const void *q, const void *k, const void *k_tilde, const void *v,
                               const float *beta, const float *alpha, const float *S0, int B,
                               int H, int T, int dk,
                               int dv, int chunk, int dtype, unsigned flags, void *o,
                               float *S_final, void *workspace, size_t workspace_bytes,
                               void *stream) {
  int st = check_sizes(B, H, T, dk, dv, chunk, dtype, true, true);
  if (st != OSDN_OK) return st;
  if (flags & ~OSDN_GATE_PER_CHANNEL) return OSDN_ERR_UNSUPPORTED;
  if ((long long)B * H == 0) return OSDN_OK;
  if (T > 0 && (!q || !k || !k_tilde || !v || !beta || !o)) return OSDN_ERR_NULL;
  const bool chan = (flags & OSDN_GATE_PER_CHANNEL) != 0;
  if (T > 0 && chan && !alpha) return OSDN_ERR_NULL;
  osdn::ChunkArgs a{q, k, k_tilde, v, beta, alpha, S0, B, H, T, dk, dv, chunk, dtype, o, S_final,
                    transforms(flags)};
  hipStream_t s = (hipStream_t)stream;
  if (use_fused(dk, dv, chunk, dtype)) {
    if (workspace && workspace_bytes >= osdn::split_workspace_bytes(B, H, T, chan))
      return hip_status(osdn::launch_split_chunk(a, true, workspace, s));
    if (!chan) return hip_status(osdn::launch_fused_chunk(a, s));
  }
  return hip_status(osdn::launch_chunk_generic(a, s));
}

OSDN_EXPORT size_t osdn_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk,
                                                int dtype, unsigned flags) {
  if (check_sizes(B, H, T, dk, dv, chunk, dtype, true, true) != OSDN_OK) return (size_t)-1;
  if (flags & ~kFlags) return (size_t)-1;
  return ws_bytes(B, H, T, dk, dv, chunk, dtype, flags);
}

OSDN_EXPORT const char *osdn_forward_path(int B, int H, int T, int dk, int dv, int chunk,
                                          int dtype, unsigned flags,
                                          size_t workspace_bytes) {
  if (check_sizes(B, H, T, dk, dv, chunk, dtype, true, true) != OSDN_OK) return "invalid";
  if (flags & ~kFlags) return "invalid";
  if ((long long)B * H == 0) return "none";
  const float one = 1.0f;
  if (split_ok(B, H, T, dk, dv, chunk, dtype, flags, workspace_bytes, &one))
    return "split";
  if (!fused_ok(B, H, T, dk, dv, chunk, dtype, flags, workspace_bytes, &one)) return "two-phase";
  return transforms(flags) ? "unsupported" : "fused";
}

OSDN_EXPORT int osdn_forward(const void *q, const void *k, const void *v, const float *beta,
                             const float *r, const float *alpha, const float *d0, const float *S0, float eta, int B,
                             int H, int T, int dk, int dv, int chunk, int dtype, unsigned flags,
                             void *o, float *S_final, float *d_final, float *log_ratio_sum,
                             void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_sizes(B, H, T, dk, dv, chunk, dtype, true, true);
  if (st != OSDN_OK) return st;
  if (flags & ~kFlags) return OSDN_ERR_UNSUPPORTED;
  const unsigned xf = transforms(flags);
  const bool split = split_ok(B, H, T, dk, dv, chunk, dtype, flags, workspace_bytes, workspace);
  const bool fused = fused_ok(B, H, T, dk, dv, chunk, dtype, flags, workspace_bytes, workspace);
  // the single fused kernel takes its inputs prepared
  if (xf && fused) return OSDN_ERR_UNSUPPORTED;
  if ((long long)B * H == 0) return OSDN_OK;
  if (T > 0 && (!q || !k || !v || !beta || !o)) return OSDN_ERR_NULL;
  if (T > 0 && (flags & OSDN_GATE_PER_CHANNEL) && !alpha) return OSDN_ERR_NULL;
  const bool off = (flags & OSDN_PRECOND_OFF) != 0;
  hipStream_t s = (hipStream_t)stream;

  if (split || fused) {
    osdn::FusedArgs a{q, k, v, beta, r, alpha, d0, S0, eta, B, H, T, dk, dv, chunk, dtype,
                      off ? 1 : 0, o, S_final, d_final, log_ratio_sum, xf};
    return hip_status(split ? osdn::launch_split_forward(a, workspace, s)
                            : osdn::launch_fused_forward(a, s));
  }

  // Two launches: the preconditioner walk writes kt into the workspace, then
  // the chunkwise pass reads it.
  const size_t need = two_phase_bytes(B, H, T, dk, dtype, flags);
  if (need > 0 && (!workspace || workspace_bytes < need)) return OSDN_ERR_WORKSPACE;
  const void *kt = k;
  const unsigned sxf = xf & (osdn::kNormQK | osdn::kGateLogits);  // what the walk transforms
  if (!off) {
    // kt in fp32 (osdn::kKtF32): the chunked walk (bf16 keys, dk = 128) with
    // its records after kt, else the token-serial walk
    osdn::ScanArgs sa{k, beta, r, d0, eta, B, H, T, dk, dtype, 0, workspace,
                      d_final, nullptr, nullptr, log_ratio_sum, sxf | osdn::kKtF32};
    st = hip_status(osdn::walk_supported(dk, dtype)
                        ? osdn::launch_walk_scan(
                              sa, (unsigned char *)workspace + two_phase_kt_bytes(B, H, T, dk),
                              workspace_bytes - two_phase_kt_bytes(B, H, T, dk), s)
                        : osdn::launch_precond_scan_serial(sa, s));
    if (st != OSDN_OK) return st;
    kt = workspace;
  } else if (log_ratio_sum) {
    osdn::ScanArgs sa{k, beta, nullptr, nullptr, 0.0f, B, H, T, dk, dtype, 1, nullptr,
                      nullptr, nullptr, nullptr, log_ratio_sum, sxf};
    st = hip_status(osdn::launch_precond_scan_serial(sa, s));
    if (st != OSDN_OK) return st;
  }
  // with kt = k (the delta rule) unnormalised keys are normalised on both sides
  osdn::ChunkArgs ca{q, k, kt, v, beta, alpha, S0, B, H, T, dk, dv, chunk, dtype, o, S_final,
                     xf | (off ? ((xf & osdn::kNormQK) ? osdn::kNormKt : 0u) : osdn::kKtF32)};
  return hip_status(osdn::launch_chunk_generic(ca, s));
}

OSDN_EXPORT int osdn_forward_noalloc(const void *q, const void *k, const void *v,
                                     const float *beta, const float *r, const float *alpha,
                                     const float *d0, const float *S0, float eta, int B, int H,
                                     int T, int dk, int dv, int chunk, int dtype, unsigned flags,
                                     void *o, float *S_final, float *d_final,
                                     float *log_ratio_sum, void *stream) {
  int st = check_sizes(B, H, T, dk, dv, chunk, dtype, true, true);
  if (st != OSDN_OK) return st;
  if (flags & ~kFlags) return OSDN_ERR_UNSUPPORTED;
  // the scratch of the fastest path, as osdn_forward_workspace_bytes reports it;
  // every byte of it is written before it is read, so nothing is cleared
  const size_t need = ws_bytes(B, H, T, dk, dv, chunk, dtype, flags);
  if (need > kScratchBytes) return OSDN_ERR_TOO_LARGE;
  void *ws = nullptr;
  if (need > 0 && (long long)B * H > 0 && T > 0) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return OSDN_ERR_HIP;
  }
  return osdn_forward(q, k, v, beta, r, alpha, d0, S0, eta, B, H, T, dk, dv, chunk, dtype, flags,
                      o, S_final, d_final, log_ratio_sum, ws, ws ? need : 0, stream);
}
