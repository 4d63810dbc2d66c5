// The preconditioner walk in two or three launches (bf16 keys, dk = 128, chunk 64).
//
// Source: gist.science technical summary of "OSDN: Improving Delta Rule with
// Provable Online Preconditioning in Linear Attention" -- §2.2 (the surrogate
// depends on k and beta only, so the walk over the key stream runs apart from
// the state; the two-phase implementation), §2.3 (APF retention keeps the d
// recurrence affine), §3 (rho_t = (1 - beta_t a_t)^2).
//
// Per (b, h) the walk is d_{t+1} = r_t d_t + c_t p_t with p_t = k_t (.) k_t,
// c_t = alpha_t g_t, g_t = 1 - beta_t a_t, a_t = <d_t, p_t>, alpha_t = eta
// beta_t / n_t (0 if n_t = ||k_t||^2 = 0).  Within a chunk of 64 tokens with
// entry value d_in, lg[t] = sum_{m<t} log2 r_m, Gamma_t = 2^lg[t] and
// R_{t,s} = 2^(lg[t] - lg[s+1]):
//   (I + M) g = 1 - beta (.) Gamma (.) (P d_in),  M_{t,s} = beta_t alpha_s R_{t,s} <p_t, p_s> (s < t)
//   d_out = Gamma_L d_in + sum_s R_{L,s} alpha_s g_s p_s
// Only the products with d_in depend on the previous chunk.  So:
//   walk_prep  chunk-parallel: (I + M)^-1 in fp32 and the per-token factors
//   walk       one workgroup per (b, h), sequential over chunks: three small
//              products per chunk give g, c_t = alpha_t g_t and the next d_in
//   walk_pipe  the two in one launch: the walks run on some compute units
//              while the others prepare the records in the order the walks
//              read them, handing each over through a flag (the walk, being
//              sequential, leaves most of the device idle)
//   walk_keys  chunk-parallel: d_t token by token from the chunk's entry value
//              and c (the recurrence itself, in fp32), writing kt_t = d_t (.) k_t
//              and, if asked, d_t
// The chunk-parallel pass of the forward (chunk_prep) runs the same in-chunk
// recurrence to form its write keys.
#include <atomic>
#include <chrono>
#include <random>

#include "device.h"
#include "launch.h"
#include "mfma.h"
#include "walk.h"
#include "walk_device.h"

namespace osdn {

namespace {

using namespace wd;

__global__ void __launch_bounds__(256)
walk_prep(const bf16 *__restrict__ k, const float *__restrict__ beta, const float *__restrict__ r,
          float eta, int T_, int NC, unsigned xf, unsigned char *__restrict__ wrec, size_t rstride) {
  __shared__ PrepSmem sm;
  // chunk-major, last chunk first, heads innermost (as chunk_prep): the walk
  // reads every head's chunk 0 first
  const int BHn = gridDim.x / NC;
  const int c = NC - 1 - (int)(blockIdx.x / BHn), bh = blockIdx.x % BHn;
  prep_chunk<false>(sm, prep_load(threadIdx.x, bh, c, k, beta, r, T_), threadIdx.x, bh, c, true,
                    r, eta, T_, NC, xf, wrec, rstride, [] {});
}

__global__ void __launch_bounds__(WT)
walk(const bf16 *__restrict__ k, const unsigned char *__restrict__ wrec, size_t rstride,
     const float *__restrict__ d0, int T_, int NC, float *__restrict__ wout,
     float *__restrict__ d_final, float *__restrict__ log_ratio,
     float *__restrict__ log_ratio_sum) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  walk_body<false, false>(smem_raw, blockIdx.x, k, wrec, rstride, d0, T_, NC, wout, d_final,
                          log_ratio, log_ratio_sum, nullptr, 0, 0);
}

// ---------------------------------------------------------------------------
// walk_pipe: walk_prep and the walk in one launch (see pipe_prep).  Workgroups
// 0 .. BH-1 walk (one per (b, h), as `walk`); the others prepare the records
// meanwhile.  The preparing workgroups never wait, so the walks, which wait
// only for them, always finish; being launched first, the walks' workgroups
// are placed first.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(WT)
walk_pipe(const bf16 *__restrict__ k, const float *__restrict__ beta, const float *__restrict__ r,
          float eta, unsigned xf, unsigned char *__restrict__ wrec, size_t rstride,
          const float *__restrict__ d0, int T_, int NC, int BH, float *__restrict__ wout,
          float *__restrict__ d_final, float *__restrict__ log_ratio,
          float *__restrict__ log_ratio_sum, unsigned long long *__restrict__ flags, int fstride,
          unsigned long long epoch) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  if ((int)blockIdx.x < BH) {
    walk_body<true, false>(smem_raw, blockIdx.x, k, wrec, rstride, d0, T_, NC, wout, d_final,
                           log_ratio, log_ratio_sum, flags, fstride, epoch);
    return;
  }
  pipe_prep(smem_raw, blockIdx.x - BH, gridDim.x - BH, BH, k, beta, r, eta, xf, wrec, rstride, T_,
            NC, flags, fstride, epoch);
}

// ---------------------------------------------------------------------------
// walk_keys: one workgroup per (b, h, chunk).  Threads 0-127 run the in-chunk
// recurrence for one key dimension each; then all threads store kt rows with
// 16-byte stores.  KT is the type of kt (bf16, or fp32 for the two-phase
// forward); xf: kNormQK -- kt is formed from the normalised key k_t / ||k_t||
// (the scale from the stored values, fp32); kGateLogits -- r arrives as logits.
// A bf16 kt is written over the staged keys (each element by the thread that
// read it, after reading it): 17 KB of LDS, so that eight workgroups fit on a
// CU and hide each other's load latency.
// ---------------------------------------------------------------------------
template <typename KT>
__global__ void __launch_bounds__(256)
walk_keys(const bf16 *__restrict__ k, const float *__restrict__ r,
          const float *__restrict__ wout, int T_, int NC, KT *__restrict__ k_tilde,
          float *__restrict__ d_all, unsigned xf) {
  constexpr int KTP = 16 / sizeof(KT);  // elements of kt per 16-byte piece
  constexpr int KTR = DK + KTP;         // padded kt row in LDS
  constexpr bool IN_PLACE = sizeof(KT) == sizeof(bf16);
  static_assert(!IN_PLACE || KTR == KP, "kt rows lie over the key rows");
  __shared__ __align__(16) unsigned char kbuf[C * KP * sizeof(bf16) + (IN_PLACE ? 0 : C * KTR * sizeof(KT))];
  bf16 *Kb = (bf16 *)kbuf;
  KT *Kt = IN_PLACE ? (KT *)kbuf : (KT *)(kbuf + C * KP * sizeof(bf16));
  __shared__ float cs[C], rs[C], sc[C];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / NC, c = blockIdx.x % NC;
  const long tok0 = (long)bh * T_ + (long)c * C;
  const int L = min(C, T_ - c * C);
  const float *wo = wout + ((long)bh * NC + c) * WOUT;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = tid + 256 * u, t = p >> 4, i0 = (p & 15) * 8;
    const uint4 kv = *(const uint4 *)(k + (tok0 + min(t, L - 1)) * DK + i0);
    const uint4 kz = t < L ? kv : uint4{0, 0, 0, 0};
    *(uint4 *)&Kb[t * KP + i0] = kz;
    // 1 / ||k_t|| from the 16 threads that hold row t (a zero row stays zero)
    const float n = group_sum<16>(sqsum8(kz));
    if ((p & 15) == 0) sc[t] = (xf & kNormQK) ? unit_scale(n) : 1.0f;
  }
  if (tid < C) {
    const int tb = min(tid, L - 1);
    const float cv = wo[DK + tid], rv = r ? r[tok0 + tb] : 1.0f;
    cs[tid] = tid < L ? cv : 0.f;
    rs[tid] = (r && tid < L) ? ((xf & kGateLogits) ? sigmoid_gate(rv) : rv) : 1.0f;
  }
  __syncthreads();
  if (tid < DK) {
    const int i = tid;
    float d = wo[i];
    for (int t0 = 0; t0 < C; t0 += 4) {
      const float4 c4 = *(const float4 *)&cs[t0], r4 = *(const float4 *)&rs[t0];
      const float4 s4 = *(const float4 *)&sc[t0];
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, rv[4] = {r4.x, r4.y, r4.z, r4.w};
      const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + e;
        const float kv = (float)Kb[t * KP + i] * sv[e];
        Elem<KT>::store(&Kt[t * KTR + i], d * kv);
        if (d_all && t < L) d_all[(tok0 + t) * DK + i] = d;
        d = fmaf(cv[e], kv * kv, rv[e] * d);
      }
    }
  }
  __syncthreads();
  constexpr int PIECES = C * DK / KTP;  // 16-byte pieces of the chunk's kt
#pragma unroll
  for (int u = 0; u < PIECES / 256; ++u) {
    const int p = tid + 256 * u, t = p / (DK / KTP), i0 = (p % (DK / KTP)) * KTP;
    if (t < L) *(uint4 *)(k_tilde + (tok0 + t) * DK + i0) = *(const uint4 *)&Kt[t * KTR + i0];
  }
}

}  // namespace

bool walk_supported(int dk, int dtype) { return dk == DK && dtype == 0; }

size_t walk_workspace_min_bytes(int B, int H, int T) {
  const size_t nc = (size_t)((T + C - 1) / C);
  return (size_t)B * H * nc * (WREC + WOUT * sizeof(float));
}

size_t walk_workspace_bytes(int B, int H, int T) {
  const size_t nc = (size_t)((T + C - 1) / C);
  return walk_workspace_min_bytes(B, H, T) + (size_t)B * H * nc * sizeof(unsigned long long);
}

// compute units of the current device (cached per device)
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// A value no earlier walk_pipe launch of this process used, and that memory
// left by anything else holds only by a 2^-64 chance: a random start, then
// one step per launch.
unsigned long long next_epoch() {
  static std::atomic<unsigned long long> ctr{[] {
    std::random_device rd;
    const unsigned long long t =
        (unsigned long long)std::chrono::steady_clock::now().time_since_epoch().count();
    return (((unsigned long long)rd() << 32) ^ rd()) ^ (t * 0x9E3779B97F4A7C15ull);
  }()};
  unsigned long long e;
  do e = ctr.fetch_add(1, std::memory_order_relaxed); while (e == 0);
  return e;
}

hipError_t launch_walk(const ScanArgs &a, unsigned char *wrec, size_t rstride, float *wout,
                       hipStream_t s, unsigned long long *flags, int fstride) {
  const int BH = a.B * a.H;
  const int NC = (a.T + C - 1) / C;
  if (BH == 0) return hipSuccess;
  // One launch when at least as many compute units are left to prepare the
  // records as there are walks: one workgroup per compute unit.
  const int cus = device_cus();
  if (flags && NC > 0 && 2 * BH <= cus) {
    hipError_t e = hipFuncSetAttribute((const void *)walk_pipe,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kPipeSmem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(walk_pipe, dim3((unsigned)cus), dim3(WT), kPipeSmem, s, (const bf16 *)a.k,
                       a.beta, a.r, a.eta, a.xf, wrec, rstride, a.d0, a.T, NC, BH, wout,
                       a.d_final, a.log_ratio, a.log_ratio_sum, flags, fstride, next_epoch());
    return hipGetLastError();
  }
  if (NC > 0)
    hipLaunchKernelGGL(walk_prep, dim3((unsigned)(BH * NC)), dim3(256), 0, s, (const bf16 *)a.k,
                       a.beta, a.r, a.eta, a.T, NC, a.xf, wrec, rstride);
  constexpr size_t shm = sizeof(WalkSmem);
  hipError_t e = hipFuncSetAttribute((const void *)walk,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(walk, dim3((unsigned)BH), dim3(WT), shm, s, (const bf16 *)a.k, wrec, rstride,
                     a.d0, a.T, NC, wout, a.d_final, a.log_ratio, a.log_ratio_sum);
  return hipGetLastError();
}

hipError_t launch_walk_scan(const ScanArgs &a, void *ws, size_t ws_bytes, hipStream_t s) {
  const int BH = a.B * a.H;
  const int NC = (a.T + C - 1) / C;
  if (BH == 0) return hipSuccess;
  unsigned char *wrec = (unsigned char *)ws;
  float *wout = (float *)(wrec + (size_t)BH * NC * WREC);
  // the ready flags past wout, if the workspace holds them
  unsigned long long *flags =
      ws_bytes >= walk_workspace_bytes(a.B, a.H, a.T)
          ? (unsigned long long *)(wrec + walk_workspace_min_bytes(a.B, a.H, a.T))
          : nullptr;
  hipError_t e = launch_walk(a, wrec, WREC, wout, s, flags, 1);
  if (e != hipSuccess || NC == 0) return e;
  if (a.xf & kKtF32)
    hipLaunchKernelGGL(walk_keys<float>, dim3((unsigned)(BH * NC)), dim3(256), 0, s,
                       (const bf16 *)a.k, a.r, (const float *)wout, a.T, NC, (float *)a.k_tilde,
                       a.d_all, a.xf);
  else
    hipLaunchKernelGGL(walk_keys<bf16>, dim3((unsigned)(BH * NC)), dim3(256), 0, s,
                       (const bf16 *)a.k, a.r, (const float *)wout, a.T, NC, (bf16 *)a.k_tilde,
                       a.d_all, a.xf);
  return hipGetLastError();
}

}  // namespace osdn
