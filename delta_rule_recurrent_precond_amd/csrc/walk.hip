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
//   walk_scan_pipe  the three in one launch: as walk_pipe, then the preparing
//              workgroups write the keys of each chunk the walks have passed
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
// walk_keys: one workgroup of 256 threads per (b, h, chunk).  Threads 0-127 run
// the in-chunk recurrence for one key dimension each; then all threads store
// kt rows with 16-byte stores.  KT is the type of kt (bf16, or fp32 for the
// two-phase forward); xf: kNormQK -- kt is formed from the normalised key
// k_t / ||k_t|| (the scale from the stored values, fp32); kGateLogits -- r
// arrives as logits.  A bf16 kt is written over the staged keys (each element
// by the thread that read it, after reading it): 18 KB of LDS, so that eight
// workgroups fit on a CU and hide each other's load latency.
// ---------------------------------------------------------------------------
template <typename KT>
struct KeysLds {
  static constexpr int KTP = 16 / sizeof(KT);  // elements of kt per 16-byte piece
  static constexpr int KTR = DK + KTP;         // padded kt row
  static constexpr bool IN_PLACE = sizeof(KT) == sizeof(bf16);
  static_assert(!IN_PLACE || KTR == KP, "kt rows lie over the key rows");
  __align__(16) unsigned char kbuf[C * KP * sizeof(bf16) + (IN_PLACE ? 0 : C * KTR * sizeof(KT))];
  float cs[C], rs[C], sc[C];
};

// NI (b, h, chunk) items at once, item n in L[n]: the loads of all of them
// first, then thread t runs dimension t % 128 of item t / 128 (tid < 128 NI).
// COH: the walk's results (wout) come from a walk running in the same launch,
// read with device-scope loads once its flag is seen; poison[n]: item n's flag
// never came, so its d starts NaN and its kt turns NaN.
template <typename KT, bool COH, int NI>
__device__ __forceinline__ void keys_body(KeysLds<KT> *L, const int tid, const int *bhs,
                                          const int *cks, const bool *poison,
                                          const bf16 *__restrict__ k, const float *__restrict__ r,
                                          const float *__restrict__ wout, int T_, int NC,
                                          KT *__restrict__ k_tilde, float *__restrict__ d_all,
                                          unsigned xf) {
  using Ld = KeysLds<KT>;
  static_assert(NI == 1 || NI == 2, "one thread per dimension of every item (256 threads)");
  long tok0[NI];
  int len[NI];
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    tok0[n] = (long)bhs[n] * T_ + (long)cks[n] * C;
    len[n] = min(C, T_ - cks[n] * C);
  }
  auto wo = [&](int n) { return wout + ((long)bhs[n] * NC + cks[n]) * WOUT; };
  auto ld_wout = [&](const float *p) {
    return COH ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *p;
  };
  uint4 kz[NI][4];
#pragma unroll
  for (int n = 0; n < NI; ++n)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = tid + 256 * u, t = p >> 4, i0 = (p & 15) * 8;
      const uint4 kv = *(const uint4 *)(k + (tok0[n] + min(t, len[n] - 1)) * DK + i0);
      kz[n][u] = t < len[n] ? kv : uint4{0, 0, 0, 0};
    }
#pragma unroll
  for (int n = 0; n < NI; ++n)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = tid + 256 * u, t = p >> 4, i0 = (p & 15) * 8;
      *(uint4 *)&((bf16 *)L[n].kbuf)[t * KP + i0] = kz[n][u];
      // 1 / ||k_t|| from the 16 threads that hold row t (a zero row stays zero)
      const float nrm = group_sum<16>(sqsum8(kz[n][u]));
      if ((p & 15) == 0) L[n].sc[t] = (xf & kNormQK) ? unit_scale(nrm) : 1.0f;
    }
  if (tid < C) {
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int tb = min(tid, len[n] - 1);
      const float cv = ld_wout(&wo(n)[DK + tid]), rv = r ? r[tok0[n] + tb] : 1.0f;
      L[n].cs[tid] = tid < len[n] ? cv : 0.f;
      L[n].rs[tid] = (r && tid < len[n]) ? ((xf & kGateLogits) ? sigmoid_gate(rv) : rv) : 1.0f;
    }
  }
  __syncthreads();
  if (tid < NI * DK) {
    const int n = tid / DK, i = tid % DK;
    Ld &M = L[n];
    const bf16 *Kb = (const bf16 *)M.kbuf;
    KT *Kt = Ld::IN_PLACE ? (KT *)M.kbuf : (KT *)(M.kbuf + C * KP * sizeof(bf16));
    // item n's values by selection (NI <= 2), not by indexing the register arrays
    const bool n0 = n == 0;
    const long t0k = n0 ? tok0[0] : tok0[NI - 1];
    const int ln = n0 ? len[0] : len[NI - 1];
    float d = ld_wout(&(n0 ? wo(0) : wo(NI - 1))[i]);
    if (COH && (n0 ? poison[0] : poison[NI - 1])) d = __uint_as_float(0x7fc00000u);
    for (int t0 = 0; t0 < C; t0 += 4) {
      const float4 c4 = *(const float4 *)&M.cs[t0], r4 = *(const float4 *)&M.rs[t0];
      const float4 s4 = *(const float4 *)&M.sc[t0];
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, rv[4] = {r4.x, r4.y, r4.z, r4.w};
      const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + e;
        const float kv = (float)Kb[t * KP + i] * sv[e];
        Elem<KT>::store(&Kt[t * Ld::KTR + i], d * kv);
        if (d_all && t < ln) d_all[(t0k + t) * DK + i] = d;
        d = fmaf(cv[e], kv * kv, rv[e] * d);
      }
    }
  }
  __syncthreads();
  constexpr int PIECES = C * DK / Ld::KTP;  // 16-byte pieces of a chunk's kt
#pragma unroll
  for (int n = 0; n < NI; ++n) {
    const KT *Kt = Ld::IN_PLACE ? (const KT *)L[n].kbuf
                                : (const KT *)(L[n].kbuf + C * KP * sizeof(bf16));
#pragma unroll
    for (int u = 0; u < PIECES / 256; ++u) {
      const int p = tid + 256 * u, t = p / (DK / Ld::KTP), i0 = (p % (DK / Ld::KTP)) * Ld::KTP;
      if (t < len[n])
        *(uint4 *)(k_tilde + (tok0[n] + t) * DK + i0) = *(const uint4 *)&Kt[t * Ld::KTR + i0];
    }
  }
}

template <typename KT>
__global__ void __launch_bounds__(256)
walk_keys(const bf16 *__restrict__ k, const float *__restrict__ r,
          const float *__restrict__ wout, int T_, int NC, KT *__restrict__ k_tilde,
          float *__restrict__ d_all, unsigned xf) {
  __shared__ KeysLds<KT> L[1];
  const int bh = blockIdx.x / NC, c = blockIdx.x % NC;
  const bool poison = false;
  keys_body<KT, false, 1>(L, threadIdx.x, &bh, &c, &poison, k, r, wout, T_, NC, k_tilde, d_all,
                          xf);
}

// ---------------------------------------------------------------------------
// walk_scan_pipe: osdn_precond_scan in one launch.  As walk_pipe (the walks in
// workgroups 0 .. BH-1, the others preparing their records), but the walks
// publish their results (device-scope stores, and a second flag per chunk
// once a chunk's are complete), and the preparing workgroups, once their
// records are done, go on with walk_keys for every chunk, each instance of
// 256 threads taking kTailNI (b, h, chunk) items a round once their flags are
// set.  The walk_keys items (chunk-major, heads innermost, the order in which
// the walks finish them) continue the records' sequence of rounds from the
// next multiple of three, so every workgroup runs about the same number of
// rounds; a round whose items run past the last one repeats it (the same
// bytes written twice; walk_keys overwrites nothing that a wait reads).
// Two flags per chunk: flags[2 (bh NC + c)] the record, + 1 the walk's results.
// ---------------------------------------------------------------------------
// walk_keys items per instance and round in the tail: two with a bf16 kt (the
// loads of both in flight together), one with an fp32 kt (whose LDS is larger)
template <typename KT>
constexpr int kTailNI = sizeof(KT) == sizeof(bf16) ? 2 : 1;
template <typename KT>
constexpr size_t kScanPipeSmem = kPipeSmem > 3 * kTailNI<KT> * sizeof(KeysLds<KT>)
                                     ? kPipeSmem
                                     : 3 * kTailNI<KT> * sizeof(KeysLds<KT>);

template <typename KT>
__global__ void __launch_bounds__(WT)
walk_scan_pipe(const bf16 *__restrict__ k, const float *__restrict__ beta,
               const float *__restrict__ r, float eta, unsigned xf,
               unsigned char *__restrict__ wrec, const float *__restrict__ d0, int T_, int NC,
               int BH, float *__restrict__ wout, float *__restrict__ d_final,
               float *__restrict__ log_ratio, float *__restrict__ log_ratio_sum,
               unsigned long long *__restrict__ flags, unsigned long long epoch,
               KT *__restrict__ k_tilde, float *__restrict__ d_all) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  constexpr int fstride = 2;
  if ((int)blockIdx.x < BH) {
    walk_body<true, true>(smem_raw, blockIdx.x, k, wrec, WREC, d0, T_, NC, wout, d_final,
                          log_ratio, log_ratio_sum, flags, fstride, epoch);
    return;
  }
  const int j = blockIdx.x - BH, NPW = gridDim.x - BH;
  const int q0 = pipe_prep(smem_raw, j, NPW, BH, k, beta, r, eta, xf, wrec, WREC, T_, NC, flags,
                           fstride, epoch);
  constexpr int NI = kTailNI<KT>;
  const int inst = threadIdx.x >> 8;
  KeysLds<KT> *L = reinterpret_cast<KeysLds<KT> *>(smem_raw) + NI * inst;
  const int total = BH * NC;
  const int first = (total + 2) / 3 * 3;  // where the walk_keys items start in the sequence
  bool gave_up = false;  // once a wait ran out, later items do not wait
  // position pos of the sequence holds walk_keys items NI pos .. NI pos + NI - 1
  for (int qr = q0; NI * (3 * (NPW * qr + j) - first) < total; ++qr) {
    const int i0 = NI * (3 * (NPW * qr + j) - first + inst);
    int bhs[NI], cks[NI];
    bool bad[NI];
#pragma unroll
    for (int n = 0; n < NI; ++n) {
      const int ii = min(i0 + n, total - 1);
      cks[n] = ii / BH;
      bhs[n] = ii % BH;
      // the walk past chunk cks[n] (a bounded wait)
      bool ok = false;
      const unsigned long long *f = &flags[((long)bhs[n] * NC + cks[n]) * fstride + 1];
      for (int i = 0; !gave_up && i < kPollLimit; ++i) {
        if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) {
          ok = true;
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
      gave_up = !ok;
      bad[n] = !ok;
    }
    // (the thread index through an opaque copy each round, so that the
    // compiler does not hoist the body's lane-dependent addresses out of the
    // loop and keep them live across it)
    int tid = threadIdx.x & 255;
    asm volatile("" : "+v"(tid));
    keys_body<KT, true, NI>(L, tid, bhs, cks, bad, k, r, wout, T_, NC, k_tilde, d_all, xf);
    __syncthreads();  // the next round's staging overwrites this round's LDS
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
  return walk_workspace_min_bytes(B, H, T) + (size_t)B * H * nc * 2 * sizeof(unsigned long long);
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
  const bool f32 = (a.xf & kKtF32) != 0;
  // One launch (walk_scan_pipe) when the workspace holds the flags past wout
  // and at least as many compute units are left to prepare the records as
  // there are walks.
  const int cus = device_cus();
  if (ws_bytes >= walk_workspace_bytes(a.B, a.H, a.T) && NC > 0 && 2 * BH <= cus) {
    unsigned long long *flags =
        (unsigned long long *)(wrec + walk_workspace_min_bytes(a.B, a.H, a.T));
    const void *fn = f32 ? (const void *)walk_scan_pipe<float> : (const void *)walk_scan_pipe<bf16>;
    const size_t shm = f32 ? kScanPipeSmem<float> : kScanPipeSmem<bf16>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
    if (e != hipSuccess) return e;
    if (f32)
      hipLaunchKernelGGL(walk_scan_pipe<float>, dim3((unsigned)cus), dim3(WT), shm, s,
                         (const bf16 *)a.k, a.beta, a.r, a.eta, a.xf, wrec, a.d0, a.T, NC, BH,
                         wout, a.d_final, a.log_ratio, a.log_ratio_sum, flags, next_epoch(),
                         (float *)a.k_tilde, a.d_all);
    else
      hipLaunchKernelGGL(walk_scan_pipe<bf16>, dim3((unsigned)cus), dim3(WT), shm, s,
                         (const bf16 *)a.k, a.beta, a.r, a.eta, a.xf, wrec, a.d0, a.T, NC, BH,
                         wout, a.d_final, a.log_ratio, a.log_ratio_sum, flags, next_epoch(),
                         (bf16 *)a.k_tilde, a.d_all);
    return hipGetLastError();
  }
  hipError_t e = launch_walk(a, wrec, WREC, wout, s);
  if (e != hipSuccess || NC == 0) return e;
  if (f32)
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
