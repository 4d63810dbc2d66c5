// Phase 1 of OSDN: the preconditioner walk over the key stream, token by token.
//
// Source: gist.science technical summary of "OSDN: Improving Delta Rule with
// Provable Online Preconditioning in Linear Attention", §2.1 (write key
// kt = d (.) k), §2.2 (closed-form surrogate and its two-phase use), §2.3 (APF
// retention on d only), §3 (token-local residual ratio).
//
// One wave per (b,h).  Lane l holds EPL = max(1, dk/64) consecutive elements
// of k_t and d; the two inner products per token (||k||^2 and <d, k (.) k>)
// are wave reductions.  The chain that is serial over tokens is
// d -> a -> c -> d; key loads run a block ahead of it.  xf: kNormQK -- the
// keys arrive unnormalised and each is divided by its norm (one more wave
// reduction per token); kGateLogits -- beta and r arrive as logits.
#include "device.h"
#include "launch.h"

namespace osdn {

namespace {

constexpr int kBlock = 16;  // tokens per prefetch block

// KT: the type of the write keys written (T, or fp32 for the two-phase forward)
template <typename T, typename KT, int DK>
__global__ void __launch_bounds__(64)
precond_scan_serial(const T *__restrict__ k, const float *__restrict__ beta,
                    const float *__restrict__ r, const float *__restrict__ d0, float eta, int T_,
                    int mode_off, KT *__restrict__ k_tilde, float *__restrict__ d_final,
                    float *__restrict__ d_all, float *__restrict__ log_ratio,
                    float *__restrict__ log_ratio_sum, unsigned xf) {
  constexpr int EPL = DK >= 64 ? DK / 64 : 1;
  const int lane = threadIdx.x;
  const long bh = blockIdx.x;
  const bool active = (lane * EPL) < DK;
  const int e0 = lane * EPL;

  float d[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) d[e] = (active && d0 && !mode_off) ? d0[bh * DK + e0 + e] : 1.0f;

  const T *kh = k + bh * (long)T_ * DK;
  const float *bh_beta = beta + bh * (long)T_;
  const float *bh_r = r ? r + bh * (long)T_ : nullptr;
  float lsum = 0.0f;

  // Two register blocks of kBlock tokens: one is consumed while the next loads.
  float kA[kBlock][EPL], bA[kBlock], rA[kBlock];
  float kB[kBlock][EPL], bB[kBlock], rB[kBlock];
  auto load_block = [&](float (&kb)[kBlock][EPL], float (&bb)[kBlock], float (&rb)[kBlock],
                        int t0) {
#pragma unroll
    for (int j = 0; j < kBlock; ++j) {
      const int t = t0 + j;
      const bool ok = t < T_;
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        kb[j][e] = (ok && active) ? Elem<T>::load(kh + (long)t * DK + e0 + e) : 0.0f;
      const float bv = ok ? bh_beta[t] : 0.0f, rv = (ok && bh_r) ? bh_r[t] : 1.0f;
      bb[j] = (ok && (xf & kGateLogits)) ? sigmoid_gate(bv) : bv;
      rb[j] = (ok && bh_r && (xf & kGateLogits)) ? sigmoid_gate(rv) : rv;
    }
  };
  auto run_block = [&](const float (&kb)[kBlock][EPL], const float (&bb)[kBlock],
                       const float (&rb)[kBlock], int t0) {
#pragma unroll
    for (int j = 0; j < kBlock; ++j) {
      const int t = t0 + j;
      if (t >= T_) break;
      float kk[EPL], p[EPL], pn = 0.0f, pa = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) kk[e] = kb[j][e];
      if (xf & kNormQK) {
        float sq = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) sq = fmaf(kk[e], kk[e], sq);
        const float sc = unit_scale(wave_sum(sq));
#pragma unroll
        for (int e = 0; e < EPL; ++e) kk[e] *= sc;
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        p[e] = kk[e] * kk[e];
        pn += p[e];
        pa += d[e] * p[e];
      }
      const float n = wave_sum(pn);
      const float a = mode_off ? n : wave_sum(pa);
      const float b = bb[j];
      const float g = 1.0f - b * a;
      const long row = bh * (long)T_ + t;
      if (!mode_off && active) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          Elem<KT>::store(k_tilde + row * DK + e0 + e, d[e] * kk[e]);
          if (d_all) d_all[row * DK + e0 + e] = d[e];
        }
      }
      const float lr = logf(g * g);
      if (log_ratio && lane == 0) log_ratio[row] = lr;
      lsum += lr;
      if (!mode_off) {
        const float c = n > 0.0f ? eta * b * g / n : 0.0f;
        const float rt = rb[j];
#pragma unroll
        for (int e = 0; e < EPL; ++e) d[e] = rt * d[e] + c * p[e];
      }
    }
  };

  if (T_ > 0) load_block(kA, bA, rA, 0);
  for (int t0 = 0; t0 < T_; t0 += 2 * kBlock) {
    if (t0 + kBlock < T_) load_block(kB, bB, rB, t0 + kBlock);
    run_block(kA, bA, rA, t0);
    if (t0 + kBlock >= T_) break;
    if (t0 + 2 * kBlock < T_) load_block(kA, bA, rA, t0 + 2 * kBlock);
    run_block(kB, bB, rB, t0 + kBlock);
  }
  if (d_final && active && !mode_off) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) d_final[bh * DK + e0 + e] = d[e];
  }
  if (log_ratio_sum && lane == 0) log_ratio_sum[bh] = lsum;
}

template <typename T, typename KT>
hipError_t launch_serial_t(const ScanArgs &a, hipStream_t s) {
  const dim3 grid((unsigned)(a.B * a.H)), block(64);
#define OSDN_SCAN_CASE(DK_)                                                                     \
  case DK_:                                                                                     \
    hipLaunchKernelGGL((precond_scan_serial<T, KT, DK_>), grid, block, 0, s, (const T *)a.k,  \
                       a.beta, a.r, a.d0, a.eta, a.T, a.mode_off, (KT *)a.k_tilde, a.d_final, \
                       a.d_all, a.log_ratio, a.log_ratio_sum, a.xf);                           \
    break;
  switch (a.dk) {
    OSDN_SCAN_CASE(16)
    OSDN_SCAN_CASE(32)
    OSDN_SCAN_CASE(64)
    OSDN_SCAN_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef OSDN_SCAN_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_precond_scan_serial(const ScanArgs &a, hipStream_t s) {
  if ((long)a.B * a.H == 0) return hipSuccess;
  if (a.dtype != 0) return launch_serial_t<float, float>(a, s);
  return (a.xf & kKtF32) ? launch_serial_t<bf16, float>(a, s) : launch_serial_t<bf16, bf16>(a, s);
}

}  // namespace osdn
