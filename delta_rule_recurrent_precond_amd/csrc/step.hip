// One decoding step of OSDN with persistent state: the token recurrence for a
// single token per (b, h), updating S and d in place.
//
// Source: gist.science technical summary of "OSDN: Improving Delta Rule with
// Provable Online Preconditioning in Linear Attention" -- §2.1 (write key
// kt = d (.) k and the delta-rule write), §2.2 (the surrogate's step on d),
// §2.3 (APF retention r), §3 (rho = (1 - beta a)^2) and the persistent (S, d)
// state the efficiency claims rest on.  For one token:
//   a = <d, k (.) k>,  n = ||k||^2,  kt = d (.) k
//   S <- alpha S (optional state gate, Gated DeltaNet's decay), or
//   S <- S diag(alpha) (per-channel gate, one per key dimension: KDA's decay)
//   u = v - S k,  S <- S + beta u kt^T,  o = S q (after the write)
//   rho = (1 - beta a)^2,  d <- r d + eta beta (1 - beta a) (k (.) k) / n  (0 if n = 0)
//
// One workgroup of 256 threads per (b, h).  The step reads and writes the
// dv x dk fp32 state once, so it is bound by HBM: a thread keeps four
// consecutive columns of some rows of S in registers between the two passes.
#include "device.h"
#include "launch.h"

namespace osdn {

namespace {

constexpr int NT = 256;

template <typename T, int DK>
__global__ void __launch_bounds__(NT)
osdn_step_kernel(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
                 const float *__restrict__ beta, const float *__restrict__ r,
                 const float *__restrict__ alpha, float eta, int dv,
                 float *__restrict__ S, float *__restrict__ d, T *__restrict__ o,
                 float *__restrict__ log_ratio, unsigned xf) {
  constexpr int TPR = DK / 4;         // threads per row of S (4 columns each)
  constexpr int RPP = NT / TPR;       // rows per pass
  __shared__ float kt_s[DK], k_s[DK], q_s[DK];
  __shared__ float red[NT / 64][2], redn[NT / 64][2];
  __shared__ float coef[2];           // beta, c

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long bh = blockIdx.x;
  const float bt = (xf & kGateLogits) ? sigmoid_gate(beta[bh]) : beta[bh];
  const bool chan = (xf & kGateChannels) != 0;
  const float at = (alpha && !chan) ? alpha[bh] : 1.0f;  // scalar state gate

  // key statistics and the write key (fp32), one thread per dimension
  float pn = 0.f, pa = 0.f, kv = 0.f, qv = 0.f, dv_ = 0.f;
  if (tid < DK) {
    kv = Elem<T>::load(k + bh * DK + tid);
    qv = Elem<T>::load(q + bh * DK + tid);
    dv_ = d[bh * DK + tid];
  }
  if (xf & kNormQK) {  // q and k arrive unnormalised: divide by their norms
    const float nk = wave_sum(kv * kv), nq = wave_sum(qv * qv);
    if (lane == 0) {
      redn[wave][0] = nk;
      redn[wave][1] = nq;
    }
    __syncthreads();
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      sk += redn[w][0];
      sq += redn[w][1];
    }
    kv *= unit_scale(sk);
    qv *= unit_scale(sq);
  }
  if (tid < DK) {
    k_s[tid] = kv;
    kt_s[tid] = dv_ * kv;
    q_s[tid] = qv;
    pn = kv * kv;
    pa = dv_ * (kv * kv);
  }
  pn = wave_sum(pn);
  pa = wave_sum(pa);
  if (lane == 0) {
    red[wave][0] = pn;
    red[wave][1] = pa;
  }
  __syncthreads();
  if (tid == 0) {
    float n = 0.f, a = 0.f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      n += red[w][0];
      a += red[w][1];
    }
    const float gk = 1.0f - bt * a;  // 1 - beta a
    if (log_ratio) log_ratio[bh] = logf(gk * gk);
    coef[0] = bt;
    coef[1] = n > 0.f ? eta * bt * gk / n : 0.f;
  }
  __syncthreads();

  // the state: rows j = tid / TPR + RPP * pass, columns 4 (tid % TPR) .. +3
  const int c4 = (tid % TPR) * 4;
  const float4 kc = *(const float4 *)&k_s[c4];
  const float4 ktc = *(const float4 *)&kt_s[c4];
  const float4 qc = *(const float4 *)&q_s[c4];
  // gates of this thread's four columns
  const float4 ac = chan ? *(const float4 *)(alpha + bh * DK + c4) : float4{at, at, at, at};
  for (int j = tid / TPR; j < dv; j += RPP) {
    float *row = S + (bh * dv + j) * DK + c4;
    float4 s = *(const float4 *)row;
    s.x *= ac.x, s.y *= ac.y, s.z *= ac.z, s.w *= ac.w;
    float sk = s.x * kc.x + s.y * kc.y + s.z * kc.z + s.w * kc.w;
    sk = group_sum<TPR>(sk);
    const float u = coef[0] * (Elem<T>::load(v + bh * dv + j) - sk);  // beta (v_j - (S k)_j)
    s.x = fmaf(u, ktc.x, s.x);
    s.y = fmaf(u, ktc.y, s.y);
    s.z = fmaf(u, ktc.z, s.z);
    s.w = fmaf(u, ktc.w, s.w);
    *(float4 *)row = s;
    float sq = s.x * qc.x + s.y * qc.y + s.z * qc.z + s.w * qc.w;
    sq = group_sum<TPR>(sq);
    if (tid % TPR == 0) Elem<T>::store(o + bh * dv + j, sq);
  }

  // d <- r d + c (k (.) k)
  if (tid < DK) {
    const float rt = r ? ((xf & kGateLogits) ? sigmoid_gate(r[bh]) : r[bh]) : 1.0f;
    const float kv = k_s[tid];
    d[bh * DK + tid] = fmaf(coef[1], kv * kv, rt * d[bh * DK + tid]);
  }
}

template <typename T>
hipError_t launch_t(const StepArgs &a, hipStream_t s) {
  const unsigned BH = (unsigned)(a.B * a.H);
  const T *q = (const T *)a.q, *k = (const T *)a.k, *v = (const T *)a.v;
  T *o = (T *)a.o;
#define OSDN_STEP(DKV)                                                                     \
  case DKV:                                                                                \
    hipLaunchKernelGGL((osdn_step_kernel<T, DKV>), dim3(BH), dim3(NT), 0, s, q, k, v,       \
                       a.beta, a.r, a.alpha, a.eta, a.dv, a.S, a.d, o, a.log_ratio, a.xf);                  \
    break;
  switch (a.dk) {
    OSDN_STEP(16)
    OSDN_STEP(32)
    OSDN_STEP(64)
    OSDN_STEP(128)
    default: return hipErrorInvalidValue;
  }
#undef OSDN_STEP
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step(const StepArgs &a, hipStream_t s) {
  if ((long)a.B * a.H == 0) return hipSuccess;
  return a.dtype == 0 ? launch_t<bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace osdn
