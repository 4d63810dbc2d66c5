// Phase 2 of OSDN, any supported shape and dtype: the chunkwise delta-rule
// pass with the preconditioned write key, in fp32 vector arithmetic.
//
// Source: gist.science technical summary of "OSDN: Improving Delta Rule with
// Provable Online Preconditioning in Linear Attention", §2.1: replacing the
// write key k by kt = d (.) k keeps DeltaNet's chunkwise pipeline, with kt in
// the chunk gram and the intra-chunk scores.  For a chunk with entry state S
// (rows t = 0..L-1):
//   A  = strict_lower(diag(beta) K Kt^T)          mixed gram (read key K, write key Kt)
//   (I + A) X = diag(beta) (V - K S^T)            pseudo-values x_t = beta_t (v_t - S_{t-1} k_t)
//   O  = Q S^T + lower(Q Kt^T) X                  o_t = S_t q_t (scores include t = s)
//   S <- S + X^T Kt
// With the optional state gate alpha (S_t = alpha_t S_{t-1} + beta_t (v_t -
// alpha_t S_{t-1} k_t) kt_t^T) and gamma_t = prod_{m<=t} alpha_m within the
// chunk: A_ts and the scores P_ts carry gamma_t / gamma_s, the residual reads
// gamma_t S k_t, the output gamma_t S q_t, and S <- gamma_L S + sum_s
// (gamma_L / gamma_s) x_s kt_s^T.  Decay ratios are 2^(lg_t - lg_s) with lg the
// running sum of log2 alpha (clamped at -126 per token, so a zero gate gives
// 2^-126 rather than an infinite logarithm).
// With the per-channel gate (GK: alpha [T][DK], S_t = S_{t-1} diag(alpha_t) +
// x_t kt_t^T) the decays are per key dimension i, 2^(lg_t,i - lg_s,i): they
// enter every sum over i term by term (A_ts = beta_t sum_i k_ti kt_si
// 2^(lg_ti - lg_si), the residual and the output read S (g_t (.) k_t) and
// S (g_t (.) q_t), and S_ji <- 2^lg_Li S_ji + sum_s 2^(lg_Li - lg_si) x_sj kt_si).
// Each exponent is a difference of running sums with s <= t, so it never
// exceeds zero.
// This is the correctness path (used for fp32 data and for shapes the
// matrix-core kernel does not cover).  One workgroup per (b, h, dv tile),
// serial over chunks, everything of a chunk staged in LDS as fp32.
#include "device.h"
#include "launch.h"

namespace osdn {

namespace {

constexpr int kThreads = 256;

// KT: the type of the write keys (T, or fp32 from the two-phase forward's scratch)
template <typename T, typename KT, int DK, int DVT, int C, bool GK>
__global__ void __launch_bounds__(kThreads)
chunk_generic(const T *__restrict__ q, const T *__restrict__ k, const KT *__restrict__ kt,
              const T *__restrict__ v, const float *__restrict__ beta,
              const float *__restrict__ alpha, const float *__restrict__ S0, int T_, int dv,
              T *__restrict__ o, float *__restrict__ S_final, unsigned xf) {
  constexpr int DKP = DK + 1;          // padded rows (bank spread)
  constexpr int CP = C + 1;
  constexpr int XP = DVT + 1;
  constexpr int PARTS = kThreads / DVT;  // lanes cooperating on one column of X
  static_assert(PARTS <= 64 && (PARTS & (PARTS - 1)) == 0, "group must fit a wave");

  __shared__ float sK[C * DKP];   // K, then Q
  __shared__ float sKt[C * DKP];
  __shared__ float sS[DVT * DKP];
  __shared__ float sA[C * CP];    // A, then the scores P
  __shared__ float sX[C * XP];    // V - K S^T scaled (R), then X
  __shared__ float sV[C * DVT];
  __shared__ float sB[C];
  __shared__ float sLg[C];        // running sum of log2 alpha within the chunk
  __shared__ float sLgk[GK ? C * DK : 1];  // GK: the same per key dimension, [t][i]

  const int tid = threadIdx.x;
  const long bh = blockIdx.x;
  const int j0 = blockIdx.y * DVT;  // first value channel of this tile

  const long tok0 = bh * (long)T_;
  // q and k rows divided by their norms when they arrive unnormalised
  auto normalise_rows = [&](float *X) {
    for (int t = tid; t < C; t += kThreads) {
      float n = 0.0f;
      for (int i = 0; i < DK; ++i) n = fmaf(X[t * DKP + i], X[t * DKP + i], n);
      const float sc = unit_scale(n);
      for (int i = 0; i < DK; ++i) X[t * DKP + i] *= sc;
    }
  };
  for (int idx = tid; idx < DVT * DK; idx += kThreads) {
    const int j = idx / DK, i = idx % DK;
    sS[j * DKP + i] = S0 ? S0[(bh * dv + j0 + j) * DK + i] : 0.0f;
  }

  for (int c0 = 0; c0 < T_; c0 += C) {
    const int L = min(C, T_ - c0);
    // 1. stage the chunk
    for (int idx = tid; idx < C * DK; idx += kThreads) {
      const int t = idx / DK, i = idx % DK;
      const bool ok = t < L;
      const long g = (tok0 + c0 + t) * DK + i;
      sK[t * DKP + i] = ok ? Elem<T>::load(k + g) : 0.0f;
      sKt[t * DKP + i] = ok ? Elem<KT>::load(kt + g) : 0.0f;
    }
    for (int idx = tid; idx < C * DVT; idx += kThreads) {
      const int t = idx / DVT, j = idx % DVT;
      sV[idx] = t < L ? Elem<T>::load(v + (tok0 + c0 + t) * (long)dv + j0 + j) : 0.0f;
    }
    for (int t = tid; t < C; t += kThreads) {
      const float bv = t < L ? beta[tok0 + c0 + t] : 0.0f;
      sB[t] = (t < L && (xf & kGateLogits)) ? sigmoid_gate(bv) : bv;
    }
    if (GK) {
      for (int i = tid; i < DK; i += kThreads) {
        float acc = 0.0f;
        for (int t = 0; t < C; ++t) {
          if (t < L) acc += fmaxf(log2f(alpha[(tok0 + c0 + t) * DK + i]), -126.0f);
          sLgk[t * DK + i] = acc;
        }
      }
    } else if (tid == 0) {
      float acc = 0.0f;
      for (int t = 0; t < C; ++t) {
        if (alpha && t < L) acc += fmaxf(log2f(alpha[tok0 + c0 + t]), -126.0f);
        sLg[t] = acc;
      }
    }
    __syncthreads();
    if (xf & kNormQK) {
      normalise_rows(sK);
      if (xf & kNormKt) normalise_rows(sKt);
      __syncthreads();
    }

    // 2. mixed gram A and right-hand side R = diag(beta)(V - K S^T)
    for (int idx = tid; idx < C * C; idx += kThreads) {
      const int t = idx / C, s = idx % C;
      float acc = 0.0f;
      if (s < t) {
        if (GK) {
          for (int i = 0; i < DK; ++i)
            acc += sK[t * DKP + i] * sKt[s * DKP + i] * exp2f(sLgk[t * DK + i] - sLgk[s * DK + i]);
          acc *= sB[t];
        } else {
          for (int i = 0; i < DK; ++i) acc += sK[t * DKP + i] * sKt[s * DKP + i];
          acc *= sB[t];
          if (alpha) acc *= exp2f(sLg[t] - sLg[s]);
        }
      }
      sA[t * CP + s] = acc;
    }
    for (int idx = tid; idx < C * DVT; idx += kThreads) {
      const int t = idx / DVT, j = idx % DVT;
      float acc = 0.0f;
      if (GK) {
        for (int i = 0; i < DK; ++i) acc += sK[t * DKP + i] * exp2f(sLgk[t * DK + i]) * sS[j * DKP + i];
      } else {
        for (int i = 0; i < DK; ++i) acc += sK[t * DKP + i] * sS[j * DKP + i];
        if (alpha) acc *= exp2f(sLg[t]);
      }
      sX[t * XP + j] = sB[t] * (sV[idx] - acc);
    }
    __syncthreads();

    // Q replaces K (K is no longer read in this chunk)
    for (int idx = tid; idx < C * DK; idx += kThreads) {
      const int t = idx / DK, i = idx % DK;
      sK[t * DKP + i] = t < L ? Elem<T>::load(q + (tok0 + c0 + t) * DK + i) : 0.0f;
    }

    // 3. forward substitution (I + A) X = R, one column per group of PARTS lanes.
    //    Lane `part` owns rows s = part (mod PARTS); it alone writes and later
    //    reads those rows of X, so no cross-lane LDS ordering is needed.
    {
      const int j = tid / PARTS, part = tid % PARTS;
      for (int t = 0; t < L; ++t) {
        const float rhs = sX[t * XP + j];
        float acc = 0.0f;
        for (int s = part; s < t; s += PARTS) acc += sA[t * CP + s] * sX[s * XP + j];
        acc = group_sum<PARTS>(acc);
        if (part == (t % PARTS)) sX[t * XP + j] = rhs - acc;
      }
    }
    __syncthreads();
    if (xf & kNormQK) {
      normalise_rows(sK);
      __syncthreads();
    }

    // 4. intra-chunk scores P = lower(Q Kt^T) (diagonal included) into sA
    for (int idx = tid; idx < C * C; idx += kThreads) {
      const int t = idx / C, s = idx % C;
      float acc = 0.0f;
      if (s <= t) {
        if (GK) {
          for (int i = 0; i < DK; ++i)
            acc += sK[t * DKP + i] * sKt[s * DKP + i] * exp2f(sLgk[t * DK + i] - sLgk[s * DK + i]);
        } else {
          for (int i = 0; i < DK; ++i) acc += sK[t * DKP + i] * sKt[s * DKP + i];
          if (alpha) acc *= exp2f(sLg[t] - sLg[s]);
        }
      }
      sA[t * CP + s] = acc;
    }
    __syncthreads();

    // 5. output O = Q S^T + P X
    for (int idx = tid; idx < C * DVT; idx += kThreads) {
      const int t = idx / DVT, j = idx % DVT;
      if (t < L) {
        float acc = 0.0f;
        if (GK) {
          for (int i = 0; i < DK; ++i)
            acc += sK[t * DKP + i] * exp2f(sLgk[t * DK + i]) * sS[j * DKP + i];
        } else {
          for (int i = 0; i < DK; ++i) acc += sK[t * DKP + i] * sS[j * DKP + i];
          if (alpha) acc *= exp2f(sLg[t]);
        }
        for (int s = 0; s <= t; ++s) acc += sA[t * CP + s] * sX[s * XP + j];
        Elem<T>::store(o + (tok0 + c0 + t) * (long)dv + j0 + j, acc);
      }
    }
    __syncthreads();

    // 6. state update S += X^T Kt
    for (int idx = tid; idx < DVT * DK; idx += kThreads) {
      const int j = idx / DK, i = idx % DK;
      float acc = sS[j * DKP + i];
      if (GK) {
        const float lgL = sLgk[(L - 1) * DK + i];
        acc *= exp2f(lgL);
        for (int s = 0; s < L; ++s)
          acc += exp2f(lgL - sLgk[s * DK + i]) * sX[s * XP + j] * sKt[s * DKP + i];
      } else if (alpha) {
        const float lgL = sLg[L - 1];
        acc *= exp2f(lgL);
        for (int s = 0; s < L; ++s) acc += exp2f(lgL - sLg[s]) * sX[s * XP + j] * sKt[s * DKP + i];
      } else {
        for (int s = 0; s < L; ++s) acc += sX[s * XP + j] * sKt[s * DKP + i];
      }
      sS[j * DKP + i] = acc;
    }
    __syncthreads();
  }

  if (S_final) {
    for (int idx = tid; idx < DVT * DK; idx += kThreads) {
      const int j = idx / DK, i = idx % DK;
      S_final[(bh * dv + j0 + j) * DK + i] = sS[j * DKP + i];
    }
  }
}

template <typename T, typename KT, int DK, int DVT, bool GK>
hipError_t launch_c(const ChunkArgs &a, hipStream_t s, dim3 grid) {
  const dim3 block(kThreads);
#define OSDN_GEN_CASE(C_)                                                                      \
  case C_:                                                                                     \
    hipLaunchKernelGGL((chunk_generic<T, KT, DK, DVT, C_, GK>), grid, block, 0, s,             \
                       (const T *)a.q, (const T *)a.k, (const KT *)a.k_tilde, (const T *)a.v,  \
                       a.beta, a.alpha, a.S0, a.T, a.dv, (T *)a.o, a.S_final, a.xf);          \
    break;
  switch (a.chunk) {
    OSDN_GEN_CASE(16)
    OSDN_GEN_CASE(32)
    OSDN_GEN_CASE(64)
    default:
      return hipErrorInvalidValue;
  }
#undef OSDN_GEN_CASE
  return hipGetLastError();
}

template <typename T, typename KT, int DVT, bool GK>
hipError_t launch_dk(const ChunkArgs &a, hipStream_t s, dim3 grid) {
  switch (a.dk) {
    case 16: return launch_c<T, KT, 16, DVT, GK>(a, s, grid);
    case 32: return launch_c<T, KT, 32, DVT, GK>(a, s, grid);
    case 64: return launch_c<T, KT, 64, DVT, GK>(a, s, grid);
    case 128: return launch_c<T, KT, 128, DVT, GK>(a, s, grid);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, typename KT, bool GK>
hipError_t launch_g(const ChunkArgs &a, hipStream_t s) {
  const int dvt = a.dv >= 32 ? 32 : 16;
  const dim3 grid((unsigned)(a.B * a.H), (unsigned)(a.dv / dvt));
  return dvt == 32 ? launch_dk<T, KT, 32, GK>(a, s, grid) : launch_dk<T, KT, 16, GK>(a, s, grid);
}

// the per-channel gate takes its own instances (a [C][DK] table of decays)
template <typename T, typename KT>
hipError_t launch_t(const ChunkArgs &a, hipStream_t s) {
  if ((a.xf & kGateChannels) && a.alpha) return launch_g<T, KT, true>(a, s);
  return launch_g<T, KT, false>(a, s);
}

}  // namespace

hipError_t launch_chunk_generic(const ChunkArgs &a, hipStream_t s) {
  if ((long)a.B * a.H == 0) return hipSuccess;
  if (a.dtype != 0) return launch_t<float, float>(a, s);
  return (a.xf & kKtF32) ? launch_t<bf16, float>(a, s) : launch_t<bf16, bf16>(a, s);
}

}  // namespace osdn
