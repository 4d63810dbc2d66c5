// Fused OSDN forward on CDNA4 matrix cores: chunk length 64, dk = dv = 128,
// bf16 q/k/v/o in HBM, fp16 matrix-core operands with fp32 accumulation,
// fp32 state and preconditioner.
//
// Source: gist.science technical summary of "OSDN: Improving Delta Rule with
// Provable Online Preconditioning in Linear Attention" -- §2.1 (the write key
// kt = d (.) k replaces k in the chunk gram, the intra-chunk scores and the
// state update; nothing else in the chunkwise pipeline changes), §2.2 (the
// closed-form surrogate whose gradient drives d, depending on k and beta
// only, which is what lets the preconditioner walk run ahead of the state
// pass), §2.3 (APF retention acts on d only and keeps the d recurrence
// affine), §3 (token-local residual ratio rho_t = (1 - beta_t a_t)^2).
//
// One workgroup (4 waves) per (b, h, 32-wide tile of value channels), serial
// over chunks.  Per chunk of C = 64 tokens with entry state S and entry
// preconditioner d0:
//
//  preconditioner walk (affine in d, unrolled over the chunk):
//    p_t = k_t (.) k_t, n_t = ||k_t||^2, alpha_t = eta beta_t / n_t (0 if n_t = 0)
//    Gamma_t = prod_{m<t} r_m, R_{t,s} = prod_{s<m<t} r_m
//    e_j <- <d0, p_j>; for t = 0..C-1:  g_t = 1 - beta_t e_t,  c_t = alpha_t g_t,
//                                        e_j <- r_t e_j + c_t <p_j, p_t>
//      (e_t at step t equals a_t = <d_t, p_t>; the inner products <p_j, p_t>
//       form a gram computed on matrix cores)
//    d_t = Gamma_t d0 + sum_{s<t} R_{t,s} c_s p_s     (matrix cores, for kt only)
//    d_next = Gamma_C d0 + sum_s R_{C,s} c_s p_s      (fp32)
//    log rho_t = log g_t^2
//  state pass (mixed keys: K on the read side, Kt on the write side):
//    A = strict_lower(diag(beta) K Kt^T),  Tinv = (I + A)^-1 (blocked, 16x16 blocks)
//    R = diag(beta) (V - K S^T),  X = Tinv R
//    O = Q S^T + lower(Q Kt^T) X,  S <- S + X^T Kt
//
// The write keys enter fp16 scaled by a power of two ds (exact) chosen from
// the chunk's entry preconditioner, and every product with them is scaled
// back in fp32, so small preconditioners (APF) stay in fp16's normal range.
#include "device.h"
#include "launch.h"

namespace osdn {

namespace {

typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int C = 64;       // chunk length
constexpr int DK = 128;     // key dimension
constexpr int DVT = 32;     // value channels per workgroup
constexpr int NTH = 256;    // threads per workgroup
constexpr int KP = 136;     // padded row (halves) of [C][DK] tiles
constexpr int CP = 72;      // padded row (halves) of [*][C] tiles
constexpr int AP = 68;      // padded row (floats) of fp32 [C][C] tiles
constexpr int VP = 68;      // padded row (bf16) of the transposed value tile

enum Mode { kOsdn = 0, kDeltaNet = 1, kGiven = 2 };

struct Smem {
  f16 K[C * KP];        // chunk keys [t][i]
  f16 KT[DK * CP];      // chunk keys transposed [i][t]; in the preconditioned
                        // modes it is overwritten by the scaled write keys [i][t]
  f16 Q[C * KP];        // chunk queries [t][i]
  f16 Kt[C * KP];       // scaled write keys [t][i]
  f16 S[DVT * KP];      // state tile [j][i] (fp16 copy of the fp32 master)
  f16 Tm[C * CP];       // (I + A)^-1 [t][s]; the preconditioner walk's L first
  f16 P[C * CP];        // lower(Q Kt^T) [t][s]
  f16 RT[DVT * CP];     // R^T [j][t]
  f16 XT[DVT * CP];     // X^T [j][t]
  unsigned short VT[DVT * VP];  // value tile transposed [j][t], bf16 bits
  float A[C * AP];      // gram A [t][s] (also the walk's key gram)
  float d[2][DK];       // preconditioner at chunk entry (ping-pong)
  float dpart[2][DK];   // partial sums of the next entry preconditioner
  float beta[C], r[C], n[C], b[C], alpha[C], c[C], w[C];
  float lg[C + 1];      // lg[t] = sum_{m<t} log r_m
  float red[8];
};

__device__ __forceinline__ f32x4 mma32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 ld8(const f16 *p) { return *(const f16x8 *)p; }

// fp32 -> fp16, rounding a materialised fp32 value to nearest even.  The empty
// asm keeps the compiler from fusing the conversion into the producing FMA
// (a mixed-precision FMA would round once, straight to fp16), so equal fp32
// values always give equal fp16 values whichever code path produced them --
// which is what makes results bitwise reproducible across call boundaries.
__device__ __forceinline__ f16 h(float x) {
  asm volatile("" : "+v"(x));
  return (f16)x;
}

__device__ __forceinline__ float bf2f(unsigned short u) {
  return __builtin_bit_cast(float, ((unsigned)u) << 16);
}

// Lower-triangular 16x16 tile list of a 64x64 matrix (row tile, col tile).
__device__ __forceinline__ void tri_tile(int idx, int &rt, int &ct) {
  // (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) (3,1) (3,2) (3,3)
  rt = idx >= 6 ? 3 : idx >= 3 ? 2 : idx >= 1 ? 1 : 0;
  ct = idx - (rt * (rt + 1)) / 2;
}

template <int MODE>
__global__ void __launch_bounds__(NTH, 1)
osdn_fused_forward(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                   const bf16 *__restrict__ kt_in, const bf16 *__restrict__ v,
                   const float *__restrict__ beta, const float *__restrict__ r,
                   const float *__restrict__ d0, const float *__restrict__ S0, float eta,
                   int BH, int T_, bf16 *__restrict__ o, float *__restrict__ S_final,
                   float *__restrict__ d_final, float *__restrict__ log_ratio_sum) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem &sm = *reinterpret_cast<Smem *>(smem_raw);
  constexpr int NTILE = 128 / DVT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // Workgroup -> (head, value tile).  Consecutive workgroup ids are spread over
  // the 8 XCDs; keep the tiles of one head on one XCD so they share its L2.
  int bh, tile;
  {
    const int b = blockIdx.x;
    if ((BH & 7) == 0) {
      const int x = b & 7, idx = b >> 3;
      bh = (idx / NTILE) * 8 + x;
      tile = idx % NTILE;
    } else {
      bh = b / NTILE;
      tile = b % NTILE;
    }
  }
  const int j0 = tile * DVT;
  const long tok0 = (long)bh * T_;
  const bool writer = tile == 0;  // writes the per-head outputs (d, log-ratio sum)

  // ---- zero the upper triangles that the triangular products read as zero ----
  for (int idx = tid; idx < C * CP; idx += NTH) {
    sm.Tm[idx] = h(0.0f);
    sm.P[idx] = h(0.0f);
  }
  for (int i = tid; i < DK; i += NTH) sm.d[0][i] = (MODE == kOsdn && d0) ? d0[(long)bh * DK + i] : 1.0f;

  // ---- state: fp32 master S^T tiles in registers, wave w owns i-tiles 2w, 2w+1 ----
  f32x4 Sacc[2][2];  // [i sub-tile][j tile]
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int i0 = 16 * (2 * wave + mi) + 4 * g4;
      const int j = 16 * n + l16;
      if (S0) {
        const float4 s4 = *(const float4 *)(S0 + ((long)bh * 128 + j0 + j) * DK + i0);
        Sacc[mi][n] = f32x4{s4.x, s4.y, s4.z, s4.w};
      } else {
        Sacc[mi][n] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  auto write_state_f16 = [&]() {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int i0 = 16 * (2 * wave + mi) + 4 * g4;
        const int j = 16 * n + l16;
        const f16x4 hs = {h(Sacc[mi][n][0]), h(Sacc[mi][n][1]), h(Sacc[mi][n][2]),
                          h(Sacc[mi][n][3])};
        *(f16x4 *)&sm.S[j * KP + i0] = hs;
      }
  };
  write_state_f16();

  // ---- global -> register staging of one chunk (issued a chunk ahead) ----
  // K, Q, (k~ in the given-key mode): 64 rows x 16 pieces of 16 B; thread tid
  // takes rows tid/16 + 16 m, piece tid%16.  V tile: 64 rows x 4 pieces.
  uint4 pk[4], pq[4], pkt[4], pv;
  float pb = 0.f, pr = 1.f;
  auto load_chunk = [&](int c0) {
    const int L = min(C, T_ - c0);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int t = tid / 16 + 16 * m, piece = tid % 16;
      const bool ok = t < L;
      const long off = (tok0 + c0 + t) * DK + piece * 8;
      pk[m] = ok ? *(const uint4 *)(k + off) : uint4{0, 0, 0, 0};
      pq[m] = ok ? *(const uint4 *)(q + off) : uint4{0, 0, 0, 0};
      if (MODE == kGiven) pkt[m] = ok ? *(const uint4 *)(kt_in + off) : uint4{0, 0, 0, 0};
    }
    {
      const int t = tid / 4, piece = tid % 4;
      pv = t < L ? *(const uint4 *)(v + (tok0 + c0 + t) * 128 + j0 + piece * 8)
                 : uint4{0, 0, 0, 0};
    }
    if (tid < C) {
      const bool ok = tid < L;
      pb = ok ? beta[tok0 + c0 + tid] : 0.f;
      pr = (ok && r) ? r[tok0 + c0 + tid] : 1.f;
    }
  };

  float lr_sum = 0.f;  // wave 0 of the writer accumulates sum_t log rho_t
  int dcur = 0;
  if (T_ > 0) load_chunk(0);

  for (int c0 = 0; c0 < T_; c0 += C) {
    const int L = min(C, T_ - c0);
    // ================= P1: staging registers -> LDS =================
    __syncthreads();  // previous chunk is done with every buffer
    float kmax = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int t = tid / 16 + 16 * m, i0 = (tid % 16) * 8;
      const unsigned short *uk = (const unsigned short *)&pk[m];
      const unsigned short *uq = (const unsigned short *)&pq[m];
      f16x8 hk, hq;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hk[e] = h(bf2f(uk[e]));
        hq[e] = h(bf2f(uq[e]));
        if (MODE != kGiven) sm.KT[(i0 + e) * CP + t] = hk[e];
      }
      *(f16x8 *)&sm.K[t * KP + i0] = hk;
      *(f16x8 *)&sm.Q[t * KP + i0] = hq;
      if (MODE == kGiven) {
        const unsigned short *ut = (const unsigned short *)&pkt[m];
#pragma unroll
        for (int e = 0; e < 8; ++e) kmax = fmaxf(kmax, fabsf(bf2f(ut[e])));
      }
    }
    {
      const int t = tid / 4, jj = (tid % 4) * 8;
      const unsigned short *uv = (const unsigned short *)&pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.VT[(jj + e) * VP + t] = uv[e];
    }
    if (tid < C) {
      sm.beta[tid] = pb;
      sm.r[tid] = pr;
    }
    float ds = 1.0f;  // power-of-two scale of the fp16 write keys
    if (MODE == kGiven) {
      kmax = fmaxf(kmax, __shfl_xor(kmax, 1));
      kmax = fmaxf(kmax, __shfl_xor(kmax, 2));
      kmax = fmaxf(kmax, __shfl_xor(kmax, 4));
      kmax = fmaxf(kmax, __shfl_xor(kmax, 8));
      kmax = fmaxf(kmax, __shfl_xor(kmax, 16));
      kmax = fmaxf(kmax, __shfl_xor(kmax, 32));
      if (lane == 0) sm.red[wave] = kmax;
    }
    __syncthreads();

    if (MODE == kGiven) {
      const float km = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
      ds = km > 0.f ? exp2f(ceilf(log2f(km))) : 1.0f;
      const float inv = 1.0f / ds;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int t = tid / 16 + 16 * m, i0 = (tid % 16) * 8;
        const unsigned short *ut = (const unsigned short *)&pkt[m];
        f16x8 hv;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          hv[e] = h(bf2f(ut[e]) * inv);
          sm.KT[(i0 + e) * CP + t] = hv[e];
        }
        *(f16x8 *)&sm.Kt[t * KP + i0] = hv;
      }
    }
    // prefetch the next chunk (the staging registers are consumed) while this one runs
    if (c0 + C < T_) load_chunk(c0 + C);

    const f16 *Kt = (MODE == kDeltaNet) ? sm.K : sm.Kt;
    const f16 *KtT = sm.KT;

    // ================= P2: key statistics =================
    // wave w, tokens 16w + l16, dims 32 g4 .. +31
    if (MODE != kGiven) {
      const int t = 16 * wave + l16;
      const float *dv = sm.d[dcur];
      float pn = 0.f, pa = 0.f, dmx = 0.f;
#pragma unroll
      for (int q8 = 0; q8 < 4; ++q8) {
        const int i0 = 32 * g4 + 8 * q8;
        const f16x8 kk = ld8(&sm.K[t * KP + i0]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)kk[e];
          const float p = x * x;
          pn += p;
          pa += dv[i0 + e] * p;
          dmx = fmaxf(dmx, dv[i0 + e]);
        }
      }
      pn += __shfl_xor(pn, 16);
      pn += __shfl_xor(pn, 32);
      pa += __shfl_xor(pa, 16);
      pa += __shfl_xor(pa, 32);
      dmx = fmaxf(dmx, __shfl_xor(dmx, 16));
      dmx = fmaxf(dmx, __shfl_xor(dmx, 32));
      if (g4 == 0) {
        const float bt = sm.beta[t];
        sm.n[t] = pn;
        sm.b[t] = pa;
        sm.alpha[t] = (MODE == kOsdn && pn > 0.f) ? eta * bt / pn : 0.f;
      }
      if (lane == 0) sm.red[wave] = dmx;
      // prefix sums of log r (wave 0, lanes = tokens)
      if (wave == 0 && MODE == kOsdn) {
        const float lr = fmaxf(logf(sm.r[lane]), -80.f);
        float incl = lr;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(incl, off);
          if (lane >= off) incl += y;
        }
        sm.lg[lane + 1] = incl;
        if (lane == 0) sm.lg[0] = 0.f;
      }
    }
    __syncthreads();

    if (MODE == kOsdn) {
      const float dmax = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
      ds = dmax > 0.f ? exp2f(ceilf(log2f(dmax))) : 1.0f;

      // ---- key gram G = strict_lower(P P^T), P = k (.) k in fp16 -> sm.A ----
      for (int job = wave; job < 10; job += 4) {
        int rt, ct;
        tri_tile(job, rt, ct);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          f16x8 a = ld8(&sm.K[(16 * rt + l16) * KP + 32 * kk + 8 * g4]);
          f16x8 b = ld8(&sm.K[(16 * ct + l16) * KP + 32 * kk + 8 * g4]);
          acc = mma32(a * a, b * b, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * rt + 4 * g4 + e, col = 16 * ct + l16;
          sm.A[row * AP + col] = col < row ? acc[e] : 0.f;
        }
      }
      // zero the strictly upper tiles of the gram (read by the walk)
      for (int idx = tid; idx < C * C; idx += NTH) {
        const int row = idx / C, col = idx % C;
        if ((col >> 4) > (row >> 4)) sm.A[row * AP + col] = 0.f;
      }
      __syncthreads();

      // ---- the walk proper: one wave, lanes = tokens of the chunk ----
      if (wave == 0) {
        const int j = lane;
        float G[C];
#pragma unroll
        for (int q4 = 0; q4 < C / 4; ++q4) {
          const float4 g = *(const float4 *)&sm.A[j * AP + 4 * q4];
          G[4 * q4 + 0] = g.x;
          G[4 * q4 + 1] = g.y;
          G[4 * q4 + 2] = g.z;
          G[4 * q4 + 3] = g.w;
        }
        const float bj = sm.beta[j];
        const float al = sm.alpha[j];
        const float rj = sm.r[j];
        float e = sm.b[j];
        float ckeep = 0.f, gkeep = 1.f;
#pragma unroll
        for (int t = 0; t < C; ++t) {
          const float g = fmaf(-bj, e, 1.0f);
          const float cl = al * g;
          const float ct = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cl), t));
          const float rt = __builtin_bit_cast(
              float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rj), t));
          if (j == t) {
            ckeep = cl;
            gkeep = g;
          }
          e = fmaf(ct, G[t], rt * e);
        }
        sm.c[j] = ckeep;
        // weight of c_s p_s in the next entry preconditioner: R_{L,s}
        sm.w[j] = j < L ? expf(sm.lg[L] - sm.lg[j + 1]) * ckeep : 0.f;
        const float lr = j < L ? logf(gkeep * gkeep) : 0.f;
        lr_sum += wave_sum(lr);
      }
      __syncthreads();

      // ---- L[t][s] = R_{t,s} c_s (s < t) into sm.Tm (fp16) ----
      for (int idx = tid; idx < C * C; idx += NTH) {
        const int t = idx / C, s = idx % C;
        const float val = s < t ? expf(sm.lg[t] - sm.lg[s + 1]) * sm.c[s] : 0.f;
        sm.Tm[t * CP + s] = h(val);
      }
      // ---- next entry preconditioner (fp32): partial sums over halves of s ----
      {
        const int i = tid & 127, h = tid >> 7;
        float acc = 0.f;
#pragma unroll 8
        for (int s = 32 * h; s < 32 * h + 32; ++s) {
          const float x = (float)sm.KT[i * CP + s];
          acc = fmaf(sm.w[s], x * x, acc);
        }
        sm.dpart[h][i] = acc;
      }
      __syncthreads();
      if (tid < DK) {
        sm.d[dcur ^ 1][tid] =
            expf(sm.lg[L]) * sm.d[dcur][tid] + sm.dpart[0][tid] + sm.dpart[1][tid];
      }

      // ---- d_t for the chunk: D = Gamma d0^T + L P (matrix cores), kt = D (.) k / ds ----
      // Wave w owns i tiles 2w, 2w+1: it alone reads and then rewrites those rows of KT.
      {
        const float inv = 1.0f / ds;
        f16x4 kto[2][4];
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) {
          const int n = 2 * wave + nn;  // i tile
#pragma unroll
          for (int m = 0; m < 4; ++m) {  // t tile
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const int nk = m < 2 ? 1 : 2;
            for (int kk = 0; kk < nk; ++kk) {
              const f16x8 a = ld8(&sm.Tm[(16 * m + l16) * CP + 32 * kk + 8 * g4]);
              const f16x8 b = ld8(&sm.KT[(16 * n + l16) * CP + 32 * kk + 8 * g4]);
              acc = mma32(a, b * b, acc);
            }
            const int i = 16 * n + l16;
            const int t0 = 16 * m + 4 * g4;
            const f16x4 kv = *(const f16x4 *)&sm.KT[i * CP + t0];
            const float dbase = sm.d[dcur][i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float dt = fmaf(expf(sm.lg[t0 + e]), dbase, acc[e]);
              kto[nn][m][e] = h(dt * (float)kv[e] * inv);
            }
          }
        }
#pragma unroll
        for (int nn = 0; nn < 2; ++nn)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int i = 16 * (2 * wave + nn) + l16;
            const int t0 = 16 * m + 4 * g4;
            *(f16x4 *)&sm.KT[i * CP + t0] = kto[nn][m];
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.Kt[(t0 + e) * KP + i] = kto[nn][m][e];
          }
      }
      __syncthreads();
      dcur ^= 1;
    } else if (MODE == kDeltaNet) {
      // residual ratio of the plain delta rule: rho_t = (1 - beta_t ||k_t||^2)^2
      if (wave == 0) {
        const float g = 1.0f - sm.beta[lane] * sm.n[lane];
        lr_sum += wave_sum(lane < L ? logf(g * g) : 0.f);
      }
    } else {
      __syncthreads();
    }

    // ================= P3: grams A = beta K Kt^T (strict), P = Q Kt^T (incl.) =================
    for (int job = wave; job < 20; job += 4) {
      const bool isA = job < 10;
      int rt, ct;
      tri_tile(isA ? job : job - 10, rt, ct);
      const f16 *src = isA ? sm.K : sm.Q;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const f16x8 a = ld8(&src[(16 * rt + l16) * KP + 32 * kk + 8 * g4]);
        const f16x8 b = ld8(&Kt[(16 * ct + l16) * KP + 32 * kk + 8 * g4]);
        acc = mma32(a, b, acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * rt + 4 * g4 + e, col = 16 * ct + l16;
        if (isA) {
          sm.A[row * AP + col] = col < row ? sm.beta[row] * ds * acc[e] : 0.f;
        } else {
          sm.P[row * CP + col] = h(col <= row ? ds * acc[e] : 0.f);
        }
      }
    }
    __syncthreads();

    // ================= P4: Tinv = (I + A)^-1, 16x16 blocks =================
    // diagonal blocks: wave w inverts block w, lane c (< 16) solves column c
    if (lane < 16) {
      const int base = 16 * wave;
      float x[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        float acc = (t == lane) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < t; ++s) acc = fmaf(-sm.A[(base + t) * AP + base + s], x[s], acc);
        x[t] = acc;
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) sm.Tm[(base + t) * CP + base + lane] = h(x[t]);
    }
    __syncthreads();
    // off-diagonal blocks, by distance from the diagonal:
    //   T_ij = -T_ii * sum_{k=j}^{i-1} A_ik T_kj
    auto a_op = [&](int bi, int bk) {  // A block (bi, bk) as 16x16x16 A operand
      f16x4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = h(sm.A[(16 * bi + l16) * AP + 16 * bk + 4 * g4 + e]);
      return a;
    };
    auto t_bop = [&](int bk, int bj) {  // T block (bk, bj) as B operand (k = row)
      f16x4 b;
#pragma unroll
      for (int e = 0; e < 4; ++e) b[e] = sm.Tm[(16 * bk + 4 * g4 + e) * CP + 16 * bj + l16];
      return b;
    };
    auto t_aop = [&](int bi) {  // diagonal T block (bi, bi) as A operand
      return *(const f16x4 *)&sm.Tm[(16 * bi + l16) * CP + 16 * bi + 4 * g4];
    };
    auto finish_block = [&](int bi, int bj, f32x4 y) {
      const f16x4 yb = {h(y[0]), h(y[1]), h(y[2]), h(y[3])};
      f32x4 z = mma16(t_aop(bi), yb, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int e = 0; e < 4; ++e) sm.Tm[(16 * bi + 4 * g4 + e) * CP + 16 * bj + l16] = h(-z[e]);
    };
#pragma unroll
    for (int dist = 1; dist < 4; ++dist) {
      if (wave < 4 - dist) {
        const int bj = wave, bi = wave + dist;
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        for (int bk = bj; bk < bi; ++bk) y = mma16(a_op(bi, bk), t_bop(bk, bj), y);
        finish_block(bi, bj, y);
      }
      __syncthreads();
    }

    // ================= P5: K S^T, Q S^T; R = diag(beta)(V - K S^T) =================
    f32x4 O[2];
    {
      f32x4 KS[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      O[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      O[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const f16x8 ak = ld8(&sm.K[(16 * wave + l16) * KP + 32 * kk + 8 * g4]);
        const f16x8 aq = ld8(&sm.Q[(16 * wave + l16) * KP + 32 * kk + 8 * g4]);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const f16x8 b = ld8(&sm.S[(16 * n + l16) * KP + 32 * kk + 8 * g4]);
          KS[n] = mma32(ak, b, KS[n]);
          O[n] = mma32(aq, b, O[n]);
        }
      }
      const int t0 = 16 * wave + 4 * g4;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int j = 16 * n + l16;
        const ushort4 vv = *(const ushort4 *)&sm.VT[j * VP + t0];
        const float va[4] = {bf2f(vv.x), bf2f(vv.y), bf2f(vv.z), bf2f(vv.w)};
        f16x4 rr;
#pragma unroll
        for (int e = 0; e < 4; ++e) rr[e] = h(sm.beta[t0 + e] * (va[e] - KS[n][e]));
        *(f16x4 *)&sm.RT[j * CP + t0] = rr;
      }
    }
    __syncthreads();

    // ================= P6: X = Tinv R =================
    {
      const int nk = wave < 2 ? 1 : 2;
      f32x4 X[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      for (int kk = 0; kk < nk; ++kk) {
        const f16x8 a = ld8(&sm.Tm[(16 * wave + l16) * CP + 32 * kk + 8 * g4]);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const f16x8 b = ld8(&sm.RT[(16 * n + l16) * CP + 32 * kk + 8 * g4]);
          X[n] = mma32(a, b, X[n]);
        }
      }
      const int t0 = 16 * wave + 4 * g4;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int j = 16 * n + l16;
        const f16x4 xx = {h(X[n][0]), h(X[n][1]), h(X[n][2]), h(X[n][3])};
        *(f16x4 *)&sm.XT[j * CP + t0] = xx;
      }
    }
    __syncthreads();

    // ================= P7: O += P X, store o; S += ds Kt^T X =================
    {
      const int nk = wave < 2 ? 1 : 2;
      for (int kk = 0; kk < nk; ++kk) {
        const f16x8 a = ld8(&sm.P[(16 * wave + l16) * CP + 32 * kk + 8 * g4]);
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          const f16x8 b = ld8(&sm.XT[(16 * n + l16) * CP + 32 * kk + 8 * g4]);
          O[n] = mma32(a, b, O[n]);
        }
      }
      const int t0 = 16 * wave + 4 * g4;
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int j = j0 + 16 * n + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (t0 + e < L) o[(tok0 + c0 + t0 + e) * 128 + j] = (bf16)O[n][e];
      }
      // state update on this wave's i tiles
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int itile = 2 * wave + mi;
        f32x4 U[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const f16x8 a = ld8(&KtT[(16 * itile + l16) * CP + 32 * kk + 8 * g4]);
#pragma unroll
          for (int n = 0; n < 2; ++n) {
            const f16x8 b = ld8(&sm.XT[(16 * n + l16) * CP + 32 * kk + 8 * g4]);
            U[n] = mma32(a, b, U[n]);
          }
        }
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
          for (int e = 0; e < 4; ++e) Sacc[mi][n][e] = fmaf(ds, U[n][e], Sacc[mi][n][e]);
      }
      write_state_f16();
    }
  }

  // ================= outputs after the last chunk =================
  if (S_final) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const int i0 = 16 * (2 * wave + mi) + 4 * g4;
        const int j = 16 * n + l16;
        *(float4 *)(S_final + ((long)bh * 128 + j0 + j) * DK + i0) =
            float4{Sacc[mi][n][0], Sacc[mi][n][1], Sacc[mi][n][2], Sacc[mi][n][3]};
      }
  }
  __syncthreads();
  if (writer) {
    if (MODE == kOsdn && d_final && tid < DK) d_final[(long)bh * DK + tid] = sm.d[dcur][tid];
    if (MODE != kGiven && log_ratio_sum && tid == 0) log_ratio_sum[bh] = lr_sum;
  }
}

template <int MODE>
hipError_t launch_mode(const FusedArgs &a, const void *kt, hipStream_t s) {
  const int BH = a.B * a.H;
  const dim3 grid((unsigned)(BH * (128 / DVT))), block(NTH);
  const size_t shm = sizeof(Smem);
  hipError_t e = hipFuncSetAttribute((const void *)osdn_fused_forward<MODE>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(osdn_fused_forward<MODE>, grid, block, shm, s, (const bf16 *)a.q,
                     (const bf16 *)a.k, (const bf16 *)kt, (const bf16 *)a.v, a.beta,
                     MODE == kOsdn ? a.r : nullptr, a.d0, a.S0, a.eta, BH, a.T, (bf16 *)a.o,
                     a.S_final, a.d_final, a.log_ratio_sum);
  return hipGetLastError();
}

}  // namespace

bool fused_supported(int dk, int dv, int chunk, int dtype) {
  return dtype == 0 && dk == DK && dv == 128 && chunk == C;
}

hipError_t launch_fused_forward(const FusedArgs &a, hipStream_t s) {
  if ((long)a.B * a.H == 0) return hipSuccess;
  return a.precond_off ? launch_mode<kDeltaNet>(a, nullptr, s) : launch_mode<kOsdn>(a, nullptr, s);
}

hipError_t launch_fused_chunk(const ChunkArgs &a, hipStream_t s) {
  if ((long)a.B * a.H == 0) return hipSuccess;
  FusedArgs f{a.q, a.k, a.v, a.beta, nullptr, nullptr, a.S0, 0.f, a.B, a.H, a.T, a.dk, a.dv,
              a.chunk, a.dtype, 0, a.o, a.S_final, nullptr, nullptr};
  return launch_mode<kGiven>(f, a.k_tilde, s);
}

}  // namespace osdn
