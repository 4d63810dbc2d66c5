// The preconditioner walk in three launches (bf16 keys, dk = 128, chunk 64).
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
//   walk_keys  chunk-parallel: d_t token by token from the chunk's entry value
//              and c (the recurrence itself, in fp32), writing kt_t = d_t (.) k_t
//              and, if asked, d_t
// The chunk-parallel pass of the forward (chunk_prep) runs the same in-chunk
// recurrence to form its write keys.
#include "device.h"
#include "launch.h"
#include "mfma.h"
#include "walk.h"

namespace osdn {

namespace {

constexpr int C = 64;
constexpr int DK = 128;
constexpr int KP = 136;  // padded row (halves) of [64][128] tiles in LDS
constexpr int FP = 68;   // padded row (floats) of [64][64] fp32 tiles in LDS

// ---------------------------------------------------------------------------
// walk_prep: one workgroup of 4 waves per (b, h, chunk).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
walk_prep(const bf16 *__restrict__ k, const float *__restrict__ beta, const float *__restrict__ r,
          float eta, int T_, int NC, int c0, int ncs, unsigned xf, unsigned char *__restrict__ wrec) {
  // The fp16 keys are needed only for the key gram; (I + M)^-1 reuses their space.
  __shared__ __align__(16) float F[C * FP];           // key gram G, then M (strictly lower)
  __shared__ __align__(16) unsigned char KM[C * KP * 2];  // fp16 keys, then (I + M)^-1 [64][FP]
  __shared__ float Yw[3][16][17];                     // per-wave staging of a block sum
  __shared__ float bs[C], al[C], nn[C], lg[C + 4];
  __shared__ float ss[C];  // 1 / ||k_t||^2 for unnormalised keys, else 1
  static_assert(C * KP * 2 >= C * FP * 4, "the inverse fits in the keys' space");
  f16 *Kh = (f16 *)KM;
  float *Mi = (float *)KM;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c16 = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / ncs, c = c0 + blockIdx.x % ncs;  // chunks c0 .. c0+ncs-1
  const long tok0 = (long)bh * T_ + (long)c * C;
  const int L = min(C, T_ - c * C);

  // loads: 1024 pieces of 8 keys, 4 per thread; rows past the end reread the
  // last row and are zeroed when staged
  uint4 rk[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = tid + 256 * u, t = min(p >> 4, L - 1);
    rk[u] = *(const uint4 *)(k + (tok0 + t) * DK + (p & 15) * 8);
  }
  const int tb = min(lane, L - 1);
  float pb = beta[tok0 + tb];
  float pr = r ? r[tok0 + tb] : 1.0f;
  if (xf & kGateLogits) {
    pb = sigmoid_gate(pb);
    pr = sigmoid_gate(pr);
  }

  // stage the stored keys (exact in fp16); n_t from the stored bf16 values (16
  // threads per token).  Unnormalised keys enter through the fp32 factor
  // 1 / n_t on p_t (the normalised key's p is p_t / n_t), never through fp16.
  const f16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = tid + 256 * u, t = p >> 4, i0 = (p & 15) * 8;
    const bool ok = t < L;
    *(f16x8 *)&Kh[t * KP + i0] = ok ? cvt8(rk[u]) : z8;
    const unsigned short *s = (const unsigned short *)&rk[u];
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = bf2f(s[e]);
      sq = fmaf(x, x, sq);
    }
    sq = group_sum<16>(ok ? sq : 0.f);
    if ((p & 15) == 0) {
      const float sc = (xf & kNormQK) ? (sq > 0.f ? 1.0f / sq : 0.f) : 1.0f;
      ss[t] = sc;
      nn[t] = sq * sc;  // ||k_t||^2 of the key the recurrence sees
    }
  }
  if (wave == 0) {
    bs[lane] = lane < L ? pb : 0.f;
    // lg[t] = sum_{m<t} log2 r_m, clamped so that r = 0 stays finite
    float incl = (r && lane < L) ? fmaxf(flog2(pr), -126.f) : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    lg[lane + 1] = incl;
    if (lane == 0) lg[0] = 0.f;
  }
  __syncthreads();

  if (tid < C) al[tid] = nn[tid] > 0.f ? eta * bs[tid] / nn[tid] : 0.f;
  // lower tiles of the key gram G = P P^T with P = k (.) k in fp16
  for (int job = wave; job < 10; job += 4) {
    int rt, ct;
    tri_tile(job, rt, ct);
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const f16x8 a = ld8(&Kh[(16 * rt + c16) * KP + 32 * kk + 8 * g]);
      const f16x8 b = ld8(&Kh[(16 * ct + c16) * KP + 32 * kk + 8 * g]);
      acc = mma32(a * a, b * b, acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) F[(16 * rt + 4 * g + e) * FP + 16 * ct + c16] = acc[e];
  }
  __syncthreads();

  // M in place: thread (row t, quarter q) scales columns 16q..16q+15, zero on
  // and above the diagonal; the blocks of (I + M)^-1 above the diagonal are zero
  {
    const int t = tid >> 2, q = tid & 3;
    const float bl = bs[t], lt = lg[t], ssl = ss[t];
    float row[16];
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      const float4 f4 = *(const float4 *)&F[t * FP + 16 * q + j];
      row[j] = f4.x, row[j + 1] = f4.y, row[j + 2] = f4.z, row[j + 3] = f4.w;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int s = 16 * q + j;
      row[j] = s < t ? bl * al[s] * fexp2(lt - lg[s + 1]) * (ssl * ss[s]) * row[j] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      *(float4 *)&F[t * FP + 16 * q + j] = float4{row[j], row[j + 1], row[j + 2], row[j + 3]};
      if (16 * q > t) *(float4 *)&Mi[t * FP + 16 * q + j] = float4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __syncthreads();

  // diagonal blocks of (I + M)^-1, block `wave`
  {
    const int b = wave;
    float x[4];
    tri16_inverse_quad(&F[(16 * b) * FP + 16 * b], FP, lane, x);
#pragma unroll
    for (int j = 0; j < 4; ++j) Mi[(16 * b + (lane & 3) + 4 * j) * FP + 16 * b + (lane >> 2)] = x[j];
  }
  __syncthreads();

  // off-diagonal blocks by distance, one wave per block on the fp32 matrix
  // cores: Y = sum_{k=j}^{i-1} M_ik Mi_kj, then Mi_ij = -Mi_ii Y (Y passes
  // through the wave's own LDS rows to become the second product's operand)
  {
    const int r16 = lane & 15, k4 = lane >> 4;
#pragma unroll
    for (int dist = 1; dist < 4; ++dist) {
      if (wave + dist < 4) {
        const int bj = wave, bi = wave + dist;
        f32x4 y = zero4();
        for (int bk = bj; bk < bi; ++bk)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            y = __builtin_amdgcn_mfma_f32_16x16x4f32(
                F[(16 * bi + r16) * FP + 16 * bk + 4 * kk + k4],
                Mi[(16 * bk + 4 * kk + k4) * FP + 16 * bj + r16], y, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) Yw[wave][4 * k4 + e][r16] = y[e];
        wave_lds_sync();
        f32x4 z = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          z = __builtin_amdgcn_mfma_f32_16x16x4f32(Mi[(16 * bi + r16) * FP + 16 * bi + 4 * kk + k4],
                                                   Yw[wave][4 * kk + k4][r16], z, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) Mi[(16 * bi + 4 * k4 + e) * FP + 16 * bj + r16] = -z[e];
      }
      __syncthreads();
    }
  }

  // the record
  unsigned char *rec = wrec + ((long)bh * NC + c) * WREC;
  float4 *dst = (float4 *)(rec + W_MINV);
  for (int idx = tid; idx < C * C / 4; idx += 256)
    dst[idx] = *(const float4 *)&Mi[(idx >> 4) * FP + (idx & 15) * 4];
  if (tid < C) {
    const int t = tid;
    ((float *)(rec + W_U))[t] = bs[t] * fexp2(lg[t]);
    ((float *)(rec + W_A))[t] = al[t];
    ((float *)(rec + W_WA))[t] = t < L ? fexp2(lg[C] - lg[t + 1]) * al[t] : 0.f;
    ((float *)(rec + W_S))[t] = ss[t];
  }
  if (tid == 0) *(float *)(rec + W_GL) = fexp2(lg[C]);
}

// ---------------------------------------------------------------------------
// walk: one workgroup of 4 waves per (b, h), sequential over chunks c0..c1-1
// (the entry d of chunk c0 is d0, or what the launch before left in wout),
// three barriers per chunk:
//   A  b_t = <d, p_t> (4 threads per token), rhs_t = 1 - beta_t Gamma_t b_t
//   B  g = (I + M)^-1 rhs (4 threads per token); c_t, w_t = R_{L,t} alpha_t g_t
//   C  threads 0-127: d <- Gamma_L d + sum_t w_t p_t, one dimension each (kept
//      in a register); threads 128-255: log rho_t, and the LDS stores of the
//      next chunk, whose keys and record they load two chunks ahead (two
//      register sets), so the loads have two iterations to arrive
// ---------------------------------------------------------------------------
struct alignas(16) WalkSmem {
  bf16 K[2][C * KP];         // keys
  float Mi[2][C * FP];       // (I + M)^-1
  float vec[2][4][C];        // u = beta Gamma, alpha, R_{L,t} alpha, the 1/||k||^2 factor
  float gL[2][4];            // Gamma_L
  float d[DK];               // entry d of the chunk in the pass
  float rhs[C], w[C], g[C];
  float red[4];
};

__global__ void __launch_bounds__(256)
walk(const bf16 *__restrict__ k, const unsigned char *__restrict__ wrec,
     const float *__restrict__ d0, int T_, int NC, int c0, int c1, float *__restrict__ wout,
     float *__restrict__ d_final, float *__restrict__ log_ratio,
     float *__restrict__ log_ratio_sum) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  WalkSmem &sm = *reinterpret_cast<WalkSmem *>(smem_raw);
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int t = tid >> 2, part = tid & 3;  // phases A and B
  const bool owner = tid < DK;             // phase C: dimension tid
  const int lt = tid - DK;                 // loader index (threads 128-255)

  // loads of one chunk by threads 128-255: 1024 pieces of 8 keys, 8 each; the
  // record as 1089 pieces of 16 bytes (1024 of the inverse, 64 of vectors,
  // Gamma_L), 9 each
  constexpr int RP = (W_GL + 16) / 16;
  constexpr int NRP = (RP + 127) / 128;
  struct Regs {
    uint4 k[8], rr[NRP];
    int L;
  };
  Regs ra, rb;
  auto load = [&](Regs &R, int cc) {
    cc = min(cc, c1 - 1);
    const long t0 = (long)bh * T_ + (long)cc * C;
    const int L = min(C, T_ - cc * C);
    R.L = L;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = lt + 128 * u, tt = min(p >> 4, L - 1);
      R.k[u] = *(const uint4 *)(k + (t0 + tt) * DK + (p & 15) * 8);
    }
    const uint4 *rs = (const uint4 *)(wrec + ((long)bh * NC + cc) * WREC);
#pragma unroll
    for (int u = 0; u < NRP; ++u) R.rr[u] = rs[min(lt + 128 * u, RP - 1)];
  };
  auto stash = [&](const Regs &R, int buf) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = lt + 128 * u, tt = p >> 4, i0 = (p & 15) * 8;
      *(uint4 *)&sm.K[buf][tt * KP + i0] = tt < R.L ? R.k[u] : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < NRP; ++u) {
      const int p = lt + 128 * u;
      if (p < C * C / 4) {
        *(uint4 *)&sm.Mi[buf][(p >> 4) * FP + (p & 15) * 4] = R.rr[u];
      } else if (p < RP - 1) {
        const int v = p - C * C / 4;  // 16 pieces per vector
        *(uint4 *)&sm.vec[buf][v >> 4][(v & 15) * 4] = R.rr[u];
      } else if (p == RP - 1) {
        *(uint4 *)&sm.gL[buf][0] = R.rr[u];
      }
    }
  };

  float dreg = 0.f;  // owners: d of their dimension, entry value of the chunk in the pass
  if (owner) {
    if (c0 == 0) {
      dreg = d0 ? d0[(long)bh * DK + tid] : 1.0f;
      if (NC > 0) wout[(long)bh * NC * WOUT + tid] = dreg;
    } else {
      dreg = wout[((long)bh * NC + c0) * WOUT + tid];
    }
    sm.d[tid] = dreg;
  } else if (c1 > c0) {
    load(ra, c0);
    load(rb, c0 + 1);
    stash(ra, c0 & 1);
  }
  float lr_acc = 0.f;  // sum of log rho_t (threads 128-191)
  __syncthreads();

  auto iteration = [&](int c, Regs &next, Regs &free_) {
    const int cb = c & 1;
    const long t0 = (long)bh * T_ + (long)c * C;
    const int L = min(C, T_ - c * C);
    if (!owner) load(free_, c + 2);
    // A
    {
      const bf16 *kr = &sm.K[cb][t * KP + 32 * part];
      float b0 = 0.f, b1 = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 kv = *(const uint4 *)(kr + 8 * j);
        const unsigned short *sv = (const unsigned short *)&kv;
        const int i0 = 32 * part + 8 * j;
        const float4 p0 = *(const float4 *)&sm.d[i0], p1 = *(const float4 *)&sm.d[i0 + 4];
        const float dv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const float x0 = bf2f(sv[e]), x1 = bf2f(sv[e + 1]);
          b0 = fmaf(dv[e], x0 * x0, b0);
          b1 = fmaf(dv[e + 1], x1 * x1, b1);
        }
      }
      const float b = group_sum<4>(b0 + b1);
      if (part == 0) sm.rhs[t] = 1.0f - sm.vec[cb][0][t] * (sm.vec[cb][3][t] * b);
    }
    __syncthreads();
    // B
    {
      const float *mrow = &sm.Mi[cb][t * FP + 16 * part];
      const float *rv = &sm.rhs[16 * part];
      float ga = 0.f, gb = 0.f;
#pragma unroll
      for (int j = 0; j < 16; j += 4) {
        const float4 m4 = *(const float4 *)(mrow + j), r4 = *(const float4 *)(rv + j);
        ga = fmaf(m4.x, r4.x, ga);
        gb = fmaf(m4.y, r4.y, gb);
        ga = fmaf(m4.z, r4.z, ga);
        gb = fmaf(m4.w, r4.w, gb);
      }
      const float gt = group_sum<4>(ga + gb);
      if (part == 0) {
        sm.w[t] = sm.vec[cb][2][t] * gt * sm.vec[cb][3][t];
        sm.g[t] = gt;
        wout[((long)bh * NC + c) * WOUT + DK + t] = sm.vec[cb][1][t] * gt;
      }
    }
    __syncthreads();
    // C
    if (owner) {
      // every read issued before the sum (the scheduling barrier keeps them there)
      bf16 kx[C];
      float4 wv[C / 4];
#pragma unroll
      for (int s = 0; s < C; ++s) kx[s] = sm.K[cb][s * KP + tid];
#pragma unroll
      for (int j = 0; j < C / 4; ++j) wv[j] = *(const float4 *)&sm.w[4 * j];
      const float gl = sm.gL[cb][0];
      __builtin_amdgcn_sched_barrier(0);
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int j = 0; j < C / 4; ++j) {
        const float x0 = (float)kx[4 * j], x1 = (float)kx[4 * j + 1];
        const float x2 = (float)kx[4 * j + 2], x3 = (float)kx[4 * j + 3];
        a0 = fmaf(wv[j].x, x0 * x0, a0);
        a1 = fmaf(wv[j].y, x1 * x1, a1);
        a0 = fmaf(wv[j].z, x2 * x2, a0);
        a1 = fmaf(wv[j].w, x3 * x3, a1);
      }
      dreg = fmaf(gl, dreg, a0 + a1);
      sm.d[tid] = dreg;
      if (c + 1 < NC) wout[((long)bh * NC + c + 1) * WOUT + tid] = dreg;  // next entry d
    } else {
      if (lt < C && lt < L) {
        const float gt = sm.g[lt];
        const float lr = logf(gt * gt);  // log rho_t
        lr_acc += lr;
        if (log_ratio) log_ratio[t0 + lt] = lr;
      }
      if (c + 1 < c1) stash(next, cb ^ 1);
    }
    __syncthreads();
  };
  for (int c = c0; c < c1; c += 2) {
    iteration(c, rb, ra);
    if (c + 1 < c1) iteration(c + 1, ra, rb);
  }

  if (d_final && owner && c1 == NC) d_final[(long)bh * DK + tid] = dreg;
  if (log_ratio_sum) {
    // this launch's chunks, added to the sums of the launches before it
    const float s = wave_sum(lr_acc);
    if ((tid & 63) == 0) sm.red[tid >> 6] = s;
    __syncthreads();
    if (tid == 0) {
      const float part = (sm.red[0] + sm.red[1]) + (sm.red[2] + sm.red[3]);
      log_ratio_sum[bh] = c0 == 0 ? part : log_ratio_sum[bh] + part;
    }
  }
}

// ---------------------------------------------------------------------------
// walk_keys: one workgroup per (b, h, chunk).  Threads 0-127 run the in-chunk
// recurrence for one key dimension each; then all threads store kt rows with
// 16-byte stores.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
walk_keys(const bf16 *__restrict__ k, const float *__restrict__ r,
          const float *__restrict__ wout, int T_, int NC, bf16 *__restrict__ k_tilde,
          float *__restrict__ d_all) {
  __shared__ __align__(16) bf16 Kb[C * KP];
  __shared__ __align__(16) bf16 Kt[C * KP];
  __shared__ float cs[C], rs[C];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / NC, c = blockIdx.x % NC;
  const long tok0 = (long)bh * T_ + (long)c * C;
  const int L = min(C, T_ - c * C);
  const float *wo = wout + ((long)bh * NC + c) * WOUT;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = tid + 256 * u, t = p >> 4, i0 = (p & 15) * 8;
    const uint4 kv = *(const uint4 *)(k + (tok0 + min(t, L - 1)) * DK + i0);
    *(uint4 *)&Kb[t * KP + i0] = t < L ? kv : uint4{0, 0, 0, 0};
  }
  if (tid < C) {
    const int tb = min(tid, L - 1);
    const float cv = wo[DK + tid], rv = r ? r[tok0 + tb] : 1.0f;
    cs[tid] = tid < L ? cv : 0.f;
    rs[tid] = (r && tid < L) ? rv : 1.0f;
  }
  __syncthreads();
  if (tid < DK) {
    const int i = tid;
    float d = wo[i];
    for (int t0 = 0; t0 < C; t0 += 4) {
      const float4 c4 = *(const float4 *)&cs[t0], r4 = *(const float4 *)&rs[t0];
      const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, rv[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + e;
        const float kv = (float)Kb[t * KP + i];
        Kt[t * KP + i] = (bf16)(d * kv);
        if (d_all && t < L) d_all[(tok0 + t) * DK + i] = d;
        d = fmaf(cv[e], kv * kv, rv[e] * d);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = tid + 256 * u, t = p >> 4, i0 = (p & 15) * 8;
    if (t < L) *(uint4 *)(k_tilde + (tok0 + t) * DK + i0) = *(const uint4 *)&Kt[t * KP + i0];
  }
}

}  // namespace

bool walk_supported(int dk, int dtype) { return dk == DK && dtype == 0; }

size_t walk_workspace_bytes(int B, int H, int T) {
  const size_t nc = (size_t)((T + C - 1) / C);
  return (size_t)B * H * nc * (WREC + WOUT * sizeof(float));
}

hipError_t launch_walk_prep(const ScanArgs &a, int c0, int c1, unsigned char *wrec,
                            hipStream_t s) {
  const int BH = a.B * a.H;
  const int NC = (a.T + C - 1) / C;
  if (BH == 0 || c1 <= c0) return hipSuccess;
  hipLaunchKernelGGL(walk_prep, dim3((unsigned)(BH * (c1 - c0))), dim3(256), 0, s,
                     (const bf16 *)a.k, a.beta, a.r, a.eta, a.T, NC, c0, c1 - c0, a.xf, wrec);
  return hipGetLastError();
}

hipError_t launch_walk_pass(const ScanArgs &a, int c0, int c1, const unsigned char *wrec,
                            float *wout, hipStream_t s) {
  const int BH = a.B * a.H;
  const int NC = (a.T + C - 1) / C;
  if (BH == 0) return hipSuccess;
  constexpr size_t shm = sizeof(WalkSmem);
  hipError_t e = hipFuncSetAttribute((const void *)walk,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(walk, dim3((unsigned)BH), dim3(256), shm, s, (const bf16 *)a.k,
                     wrec, a.d0, a.T, NC, c0, c1, wout, a.d_final, a.log_ratio, a.log_ratio_sum);
  return hipGetLastError();
}

hipError_t launch_walk(const ScanArgs &a, unsigned char *wrec, float *wout, hipStream_t s) {
  const int NC = (a.T + C - 1) / C;
  hipError_t e = launch_walk_prep(a, 0, NC, wrec, s);
  if (e != hipSuccess) return e;
  return launch_walk_pass(a, 0, NC, wrec, wout, s);
}

hipError_t launch_walk_scan(const ScanArgs &a, void *ws, hipStream_t s) {
  const int BH = a.B * a.H;
  const int NC = (a.T + C - 1) / C;
  if (BH == 0) return hipSuccess;
  unsigned char *wrec = (unsigned char *)ws;
  float *wout = (float *)(wrec + (size_t)BH * NC * WREC);
  hipError_t e = launch_walk(a, wrec, wout, s);
  if (e != hipSuccess || NC == 0) return e;
  hipLaunchKernelGGL(walk_keys, dim3((unsigned)(BH * NC)), dim3(256), 0, s, (const bf16 *)a.k,
                     a.r, (const float *)wout, a.T, NC, (bf16 *)a.k_tilde, a.d_all);
  return hipGetLastError();
}

}  // namespace osdn
