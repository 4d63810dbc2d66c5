// Fused OSDN forward on CDNA4 matrix cores: chunk length 64, dk = dv = 128,
// bf16 q/k/v/o in HBM, fp16 matrix-core operands with fp32 accumulation,
// fp32 state and preconditioner.
//
// Source: gist.science technical summary of "OSDN: Improving Delta Rule with
// Provable Online Preconditioning in Linear Attention" -- §2.1 (the write key
// kt = d (.) k replaces k in the chunk gram, the intra-chunk scores and the
// state update), §2.2 (closed-form surrogate depending on k and beta only, so
// the preconditioner walk runs ahead of the state pass), §2.3 (APF retention
// acts on d only; the d recurrence stays affine), §3 (token-local residual
// ratio rho_t = (1 - beta_t a_t)^2).
//
// Organisation.  One workgroup of 8 waves per (b, h, 32-wide tile of value
// channels).  Waves 0-5 ("prep") prepare chunk c+1 while waves 6-7 ("state")
// run the state pass of chunk c, each on 16 value channels, and take a share
// of the prep work in the phases where the state pass has nothing to do.
// Only the prep waves read HBM; everything passed from prep to state is
// double-buffered in LDS.  Every wave meets the same 9 workgroup barriers per
// chunk, so no wave ever spins.
//
// Prep of a chunk (entry preconditioner d0, p_t = k_t (.) k_t):
//   stats      n_t = ||k_t||^2, b_t = <d0, p_t>, alpha_t = eta beta_t / n_t (0 if n_t = 0)
//   G = P P^T  (matrix cores); M_{t,s} = beta_t alpha_s R_{t,s} G_{t,s} for s < t,
//              R_{t,s} = prod_{s<m<t} r_m, Gamma_t = prod_{m<t} r_m
//   walk       (I + M) g = 1 - beta (.) Gamma (.) b, by 16x16 blocks; c = alpha (.) g.
//              g_t = 1 - beta_t a_t with a_t = <d_t, p_t>, so log rho_t = log g_t^2
//   write keys d_t = Gamma_t d0 + sum_{s<t} R_{t,s} c_s p_s (matrix cores);
//              kt = d (.) k / ds, ds a power of two >= max(d0) (exact rescaling)
//   next d     Gamma_L d0 + sum_s R_{L,s} c_s p_s in fp32
//   grams      A = strict_lower(diag(beta) K Kt^T) ds, P = lower(Q Kt^T) ds
//   Tinv       (I + A)^-1: fp32 16x16 diagonal blocks, then off-diagonal blocks
//              T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj by distance from the diagonal
// State pass of a chunk (entry state S, fp32 master S^T in registers):
//   R = diag(beta)(V - K S^T), X = Tinv R, O = Q S^T + P X, S^T += ds Kt^T X
// K S^T and Q S^T of a chunk are formed at the end of the iteration that
// prepared it, from the prep copies of K and Q, right after the state update
// of the chunk before it.
//
// Iteration schedule (prep of chunk c+1 | state pass of chunk c):
//   1  stage k, q, v, beta, r; entry d          | R = diag(beta)(V - K S^T)
//   2  stats, log-gate prefix, ds, key gram G    | X = Tinv R; values of c+1 -> registers
//   3  M blocks, diagonal inverses, rhs; loads   | O = Q S^T + P X, store o
//   4  substitution (wave 0) | R factors         | S^T update
//   5  write keys, 6 i tiles; next d partials    | write keys, 2 i tiles
//   6  diagonal A blocks + inverses; off-diag A  | score tiles P
//   7-9 off-diagonal blocks of Tinv              | K S^T, Q S^T of chunk c+1
//
// Layout trick: in a 16x16 MFMA result a lane holds 4 consecutive rows of one
// column; a 16x16x32 operand whose 32 k slots are rows 4g..4g+3 of two
// consecutive 16-row tiles has exactly that shape.  Contraction order is
// free, so results feed the next product from registers, with the partner
// operand read in the same "paired" k order.  Transposes are products with
// the identity (exact with fp32 accumulation).
#include "device.h"
#include "launch.h"
#include "mfma.h"

namespace osdn {

namespace {


constexpr int C = 64;       // chunk length
constexpr int DK = 128;     // key dimension (= value dimension)
constexpr int DVT = 32;     // value channels per workgroup
constexpr int NTH = 512;    // threads per workgroup
constexpr int NPREP = 6;    // prep waves
constexpr int PTH = NPREP * 64;
constexpr int KP = 136;     // padded row (halves) of [C][DK] tiles
constexpr int CP = 72;      // padded row (halves) of [C][C] tiles
constexpr int AP = 68;      // padded row (floats) of the fp32 [C][C] scratch

// kOsdn: the whole forward; kDeltaNet: the same with kt = k; kGiven: the
// chunkwise pass with kt read from memory; kScan: the preconditioner walk
// alone, writing kt (and optionally d_t and log rho_t) to memory.
enum Mode { kOsdn = 0, kDeltaNet = 1, kGiven = 2, kScan = 3 };
constexpr bool walk_mode(int m) { return m == kOsdn || m == kScan; }

struct Smem {
  f16 Kp[C * KP];           // keys of the chunk being prepared [t][i]
  f16 Qp[C * KP];           // queries [t][i]
  f16 Kt[C * KP];           // scaled write keys [t][i] (gram operand); before them,
                            // the chunk's value tile [t][j < 32] passes through here
  f16 KtF[2][8][2][64][8];  // write keys as S-update operands [buf][i tile][t pair][lane][8]
  f16 Tm[2][C * CP];        // (I + A)^-1 [buf][t][s]; the walk's R factors occupy the
                            // buffer being prepared until the inverse overwrites them
  f16 P[2][C * CP];         // scores lower(Q Kt^T) ds [buf][t][s]
  float F[C * AP];          // fp32 scratch: key gram -> M, then the gram A
  float Td[4][16][16];      // the walk's 16x16 diagonal-block inverses
  float d_in[DK];           // entry preconditioner of the chunk being prepared
  float dpart[4][DK];       // partial sums of the next entry preconditioner
  float beta[2][C];         // write gates [buf][t]
  float dsb[4];             // write-key scale [buf] (padded to keep 16-byte alignment)
  float r[C], n[C], bv[C], alpha[C], g[C], cc[C], w[C], rhs[C], acc[C];
  float lg[C + 4];          // lg[t] = sum_{m<t} log2 r_m
  float al[C];              // state gates of the chunk being prepared
  float lga[2][C + 4];      // [buf] lga[t] = sum_{m<=t} log2 alpha_m (state gate)
  float lgC;                // lg[L] of the chunk prepared last
  float red[15];
};
static_assert(sizeof(Smem) <= 160 * 1024, "LDS budget of one workgroup");
static_assert(offsetof(Smem, lga) % 16 == 0, "16-byte reads of the gate prefix");

// The kernel body.  Every LDS array comes in through its own restrict
// pointer, which tells the compiler that a store to one array cannot change
// another, so loads can be issued ahead of unrelated stores.
template <int MODE, bool GATED>
__device__ __forceinline__ void fused_body(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                   const bf16 *__restrict__ kt_in, const bf16 *__restrict__ v,
                   const float *__restrict__ beta, const float *__restrict__ r,
                   const float *__restrict__ alpha,
                   const float *__restrict__ d0, const float *__restrict__ S0, float eta,
                   int BH, int T_, bf16 *__restrict__ o, float *__restrict__ S_final,
                   float *__restrict__ d_final, float *__restrict__ log_ratio_sum, bf16 *__restrict__ kt_out,
    float *__restrict__ d_all, float *__restrict__ log_ratio,
    f16 *__restrict__ LKp, f16 *__restrict__ LQp, f16 *__restrict__ LKt,
           f16 (*__restrict__ LKtF)[8][2][64][8], f16 (*__restrict__ LTm)[C * CP],
           f16 (*__restrict__ LP)[C * CP], float *__restrict__ LF,
           float (*__restrict__ LTd)[16][16], float *__restrict__ Ld_in,
           float (*__restrict__ Ldpart)[DK], float (*__restrict__ Lbeta)[C],
           float *__restrict__ Ldsb, float *__restrict__ Lr, float *__restrict__ Ln,
           float *__restrict__ Lbv, float *__restrict__ Lalpha, float *__restrict__ Lg,
           float *__restrict__ Lcc, float *__restrict__ Lw, float *__restrict__ Lrhs,
           float *__restrict__ Lacc, float *__restrict__ Llg, float *__restrict__ LlgC,
           float *__restrict__ Lred, float *__restrict__ Lal,
           float (*__restrict__ Llga)[C + 4]) {
  constexpr int NTILE = MODE == kScan ? 1 : 128 / DVT;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform role
  // Lane coordinates.  They are re-derived from an opaque copy of the thread
  // index at the top of every chunk iteration, so that the compiler recomputes
  // the many lane-dependent LDS addresses and masks of an iteration instead of
  // hoisting them all out of the loop and running out of registers.
  int lane = tid & 63, c16 = lane & 15, g = lane >> 4;
  auto refresh_lane = [&]() {
    int x = tid;
    asm volatile("" : "+v"(x));
    lane = x & 63;
    c16 = lane & 15;
    g = lane >> 4;
  };

  // Workgroup -> (head, value tile); consecutive workgroup ids go to different
  // XCDs, so the tiles of one head are kept on one XCD to share its L2.
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
  const int nch = (T_ + C - 1) / C;
  const bool writer = tile == 0;  // writes the per-head outputs (d, log-ratio sum)

  // identity as a 16x16x16 operand: lane (col c16, k 4g+e)
  f16x4 ident;
  bf16x4 identb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ident[e] = (4 * g + e == c16) ? (f16)1.0f : (f16)0.0f;
    identb[e] = (4 * g + e == c16) ? (bf16)1.0f : (bf16)0.0f;
  }

  // State-gate decays gamma_t / gamma_s = 2^(lga_t - lga_s) of buffer nb for
  // rows t0..t0+3 and column s (only taken for s <= t, where they are <= 1).
  auto gate_decay = [&](int nb, int t0, int s) {
    const float4 lt = *(const float4 *)&Llga[nb][t0];
    const float ls = Llga[nb][s];
    return f32x4{fexp2(lt.x - ls), fexp2(lt.y - ls), fexp2(lt.z - ls), fexp2(lt.w - ls)};
  };

  // ------------- prep work any wave can take (chunk in buffer nb) -------------
  // Write keys of i tile n (OSDN): D = Gamma d0 + R (c (.) P), kt = D (.) k / ds,
  // stored as S-update operands (KtF) and row-major (Kt).
  auto write_keys_itile = [&](int n, int nb) {
    // every LDS operand first, then the products, then the stores
    const float inv = 1.0f / Ldsb[nb];
    const float dbase = Ld_in[16 * n + c16];
    f16x4 kin[4];
    float4 c4[4], l4[4];
    f16x8 rrow[6];  // R rows of block m for t pairs 0..m/2
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kin[j] = ld4(&LKp[(16 * j + c16) * KP + 16 * n + 4 * g]);
      c4[j] = *(const float4 *)&Lcc[16 * j + 4 * g];
      l4[j] = *(const float4 *)&Llg[16 * j + 4 * g];
    }
#pragma unroll
    for (int m = 0, x = 0; m < 4; ++m)
#pragma unroll
      for (int qq = 0; qq <= (m >> 1); ++qq, ++x)
        rrow[x] = ldpk(&LTm[nb][(16 * m + c16) * CP], 32 * qq, g);
    f32x4 kT[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kT[j] = mma16(kin[j], ident, zero4());
    f16x8 cP[2];
    {
      f16x4 cpj[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float cv[4] = {c4[j].x, c4[j].y, c4[j].z, c4[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) cpj[j][e] = h(kT[j][e] * kT[j][e] * cv[e]);
      }
      cP[0] = cat(cpj[0], cpj[1]);
      cP[1] = cat(cpj[2], cpj[3]);
    }
    f16x4 kt4[4], kr4[4];
#pragma unroll
    for (int m = 0, x = 0; m < 4; ++m) {
      f32x4 acc = {fexp2(l4[m].x) * dbase, fexp2(l4[m].y) * dbase, fexp2(l4[m].z) * dbase,
                   fexp2(l4[m].w) * dbase};
#pragma unroll
      for (int qq = 0; qq <= (m >> 1); ++qq, ++x) acc = mma32(rrow[x], cP[qq], acc);
      f32x4 ktv;
#pragma unroll
      for (int e = 0; e < 4; ++e) ktv[e] = acc[e] * kT[m][e] * inv;
      kt4[m] = h4(ktv);
      kr4[m] = h4(mma16(kt4[m], ident, zero4()));
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      *(f16x4 *)&LKtF[nb][n][m >> 1][lane][4 * (m & 1)] = kt4[m];
      *(f16x4 *)&LKt[(16 * m + c16) * KP + 16 * n + 4 * g] = kr4[m];
    }
  };
  // Write keys held row-major in `src` (the keys, or given write keys):
  // 16x16 tile (m, n) transposed through the identity into the S-update operand.
  auto write_keys_copy = [&](int job, const f16 *src, int nb) {
    const int m = job >> 3, n = job & 7;
    const f32x4 tr = mma16(ld4(&src[(16 * m + c16) * KP + 16 * n + 4 * g]), ident, zero4());
    *(f16x4 *)&LKtF[nb][n][m >> 1][lane][4 * (m & 1)] = h4(tr);
  };
  // Lower tile idx of the scores P = lower(Q Kt^T) ds.
  auto score_tile = [&](int idx, const f16 *Bsrc, int nb) {
    int rt, ct;
    tri_tile(idx, rt, ct);
    const float ds = Ldsb[nb];
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc = mma32(ld8(&LQp[(16 * rt + c16) * KP + 32 * kk + 8 * g]),
                  ld8(&Bsrc[(16 * ct + c16) * KP + 32 * kk + 8 * g]), acc);
    f32x4 dec = {1.f, 1.f, 1.f, 1.f};
    if (GATED) dec = gate_decay(nb, 16 * rt + 4 * g, 16 * ct + c16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + 4 * g + e, col = 16 * ct + c16;
      LP[nb][row * CP + col] = h(col <= row ? ds * dec[e] * acc[e] : 0.f);
    }
  };

  // R_{t,s} = 2^(lg_t - lg_{s+1}) (s < t) for the write keys, into the inverse
  // buffer being prepared: rows t = r0 + 4u and r0 + 1 + 4u, thread x (0..127)
  // keeping column x & 63 of one of the two row sets.
  auto r_factor_rows = [&](int x, int r0, int nb) {
    f16 *R16 = LTm[nb];
    const int s = x & 63, t0 = r0 + (x >> 6);
    const float lgs = Llg[s + 1];
    float lgt[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) lgt[u] = Llg[t0 + 4 * u];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int t = t0 + 4 * u;
      R16[t * CP + s] = h(s < t ? fexp2(lgt[u] - lgs) : 0.f);
    }
  };
  // Lower tile `job` of the key gram G = P P^T (P = k (.) k in fp16), raw, into F.
  auto key_gram_tile = [&](int job) {
    int rt, ct;
    tri_tile(job, rt, ct);
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const f16x8 a = ld8(&LKp[(16 * rt + c16) * KP + 32 * kk + 8 * g]);
      const f16x8 b = ld8(&LKp[(16 * ct + c16) * KP + 32 * kk + 8 * g]);
      acc = mma32(a * a, b * b, acc);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) LF[(16 * rt + 4 * g + e) * AP + 16 * ct + c16] = acc[e];
  };
  // Off-diagonal tile `job` of A = strict_lower(diag(beta) K Kt^T) ds, into F.
  auto gram_a_off_tile = [&](int job, const f16 *Bsrc, int nb) {
    int rt, ct;
    off_tile(job, rt, ct);
    const float ds = Ldsb[nb];
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc = mma32(ld8(&LKp[(16 * rt + c16) * KP + 32 * kk + 8 * g]),
                  ld8(&Bsrc[(16 * ct + c16) * KP + 32 * kk + 8 * g]), acc);
    f32x4 dec = {1.f, 1.f, 1.f, 1.f};
    if (GATED) dec = gate_decay(nb, 16 * rt + 4 * g, 16 * ct + c16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * rt + 4 * g + e, col = 16 * ct + c16;
      LF[row * AP + col] = Lbeta[nb][row] * ds * dec[e] * acc[e];
    }
  };

  // ---------------- initialisation ----------------
  for (int idx = tid; idx < C * CP; idx += NTH) {
    LP[0][idx] = (f16)0.0f;
    LP[1][idx] = (f16)0.0f;
    LTm[0][idx] = (f16)0.0f;
    LTm[1][idx] = (f16)0.0f;
  }
  for (int i = tid; i < DK; i += NTH)
    Ld_in[i] = (walk_mode(MODE) && d0) ? d0[(long)bh * DK + i] : 1.0f;
  if (tid == 0) (*LlgC) = 0.f;

  if (wave < NPREP) {
    // =====================================================================
    //                              prep waves
    // =====================================================================
    const int ptid = tid;
    uint4 pk[3], pq[3], pkt[3], pv;
    float pb = 0.f, pr = 1.f, pal = 1.f;
    float lr_sum = 0.f;  // wave 0: sum over tokens of log rho_t
    // Global loads of a chunk by all prep waves: k and q (and given write keys)
    // as 1024 pieces of 8 elements, the value tile as 256 pieces, beta and r.
    // The loads are unconditional -- rows past the end read the last row and
    // are zeroed when staged, and the chunk after the last reloads the last --
    // because a load under a condition makes the compiler wait for it where the
    // branches join, which would expose its latency.
    auto prep_load = [&](int cc_) {
      const int c0 = cc_ * C;
      const int L = min(C, T_ - c0);
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        const int p = min(ptid + PTH * u, 16 * C - 1);
        const int t = min(p >> 4, L - 1), piece = p & 15;
        const long off = (tok0 + c0 + t) * DK + piece * 8;
        pk[u] = *(const uint4 *)(k + off);
        if (MODE != kScan) pq[u] = *(const uint4 *)(q + off);
        if (MODE == kGiven) pkt[u] = *(const uint4 *)(kt_in + off);
      }
      if (MODE != kScan) {
        const int t = min((ptid & 255) >> 2, L - 1), piece = ptid & 3;
        pv = *(const uint4 *)(v + (tok0 + c0 + t) * 128 + j0 + piece * 8);
      }
      const int tb = min(ptid & 63, L - 1);
      pb = beta[tok0 + c0 + tb];
      pr = (r ? r : beta)[tok0 + c0 + tb];  // replaced by 1 when staged if r is absent
      if (GATED) pal = alpha[tok0 + c0 + tb];
    };
    if (nch > 0) prep_load(0);
    __syncthreads();

    for (int it = 0; nch > 0 && it <= nch; ++it) {
      refresh_lane();
      const int pc = it;  // chunk being prepared
      const int nb = pc & 1;
      const bool act = pc < nch;
      const int pL = act ? min(C, T_ - pc * C) : 0;

      // ------------------------------ phase 1 ------------------------------
      if (act) {
        if (wave == 0 && MODE == kOsdn && pc > 0) {
          // entry preconditioner: Gamma_L d of the previous chunk plus its sums
          const float gL = fexp2((*LlgC));
#pragma unroll
          for (int i = lane; i < DK; i += 64)
            Ld_in[i] = gL * Ld_in[i] + Ldpart[0][i] + Ldpart[1][i] + Ldpart[2][i] +
                       Ldpart[3][i];
        }
        {
          float kmax = 0.f;
          const f16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int u = 0; u < 3; ++u) {
            const int p = ptid + PTH * u;
            if (p < 16 * C) {
              const int t = p >> 4, i0 = (p & 15) * 8;
              const bool ok = t < pL;
              *(f16x8 *)&LKp[t * KP + i0] = ok ? cvt8(pk[u]) : z8;
              if (MODE != kScan) *(f16x8 *)&LQp[t * KP + i0] = ok ? cvt8(pq[u]) : z8;
              if (MODE == kGiven) {
                if (!ok) pkt[u] = uint4{0, 0, 0, 0};
                const unsigned short *ut = (const unsigned short *)&pkt[u];
#pragma unroll
                for (int e = 0; e < 8; ++e) kmax = fmaxf(kmax, fabsf(bf2f(ut[e])));
              }
            }
          }
          if (MODE != kScan && ptid < 4 * C) {  // the value tile passes through Kt, in bf16
            const int t = ptid >> 2, j = (ptid & 3) * 8;
            *(uint4 *)&LKt[t * KP + j] = t < pL ? pv : uint4{0, 0, 0, 0};
          }
          if (ptid < C) {
            Lbeta[nb][ptid] = ptid < pL ? pb : 0.f;
            Lr[ptid] = (r && ptid < pL) ? pr : 1.f;
            if (GATED) Lal[ptid] = ptid < pL ? pal : 1.f;
          }
          if (MODE == kGiven) {
            kmax = wave_max(kmax);
            if (lane == 0) Lred[wave] = kmax;
          }
        }
      }
      __syncthreads();

      // ------------------------------ phase 2 ------------------------------
      if (GATED && act && wave == 4) {
        // lga[t] = sum_{m<=t} log2 alpha_m (clamped so that alpha = 0 stays finite)
        float incl = fmaxf(flog2(Lal[lane]), -126.f);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(incl, off);
          if (lane >= off) incl += y;
        }
        Llga[nb][lane] = incl;
      }
      if (act && MODE != kGiven) {
        if (wave < 4) {
          // token statistics: wave w owns tokens 16w..16w+15, lane quarter g 32 dims
          const int t = 16 * wave + c16;
          float pn = 0.f, pa = 0.f;
#pragma unroll
          for (int q8 = 0; q8 < 4; ++q8) {
            const int i0 = 32 * g + 8 * q8;
            const f16x8 kk = ld8(&LKp[t * KP + i0]);
            const float4 da = *(const float4 *)&Ld_in[i0];
            const float4 db = *(const float4 *)&Ld_in[i0 + 4];
            const float dd[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float x = (float)kk[e];
              const float p = x * x;
              pn += p;
              pa = fmaf(dd[e], p, pa);
            }
          }
          pn += __shfl_xor(pn, 16);
          pn += __shfl_xor(pn, 32);
          pa += __shfl_xor(pa, 16);
          pa += __shfl_xor(pa, 32);
          if (g == 0) {
            Ln[t] = pn;
            Lbv[t] = pa;
            Lalpha[t] = (walk_mode(MODE) && pn > 0.f) ? eta * Lbeta[nb][t] / pn : 0.f;
          }
        } else if (wave == 4) {
          if (walk_mode(MODE)) {
            // lg[t] = sum_{m<t} log2 r_m (clamped so that r = 0 stays finite)
            const float lr = fmaxf(flog2(Lr[lane]), -126.f);
            float incl = lr;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
              const float y = __shfl_up(incl, off);
              if (lane >= off) incl += y;
            }
            Llg[lane + 1] = incl;
            if (lane == 0) Llg[0] = 0.f;
          }
        } else {
          float dm = fmaxf(Ld_in[lane], Ld_in[lane + 64]);
#pragma unroll
          for (int m_ = 1; m_ < 64; m_ <<= 1) dm = fmaxf(dm, __shfl_xor(dm, m_));
          if (lane == 0)
            Ldsb[nb] = (MODE == kOsdn && dm > 0.f) ? fexp2(ceilf(flog2(dm))) : 1.0f;
        }
        if (walk_mode(MODE)) {
          // key gram tiles 0-7 (the state waves take 8 and 9)
          if (wave < 4) key_gram_tile(wave);
          else if (wave == 4) key_gram_tile(4);
          else {
            key_gram_tile(5);
            key_gram_tile(6);
            key_gram_tile(7);
          }
        }
      }
      __syncthreads();

      // ------------------------------ phase 3 ------------------------------
      if (act) {
        if (MODE == kGiven) {
          // given write keys, rescaled by a power of two into fp16 range
          float km = 0.f;
#pragma unroll
          for (int w_ = 0; w_ < NPREP; ++w_) km = fmaxf(km, Lred[w_]);
          const float ds = km > 0.f ? fexp2(ceilf(flog2(km))) : 1.0f;
          const float inv = 1.0f / ds;
          if (ptid == 0) Ldsb[nb] = ds;
#pragma unroll
          for (int u = 0; u < 3; ++u) {
            const int p = ptid + PTH * u;
            if (p < 16 * C) {
              const int t = p >> 4, i0 = (p & 15) * 8;
              const unsigned short *ut = (const unsigned short *)&pkt[u];
              f16x8 hv;
#pragma unroll
              for (int e = 0; e < 8; ++e) hv[e] = h(bf2f(ut[e]) * inv);
              *(f16x8 *)&LKt[t * KP + i0] = hv;
            }
          }
        } else if (walk_mode(MODE)) {
          if (wave < 4) {
            // diagonal block b of M, scaled in place (a lane keeps column s and
            // rows 16b + g + 4u), then its inverse
            const int b = wave, s = 16 * b + c16;
            const float as = Lalpha[s], ls = Llg[s + 1];
            float bt[4], lt[4], fv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int t = 16 * b + g + 4 * u;
              bt[u] = Lbeta[nb][t];
              lt[u] = Llg[t];
              fv[u] = LF[t * AP + s];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int t = 16 * b + g + 4 * u;
              LF[t * AP + s] = c16 < g + 4 * u ? bt[u] * as * fexp2(lt[u] - ls) * fv[u] : 0.f;
            }
            wave_lds_sync();
            float x[4];
            tri16_inverse_quad(&LF[(16 * b) * AP + 16 * b], AP, lane, x);
#pragma unroll
            for (int j = 0; j < 4; ++j) LTd[b][(lane & 3) + 4 * j][lane >> 2] = x[j];
          } else {
            // off-diagonal blocks of M: a thread keeps column sc of each tile and
            // rows r0, r0 + 8; and the rhs
            const int l2 = ptid - 256;  // 0..127
            const int sc = l2 & 15, r0 = l2 >> 4;
            float as[3], ls[3], bt[12], lt[12], fv[12];
#pragma unroll
            for (int ct = 0; ct < 3; ++ct) {
              as[ct] = Lalpha[16 * ct + sc];
              ls[ct] = Llg[16 * ct + sc + 1];
            }
#pragma unroll
            for (int u = 0; u < 12; ++u) {
              int rt, ct;
              off_tile(u >> 1, rt, ct);
              const int t = 16 * rt + r0 + 8 * (u & 1), s = 16 * ct + sc;
              bt[u] = Lbeta[nb][t];
              lt[u] = Llg[t];
              fv[u] = LF[t * AP + s];
            }
            float rb = 0.f, rl = 0.f, rv = 0.f;
            if (l2 < C) {
              rb = Lbeta[nb][l2];
              rl = Llg[l2];
              rv = Lbv[l2];
            }
#pragma unroll
            for (int u = 0; u < 12; ++u) {
              int rt, ct;
              off_tile(u >> 1, rt, ct);
              const int t = 16 * rt + r0 + 8 * (u & 1), s = 16 * ct + sc;
              LF[t * AP + s] = fv[u] * (bt[u] * as[ct] * fexp2(lt[u] - ls[ct]));
            }
            if (l2 < C) Lrhs[l2] = 1.0f - rb * fexp2(rl) * rv;
            if (MODE == kOsdn) r_factor_rows(l2, 0, nb);  // rows 4u, 4u + 1
          }
        }
      }
      __syncthreads();

      // ------------------------------ phase 4 ------------------------------
      if (act) {
        if (wave == 0) {
          if (walk_mode(MODE)) {
            // blocked forward substitution of (I + M) g = rhs, lanes = tokens;
            // the 16 values of a block reach every lane through lane reads
            const int t = lane, bt = t >> 4;
            float tdrow[16], mrow[3][16];
#pragma unroll
            for (int u = 0; u < 16; u += 4) {
              const float4 tv = *(const float4 *)&LTd[bt][t & 15][u];
              tdrow[u] = tv.x, tdrow[u + 1] = tv.y, tdrow[u + 2] = tv.z, tdrow[u + 3] = tv.w;
#pragma unroll
              for (int b = 0; b < 3; ++b) {
                const float4 mv = *(const float4 *)&LF[t * AP + 16 * b + u];
                mrow[b][u] = mv.x, mrow[b][u + 1] = mv.y, mrow[b][u + 2] = mv.z,
                mrow[b][u + 3] = mv.w;
              }
            }
            const float alpha_t = Lalpha[t], lg_next = Llg[t + 1], lg_end = Llg[pL];
            float a = Lrhs[t];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              float y0 = 0.f, y1 = 0.f;
#pragma unroll
              for (int j = 0; j < 16; j += 2) {
                y0 = fmaf(tdrow[j], readlane(a, 16 * b + j), y0);
                y1 = fmaf(tdrow[j + 1], readlane(a, 16 * b + j + 1), y1);
              }
              if (bt == b) a = y0 + y1;
              if (b < 3) {
                float z0 = 0.f, z1 = 0.f;
#pragma unroll
                for (int j = 0; j < 16; j += 2) {
                  z0 = fmaf(mrow[b][j], readlane(a, 16 * b + j), z0);
                  z1 = fmaf(mrow[b][j + 1], readlane(a, 16 * b + j + 1), z1);
                }
                if (bt > b) a -= z0 + z1;
              }
            }
            // a == g_t == 1 - beta_t a_t
            const float cct = alpha_t * a;
            Lcc[t] = cct;
            Lw[t] = t < pL ? fexp2(lg_end - lg_next) * cct : 0.f;
            if (lane == 0) (*LlgC) = lg_end;
            const float lrt = logf(a * a);  // log rho_t
            if (MODE == kScan && log_ratio && t < pL) log_ratio[tok0 + (long)pc * C + t] = lrt;
            lr_sum += wave_sum(t < pL ? lrt : 0.f);
          } else if (MODE == kDeltaNet) {
            const float gd = 1.0f - Lbeta[nb][lane] * Ln[lane];
            lr_sum += wave_sum(lane < pL ? logf(gd * gd) : 0.f);
          }
        }
      }
      __syncthreads();

      // ------------------------------ phase 5 ------------------------------
      // the next chunk's loads: at the start of the phase in the walk alone
      // (whose iteration ends here), else at its end
      if (MODE == kScan) prep_load(min(pc + 1, nch - 1));
      if (act) {
        if (MODE == kOsdn) {
          write_keys_itile(wave, nb);  // i tiles 0..5; the state waves take 6 and 7
          // next entry preconditioner: waves 0-3 sum quarters of the chunk, a
          // thread keeps two dimensions
          if (wave < 4) {
            const int i = 2 * lane, part = wave;
            float4 w4[4];
            typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
            f16x2 kx[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) kx[u] = *(const f16x2 *)&LKp[(16 * part + u) * KP + i];
#pragma unroll
            for (int u = 0; u < 4; ++u) w4[u] = *(const float4 *)&Lw[16 * part + 4 * u];
            float a0 = 0.f, a1 = 0.f;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
              const float ws = u % 4 == 0 ? w4[u / 4].x : u % 4 == 1 ? w4[u / 4].y
                             : u % 4 == 2 ? w4[u / 4].z : w4[u / 4].w;
              const float x0 = (float)kx[u][0], x1 = (float)kx[u][1];
              a0 = fmaf(ws, x0 * x0, a0);
              a1 = fmaf(ws, x1 * x1, a1);
            }
            Ldpart[part][i] = a0;
            Ldpart[part][i + 1] = a1;
          }
        } else if (MODE == kScan) {
          // d_t token by token from the walk's c_t, d_{t+1} = r_t d_t + c_t p_t,
          // a lane per dimension (waves 0-1): write keys kt_t = d_t (.) k_t and,
          // if asked, d_t itself; d after the chunk is the next entry value
          if (wave < 2) {
            const int i = wave * 64 + lane;
            float d = Ld_in[i];
            const long base = (tok0 + (long)pc * C) * DK + i;
#pragma unroll
            for (int t0 = 0; t0 < C; t0 += 4) {
              const float4 c4 = *(const float4 *)&Lcc[t0];
              const float4 r4 = *(const float4 *)&Lr[t0];
              const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, rv[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int t = t0 + e;
                if (t < pL) {
                  const float kv = (float)LKp[t * KP + i];
                  kt_out[base + (long)t * DK] = (bf16)(d * kv);
                  if (d_all) d_all[base + (long)t * DK] = d;
                  d = fmaf(cv[e], kv * kv, rv[e] * d);
                }
              }
            }
            Ld_in[i] = d;
          }
        } else {
          const f16 *src = (MODE == kDeltaNet) ? LKp : LKt;
          for (int job = wave; job < 32; job += 8) write_keys_copy(job, src, nb);
        }
      }
      if (MODE != kScan) prep_load(min(pc + 1, nch - 1));
      __syncthreads();

      // ------------------------------ phase 6 ------------------------------
      // (the walk alone ends with phase 5)
      if (MODE != kScan && act) {
        const float ds = Ldsb[nb];
        const f16 *Bsrc = (MODE == kDeltaNet) ? LKp : LKt;
        if (wave < 4) {
          // diagonal tile of A, then its inverse (a diagonal block of Tinv)
          const int b = wave;
          f32x4 acc = zero4();
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            acc = mma32(ld8(&LKp[(16 * b + c16) * KP + 32 * kk + 8 * g]),
                        ld8(&Bsrc[(16 * b + c16) * KP + 32 * kk + 8 * g]), acc);
          f32x4 dec = {1.f, 1.f, 1.f, 1.f};
          if (GATED) dec = gate_decay(nb, 16 * b + 4 * g, 16 * b + c16);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = 16 * b + 4 * g + e, col = 16 * b + c16;
            LF[row * AP + col] = col < row ? Lbeta[nb][row] * ds * dec[e] * acc[e] : 0.f;
          }
          wave_lds_sync();
          float x[4];
          tri16_inverse_quad(&LF[(16 * b) * AP + 16 * b], AP, lane, x);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            LTm[nb][(16 * b + (lane & 3) + 4 * j) * CP + 16 * b + (lane >> 2)] = h(x[j]);
        } else {
          // score tiles 0-3 (the state waves form the off-diagonal tiles of A)
          score_tile(2 * (wave - 4), Bsrc, nb);
          score_tile(2 * (wave - 4) + 1, Bsrc, nb);
        }
      }
      if (MODE != kScan) __syncthreads();

      // ----------------- phases 7-9: off-diagonal blocks of Tinv -----------------
      // T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, blocks at distance 1, 2, 3; the
      // waves a level leaves idle form score tiles 4-9
#pragma unroll
      for (int dist = 1; dist < (MODE == kScan ? 1 : 4); ++dist) {
        if (act && wave >= 4 - dist) {
          const f16 *Bsrc = (MODE == kDeltaNet) ? LKp : LKt;
          if (dist == 1) score_tile(1 + wave, Bsrc, nb);                  // waves 3-5
          if (dist == 2 && wave <= 4) score_tile(5 + wave, Bsrc, nb);     // waves 2-4
        }
        if (act && wave < 4 - dist) {
          const int bj = wave, bi = wave + dist;
          f16 *Tn = LTm[nb];
          f32x4 y = zero4();
          for (int bk = bj; bk < bi; ++bk) {
            f16x4 a, b;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              a[e] = h(LF[(16 * bi + c16) * AP + 16 * bk + 4 * g + e]);
              b[e] = Tn[(16 * bk + 4 * g + e) * CP + 16 * bj + c16];
            }
            y = mma16(a, b, y);
          }
          const f32x4 z = mma16(ld4(&Tn[(16 * bi + c16) * CP + 16 * bi + 4 * g]), h4(y), zero4());
#pragma unroll
          for (int e = 0; e < 4; ++e) Tn[(16 * bi + 4 * g + e) * CP + 16 * bj + c16] = h(-z[e]);
        }
        __syncthreads();
      }
    }

    if (writer) {
      if (MODE == kOsdn && d_final && ptid < DK) {
        const float dv = nch > 0 ? fexp2((*LlgC)) * Ld_in[ptid] + Ldpart[0][ptid] +
                                       Ldpart[1][ptid] + Ldpart[2][ptid] + Ldpart[3][ptid]
                                 : Ld_in[ptid];
        d_final[(long)bh * DK + ptid] = dv;
      }
      if (MODE == kScan && d_final && ptid < DK) d_final[(long)bh * DK + ptid] = Ld_in[ptid];
      if (MODE != kGiven && log_ratio_sum && ptid == 0) log_ratio_sum[bh] = lr_sum;
    }
  } else {
    // =====================================================================
    //                              state waves
    // =====================================================================
    const int sn = wave - NPREP;          // 16-channel sub-tile
    const int jcol = j0 + 16 * sn + c16;  // value channel of this lane
    f32x4 Sacc[8];                        // S^T tiles: rows i = 16 i8 + 4g + e, col jcol
    f16x8 Sb[4];                          // S^T / ss in the paired k order (K S^T, Q S^T operand)
    float ss = 1.f;                       // a power of two >= max |S| of the wave's channels
    // the fp16 copy of S^T, divided by ss (exact scaling: any state magnitude)
    auto stage_S = [&]() {
      float mx = 0.f;
#pragma unroll
      for (int i8 = 0; i8 < 8; ++i8)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(Sacc[i8][e]));
      ss = pow2_above(wave_max(mx));
      const float is = pow2_inv(ss);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        f32x4 a = Sacc[2 * kk], b = Sacc[2 * kk + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] *= is;
          b[e] *= is;
        }
        Sb[kk] = cat(h4(a), h4(b));
      }
    };
#pragma unroll
    for (int i8 = 0; i8 < 8; ++i8) Sacc[i8] = zero4();
    if (S0) {
#pragma unroll
      for (int i8 = 0; i8 < 8; ++i8) {
        const float4 s4 = *(const float4 *)(S0 + ((long)bh * 128 + jcol) * DK + 16 * i8 + 4 * g);
        Sacc[i8] = f32x4{s4.x, s4.y, s4.z, s4.w};
      }
    }
    stage_S();
    __syncthreads();

    // Carried from the iteration that prepared the chunk to the one that runs
    // it: K S^T, Q S^T and the values, all in the result layout (lane: column
    // jcol, rows 16m + 4g + e).
    f32x4 KS[4], O[4], V[4];
    f16x8 Rb[2], Xb[2], Xs[2];
    float sr = 1.f;  // R and X are held divided by sr, a power of two >= max |R|
#pragma unroll
    for (int m = 0; m < 4; ++m) KS[m] = O[m] = V[m] = zero4();

    for (int it = 0; nch > 0 && it <= nch; ++it) {
      refresh_lane();
      const int jcol = j0 + 16 * sn + c16;
      const int sc = it - 1;       // chunk in the state pass
      const int cb = sc & 1;
      const bool act = MODE != kScan && sc >= 0;
      const int sL = act ? min(C, T_ - sc * C) : 0;
      const int nb = it & 1;       // buffer the prep waves are filling
      const bool pact = it < nch;  // a chunk is being prepared

      // ------------------------------ phase 1 ------------------------------
      if (act) {
        // R = diag(beta)(V - K S^T), then R / sr in fp16, in the paired k order
        // for Tinv R
        f32x4 rf[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float4 b4 = *(const float4 *)&Lbeta[cb][16 * m + 4 * g];
          const float bb[4] = {b4.x, b4.y, b4.z, b4.w};
          if (GATED) {  // the entry state reaches token t decayed by gamma_t
            const float4 l4 = *(const float4 *)&Llga[cb][16 * m + 4 * g];
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) KS[m][e] *= fexp2(lv[e]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) rf[m][e] = bb[e] * (V[m][e] - KS[m][e]);
        }
        float mr = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e) mr = fmaxf(mr, fabsf(rf[m][e]));
        sr = pow2_above(wave_max(mr));
        const float isr = pow2_inv(sr);
        f16x4 rr[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int e = 0; e < 4; ++e) rr[m][e] = h(rf[m][e] * isr);
        Rb[0] = cat(rr[0], rr[1]);
        Rb[1] = cat(rr[2], rr[3]);
      }
      __syncthreads();

      // ------------------------------ phase 2 ------------------------------
      if (act) {
        // X / sr = Tinv (R / sr) (row blocks m need t pairs 0..m/2), in the paired k order
        f32x4 X[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          f32x4 acc = zero4();
          const f16 *row = &LTm[cb][(16 * m + c16) * CP];
#pragma unroll
          for (int qq = 0; qq <= (m >> 1); ++qq) acc = mma32(ldpk(row, 32 * qq, g), Rb[qq], acc);
          X[m] = acc;
        }
        Xb[0] = cat(h4(X[0]), h4(X[1]));
        Xb[1] = cat(h4(X[2]), h4(X[3]));
        if (GATED) {
          // rows of X for the state update, decayed to the chunk end: gamma_L / gamma_s
          const float lgL = Llga[cb][C - 1];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float4 l4 = *(const float4 *)&Llga[cb][16 * m + 4 * g];
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) X[m][e] *= fexp2(lgL - lv[e]);
          }
          Xs[0] = cat(h4(X[0]), h4(X[1]));
          Xs[1] = cat(h4(X[2]), h4(X[3]));
        }
      }
      if (pact && walk_mode(MODE)) key_gram_tile(8 + sn);
      if (pact && MODE != kScan) {
        // values of the chunk being prepared (staged row-major in Kt as bf16),
        // transposed exactly
#pragma unroll
        for (int m = 0; m < 4; ++m)
          V[m] = mma16bf(*(const bf16x4 *)&LKt[(16 * m + c16) * KP + 16 * sn + 4 * g], identb,
                         zero4());
      }
      __syncthreads();

      // ------------------------------ phase 3 ------------------------------
      if (pact && MODE == kOsdn) r_factor_rows(tid - 384, 2, nb);  // rows 4u + 2, 4u + 3
      if (act) {
        // O = Q S^T + P X, rounded to bf16, then turned through the identity so
        // that a lane holds 4 consecutive channels of one token (8-byte stores)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (GATED) {
            const float4 l4 = *(const float4 *)&Llga[cb][16 * m + 4 * g];
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) O[m][e] *= fexp2(lv[e]);
          }
          const f16 *row = &LP[cb][(16 * m + c16) * CP];
          // X is held divided by sr: O = sr (Q S^T / sr + P (X / sr))
          const float isr = pow2_inv(sr);
#pragma unroll
          for (int e = 0; e < 4; ++e) O[m][e] *= isr;
#pragma unroll
          for (int qq = 0; qq <= (m >> 1); ++qq) O[m] = mma32(ldpk(row, 32 * qq, g), Xb[qq], O[m]);
#pragma unroll
          for (int e = 0; e < 4; ++e) O[m][e] *= sr;
          const bf16x4 ob = {(bf16)O[m][0], (bf16)O[m][1], (bf16)O[m][2], (bf16)O[m][3]};
          const f32x4 ot = mma16bf(ob, identb, zero4());
          const int t = 16 * m + c16;
          if (t < sL)
            *(bf16x4 *)(o + (tok0 + (long)sc * C + t) * 128 + j0 + 16 * sn + 4 * g) =
                bf16x4{(bf16)ot[0], (bf16)ot[1], (bf16)ot[2], (bf16)ot[3]};
        }
      }
      __syncthreads();

      // ------------------------------ phase 4 ------------------------------
      if (act) {
        // S^T += ds sr Kt^T (X / sr), then the fp16 copy for the next products
        const float ds = Ldsb[cb] * sr;
        const float gL = GATED ? fexp2(Llga[cb][C - 1]) : 1.f;  // gamma_L
#pragma unroll
        for (int i8 = 0; i8 < 8; ++i8) {
          f32x4 u = zero4();
#pragma unroll
          for (int qq = 0; qq < 2; ++qq)
            u = mma32(ld8(&LKtF[cb][i8][qq][lane][0]), GATED ? Xs[qq] : Xb[qq], u);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            Sacc[i8][e] = fmaf(ds, u[e], GATED ? gL * Sacc[i8][e] : Sacc[i8][e]);
        }
        stage_S();
      }
      __syncthreads();

      // ------------------------------ phase 5 ------------------------------
      if (pact && MODE != kScan) {
        if (MODE == kOsdn) {
          write_keys_itile(6 + sn, nb);
        } else {
          const f16 *src = (MODE == kDeltaNet) ? LKp : LKt;
          for (int job = wave; job < 32; job += 8) write_keys_copy(job, src, nb);
        }
      }
      __syncthreads();

      // ------------------------------ phase 6 ------------------------------
      if (MODE != kScan && pact) {
        const f16 *Bsrc = (MODE == kDeltaNet) ? LKp : LKt;
        for (int job = sn; job < 6; job += 2) gram_a_off_tile(job, Bsrc, nb);
      }
      if (MODE != kScan) __syncthreads();

      // ------------------------------ phases 7-9 ------------------------------
      // K S^T (phase 7) and Q S^T (phase 8) of the chunk being prepared, from
      // the prep copies of K and Q and the state after this iteration's update.
#pragma unroll
      for (int dist = 1; dist < (MODE == kScan ? 1 : 4); ++dist) {
        if (pact && dist < 3) {
          const f16 *src = dist == 1 ? LKp : LQp;
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            f32x4 acc = zero4();
            const f16 *row = &src[(16 * m + c16) * KP];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mma32(ldpk(row, 32 * kk, g), Sb[kk], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] *= ss;  // Sb holds S^T / ss
            if (dist == 1) KS[m] = acc;
            else O[m] = acc;
          }
        }
        __syncthreads();
      }
    }

    if (S_final) {
#pragma unroll
      for (int i8 = 0; i8 < 8; ++i8)
        *(float4 *)(S_final + ((long)bh * 128 + jcol) * DK + 16 * i8 + 4 * g) =
            float4{Sacc[i8][0], Sacc[i8][1], Sacc[i8][2], Sacc[i8][3]};
    }
  }
}

template <int MODE, bool GATED>
__global__ void __launch_bounds__(NTH)
osdn_fused_forward(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                   const bf16 *__restrict__ kt_in, const bf16 *__restrict__ v,
                   const float *__restrict__ beta, const float *__restrict__ r,
                   const float *__restrict__ alpha,
                   const float *__restrict__ d0, const float *__restrict__ S0, float eta,
                   int BH, int T_, bf16 *__restrict__ o, float *__restrict__ S_final,
                   float *__restrict__ d_final, float *__restrict__ log_ratio_sum,
                   bf16 *__restrict__ kt_out, float *__restrict__ d_all,
                   float *__restrict__ log_ratio) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem &sm = *reinterpret_cast<Smem *>(smem_raw);
  fused_body<MODE, GATED>(q, k, kt_in, v, beta, r, alpha, d0, S0, eta, BH, T_, o, S_final, d_final,
                   log_ratio_sum, kt_out, d_all, log_ratio, sm.Kp, sm.Qp, sm.Kt, sm.KtF, sm.Tm, sm.P, sm.F, sm.Td, sm.d_in,
                   sm.dpart, sm.beta, sm.dsb, sm.r, sm.n, sm.bv, sm.alpha, sm.g, sm.cc, sm.w,
                   sm.rhs, sm.acc, sm.lg, &sm.lgC, sm.red, sm.al, sm.lga);
}

template <int MODE, bool GATED>
hipError_t launch_mg(const FusedArgs &a, const void *kt, hipStream_t s) {
  const int BH = a.B * a.H;
  const dim3 grid((unsigned)(BH * (128 / DVT))), block(NTH);
  const size_t shm = sizeof(Smem);
  hipError_t e = hipFuncSetAttribute((const void *)osdn_fused_forward<MODE, GATED>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((osdn_fused_forward<MODE, GATED>), grid, block, shm, s, (const bf16 *)a.q,
                     (const bf16 *)a.k, (const bf16 *)kt, (const bf16 *)a.v, a.beta,
                     MODE == kOsdn ? a.r : nullptr, a.alpha, a.d0, a.S0, a.eta, BH, a.T, (bf16 *)a.o,
                     a.S_final, a.d_final, a.log_ratio_sum, (bf16 *)nullptr, (float *)nullptr,
                     (float *)nullptr);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(const FusedArgs &a, const void *kt, hipStream_t s) {
  return a.alpha ? launch_mg<MODE, true>(a, kt, s) : launch_mg<MODE, false>(a, kt, s);
}

}  // namespace

bool fused_supported(int dk, int dv, int chunk, int dtype) {
  return dtype == 0 && dk == DK && dv == 128 && chunk == C;
}

hipError_t launch_fused_forward(const FusedArgs &a, hipStream_t s) {
  if ((long)a.B * a.H == 0) return hipSuccess;
  return a.precond_off ? launch_mode<kDeltaNet>(a, nullptr, s) : launch_mode<kOsdn>(a, nullptr, s);
}

bool fused_scan_supported(int dk, int dtype) { return dtype == 0 && dk == DK; }

hipError_t launch_fused_scan(const ScanArgs &a, hipStream_t s) {
  const int BH = a.B * a.H;
  if (BH == 0) return hipSuccess;
  const size_t shm = sizeof(Smem);
  hipError_t e = hipFuncSetAttribute((const void *)osdn_fused_forward<kScan, false>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((osdn_fused_forward<kScan, false>), dim3((unsigned)BH), dim3(NTH), shm, s,
                     (const bf16 *)nullptr, (const bf16 *)a.k, (const bf16 *)nullptr,
                     (const bf16 *)nullptr, a.beta, a.r, (const float *)nullptr, a.d0, (const float *)nullptr, a.eta, BH,
                     a.T, (bf16 *)nullptr, (float *)nullptr, a.d_final, a.log_ratio_sum,
                     (bf16 *)a.k_tilde, a.d_all, a.log_ratio);
  return hipGetLastError();
}

hipError_t launch_fused_chunk(const ChunkArgs &a, hipStream_t s) {
  if ((long)a.B * a.H == 0) return hipSuccess;
  FusedArgs f{a.q, a.k, a.v, a.beta, nullptr, a.alpha, nullptr, a.S0, 0.f, a.B, a.H, a.T, a.dk, a.dv,
              a.chunk, a.dtype, 0, a.o, a.S_final, nullptr, nullptr};
  return launch_mode<kGiven>(f, a.k_tilde, s);
}

}  // namespace osdn
