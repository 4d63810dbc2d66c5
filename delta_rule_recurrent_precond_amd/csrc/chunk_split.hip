// Two-kernel chunkwise pass for bf16 data, dk = dv = 128, chunk length 64.
//
// Source: gist.science technical summary of "OSDN: Improving Delta Rule with
// Provable Online Preconditioning in Linear Attention" -- §2.1 and the
// two-phase implementation of §2.2: given the write keys kt, the chunkwise
// delta-rule pass is DeltaNet's, with kt in place of k in the chunk gram, the
// intra-chunk scores and the state update.
//
// Within a chunk with entry state S (rows of S are value channels):
//   A = strict_lower(diag(beta) K Kt^T),  T = (I + A)^-1,  P = lower(Q Kt^T)
//   X = T diag(beta) (V - K S^T),  O = Q S^T + P X,  S <- S + X^T Kt
// Everything except the three products with S depends on one chunk only, so a
// chunk-parallel kernel (chunk_prep) forms it for all chunks at once and
// writes, per (b, h, chunk), the operands the sequential pass needs; the state
// kernel (chunk_state) then runs the pass, one wave per (b, h, 16 value
// channels), streaming those operands and q, k, v.  Numerically it follows the
// fused kernel step for step (the same fp16 operands, the same accumulation
// order), so both paths agree to rounding.
//
// Record of one (b, h, chunk) in the caller's workspace (REC bytes):
//   KtF  fp16 [8 i tiles][2 t pairs][64 lanes][8]  kt^T / ds as S-update operands
//   TmA  fp16 [6 ops][64 lanes][8]  rows of T as 16x16x32 A operands, paired k order
//   PA   fp16 [6 ops][64 lanes][8]  rows of P ds as A operands, paired k order
//   ds   fp32 write-key scale: kt is stored divided by ds, a power of two
//   lr   fp32 (kt = k only) sum over the chunk of log rho_t, rho_t = (1 - beta_t ||k_t||^2)^2
//   gL   fp32 (state gate) gamma_L, the decay of the chunk's entry state
//   sc   fp32 [2][64] (unnormalised q, k or a state gate) per-token factors of the
//        rows of K S^T and Q S^T: e_k/||k_t|| gamma_t and e_q/||q_t|| gamma_t
//        (gamma_t: product of the gates of the chunk up to t; L: its last row)
//   e    fp32 [2] (unnormalised q, k) 1 / e_k and 1 / e_q: raw k and q are staged
//        divided by these powers of two (>= the chunk's largest |k|, |q|), which
//        keeps every stored value exact in fp16 whatever the inputs' scale
// op x = 0..5 is (row block m, t pair qq) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1).
//
// With the state gate alpha (OSDN on the Gated DeltaNet backbone, read as
// S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) kt_t^T) the chunk
// form takes the decays gamma_t / gamma_s = 2^(lg_t - lg_s), lg_t the running
// sum of log2 alpha within the chunk, each term clamped at -126:
//   A_ts and P_ts gain gamma_t / gamma_s, the rows of K S^T and Q S^T gamma_t,
//   the S-update operand of token s gamma_L / gamma_s (applied to kt_s in fp32
//   before its fp16 rounding), and S <- gamma_L S + ...
//
// With one gate per key dimension (GK; the Kimi Delta Attention backbone,
// S_t = S_{t-1} diag(alpha_t) + beta_t (v_t - S_{t-1} diag(alpha_t) k_t) kt_t^T)
// the decays g_t = prod_{m<=t} alpha_m are vectors and enter every sum over the
// key dimension term by term:
//   A_ts = beta_t <k_t (.) g_t, kt_s / g_s>,  P_ts = <q_t (.) g_t, kt_s / g_s>,
//   K S^T -> (K (.) G) S^T,  Q S^T -> (Q (.) G) S^T,  S <- S diag(g_L) + X^T (Kt (.) g_L / G).
// No ratio g_t / g_s is ever formed by division.  A and P are built from
// products of alpha over the tokens between s and t:
//   - a 16x16 tile below the diagonal (row block r > column block c) factors
//     through the block boundaries, every factor <= 1: the rows of block r
//     take the product from the block's start to t (staged in place), the
//     columns take the product from s + 1 to the end of block c (staged in
//     place), and the products over the full blocks between c and r scale the
//     row operand as it is loaded;
//   - the diagonal 16x16 blocks are summed term by term on the vector ALU with
//     a running product down the rows.
// A zero gate therefore resets exactly.  The record then carries K (.) G and
// Q (.) G (fp16, what the state kernel stages in place of k and q) and g_L.
#include "device.h"
#include "launch.h"
#include "mfma.h"
#include "walk.h"
#include "walk_device.h"

namespace osdn {

namespace {

// kOsdn: kt formed from the walk's results; kDeltaNet: kt = k; kGiven: kt read
// from memory
enum PrepMode { kOsdn = 0, kDeltaNet = 1, kGiven = 2 };

constexpr int C = 64;
constexpr int DK = 128;
constexpr size_t REC = 32768;
constexpr size_t OFF_KTF = 0;
constexpr size_t OFF_TM = 16384;
constexpr size_t OFF_P = 22528;
constexpr size_t OFF_DS = 28672;
constexpr size_t OFF_LR = 28676;  // kt = k: sum over the chunk of log rho_t
constexpr size_t OFF_GL = 28680;  // gamma_L
constexpr size_t OFF_SC = 28688;  // per-token factors of the K rows, then of the Q rows
constexpr size_t OFF_KF = OFF_SC, OFF_QF = OFF_SC + 256;
// NORM: the powers of two that raw k and q are divided by when staged (fp32
// 1 / e_k, 1 / e_q), then padding to a 16-byte piece
constexpr size_t OFF_E = OFF_SC + 512, OFF_END = OFF_E + 16;
// the record with the per-channel gate: the above, then K (.) G and Q (.) G as
// fp16 [64][128] row-major, then g_L fp32 [128]
constexpr size_t OFF_KG = 32768, OFF_QG = 49152, OFF_GV = 65536, RECK = 66048;
constexpr int LDT = 24;  // padded row (halves) of the 16x16 fp16 blocks in LDS
constexpr int LDF = 20;  // padded row (floats) of the 16x16 fp32 blocks in LDS

__device__ __forceinline__ int op_index(int m, int qq) { return m < 2 ? m : 2 * m - 2 + qq; }

// zeros that a lane loads in place of a row of alpha (per-channel gate: the
// step of the diagonal sums that starts a column); never written
__device__ __align__(16) float g_zero16[16];

// ---------------------------------------------------------------------------
// chunk_prep: one workgroup of 4 waves per (b, h, chunk).  k, kt and q are
// loaded with all loads in flight at once, staged in LDS as fp16, and every
// product reads its operands from there.
// ---------------------------------------------------------------------------
constexpr int KP = 136;  // padded row (halves) of the staged [64][128] tiles

// kOsdn: threads 0-127 run the in-chunk preconditioner recurrence
// d_{t+1} = r_t d_t + c_t (k_t (.) k_t) from the chunk's entry d and the c_t
// of the walk (one key dimension each, fp32), forming kt_t = d_t (.) k_t twice:
// once for its largest magnitude (the scale ds), once to stage kt / ds.
// NORM (forward only): q and k arrive unnormalised.  q is staged normalised;
// for kOsdn k is staged as stored (exact) and its 1/||k_t|| enters the
// recurrence and the rows of A in fp32; for kt = k it is staged normalised.
// The scales go to the record for the state kernel.  GATED: the state gate's
// decays enter A, P and the S-update operands, and its row factors go to the
// record.  GK: the per-channel gate, as described at the top.  xf & kGateLogits:
// beta and r arrive as logits.
// The LDS of one chunk_prep instance.  q is needed only for the scores; the
// blocks of A and T then reuse its space.  QT (write keys of their own, no
// per-channel gate): the products of k with kt are formed first and held in
// registers, then q takes k's tile, then the blocks take it: two [64][128]
// tiles in all (36 KB, four workgroups per CU, where a tile of its own for q
// allows three)
template <int MODE, bool NORM, bool GATED, bool GK>
struct alignas(16) PrepLds {
  static constexpr bool QT = !GK && MODE != kDeltaNet;
  // (arrays an instance does not use keep a token size)
  f16 Ks[C * KP];                                        // k (QT: then q, then the blocks)
  f16 Kts[(MODE == kDeltaNet && !GK) ? 8 : C * KP];      // kt / ds
  alignas(16) unsigned char QF[QT ? 16 : C * KP * 2];
  float bs[C];
  float cs[(MODE == kOsdn || GATED) ? C : 4];            // kOsdn: c_t (GATED: then xdl)
  float rs[MODE == kOsdn ? C : 4];                       // kOsdn: r_t
  float sk[NORM ? C : 4], sq_[(NORM && MODE != kOsdn) ? C : 4];  // 1 / ||k_t||, 1 / ||q_t||
  float lga[GATED ? C : 4];                              // GATED: lg_t, the running sum of log2 alpha
  // GK: the diagonal blocks of A and P (fp32 sums); the products of alpha over
  // each 16-token block, per key dimension [block][i] (alpha itself is read
  // from global memory where it is used)
  float Adg[GK ? 4 * 16 * LDF : 4], Pdg[GK ? 4 * 16 * LDF : 4];
  alignas(16) float Bk[GK ? 4 * DK : 4];
  alignas(16) f16 Zrow[GK ? DK : 8];  // GK: zeros
  float red[4];
  // XN with kt = k: the chunk's largest |k| and |q| per wave (kOsdn passes them
  // through its kt tile instead, which nothing writes before the staging)
  float nred_[(NORM && !GK && MODE != kOsdn) ? 8 : 1];
};

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
// A store into a chunk record at byte offset off: plain, or (PUB) a
// device-scope (sc1) store for readers in other workgroups of the same launch.
// rec is wave-uniform.
template <bool PUB, typename T>
__device__ __forceinline__ void rec_put(unsigned char *rec, int off, const T &v) {
  if constexpr (!PUB) {
    *(T *)(rec + off) = v;
  } else {
    const __amdgpu_buffer_rsrc_t rr = wd::rsrc_over(rec, (int)REC);
    if constexpr (sizeof(T) == 4)
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), rr, off, 0, wd::kSc1);
    else if constexpr (sizeof(T) == 8)
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rr, off, 0, wd::kSc1);
    else {
      static_assert(sizeof(T) == 16, "records are stored 4, 8 or 16 bytes at a time");
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(wd::u32x4, v), rr, off, 0,
                                             wd::kSc1);
    }
  }
}

// One chunk (bh, c) by the 256 threads tid = 0..255 of the caller (every
// thread of the workgroup takes part in the same barriers, so several
// instances may share a workgroup).  COH: the walk's results (wout) are read
// with device-scope loads, the walk having written them in the same launch;
// poison: they are not known to be complete (the chunk's keys turn NaN).
template <int MODE, bool NORM, bool GATED, bool GK, bool COH, bool PUB = false>
__device__ __forceinline__ void chunk_prep_body(
    PrepLds<MODE, NORM, GATED, GK> &Ld, const int tid, const int bh, const int c,
    const bool poison, const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ kt_in, const float *__restrict__ beta, int T_, int NC,
    unsigned char *__restrict__ ws, const float *__restrict__ r, const float *__restrict__ wout,
    const float *__restrict__ alpha, unsigned xf, unsigned long long *__restrict__ pflag = nullptr,
    unsigned long long epoch = 0) {
  static_assert(!PUB || !GK, "the published records are the two-tile ones");
  constexpr bool QT = PrepLds<MODE, NORM, GATED, GK>::QT;
  f16 *const Ks = Ld.Ks;
  f16 *const Kts = Ld.Kts;
  unsigned char *const QF = Ld.QF;
  f16 *Qs = QT ? Ks : (f16 *)QF;                                       // q
  unsigned char *const Bl = QT ? (unsigned char *)Ks : QF;
  float(*Fd)[16][LDF] = (float(*)[16][LDF])Bl;                         // diagonal blocks of A
  f16(*Aoff)[16][LDT] = (f16(*)[16][LDT])(Bl + 4 * 16 * LDF * 4);       // off-diagonal blocks of A
  f16(*Tdg)[16][LDT] = (f16(*)[16][LDT])(Bl + 4 * 16 * LDF * 4 + 6 * 16 * LDT * 2);  // diag of T
  static_assert(4 * 16 * LDF * 4 + 10 * 16 * LDT * 2 <= C * KP * 2, "A and T blocks fit");
  float *const bs = Ld.bs, *const cs = Ld.cs, *const rs = Ld.rs;
  float *const sk = Ld.sk, *const sq_ = Ld.sq_, *const lga = Ld.lga;
  float *const Adg = Ld.Adg, *const Pdg = Ld.Pdg, *const Bk = Ld.Bk;
  f16 *const Zrow = Ld.Zrow;
  float *const red = Ld.red, *const nred_ = Ld.nred_;
  // Two arrays share space, so that the raw-input gated pass fits three
  // workgroups per CU: 1 / ||q_t|| (last read by the record's factors) lies in
  // kt's tile past the 512 bytes that carry d_32 (kOsdn writes kt only after
  // the recurrence), and gamma_L / gamma_t is written over c_t once the
  // recurrence is done.
  float *const sq = MODE == kOsdn ? (float *)Kts + 128 : sq_;
  float *const xdl = cs;          // GATED: gamma_L / gamma_t
  auto ld_wout = [&](const float *p) {
    return COH ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *p;
  };

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c16 = lane & 15, g = lane >> 4;
  const long tok0 = (long)bh * T_ + (long)c * C;
  const int L = min(C, T_ - c * C);
  unsigned char *rec = ws + ((long)bh * NC + c) * (GK ? RECK : REC);
  // XN: raw q and k are staged exactly, divided by a power of two per chunk,
  // and their normalisation enters as fp32 row and column factors of the
  // products (rounding the unit vectors to fp16 instead would put up to 2^-12
  // relative error on every element, which a near-orthogonal q . kt -- the
  // first token's output -- amplifies without bound)
  constexpr bool XN = NORM && !GK;
  // the write keys (GK keeps a copy of k for kt = k: the rows of Ks are rescaled)
  const f16 *Ktp = (MODE == kDeltaNet && !GK) ? Ks : Kts;

  // ---- loads: 1024 pieces of 8 elements per tensor, 4 per thread.  Rows past
  // the end reread the last row (a load under a condition would make the
  // compiler wait for it where the branches join) and are zeroed here.
  // k (and the given kt) first, q last: the staging of k then waits for k
  // alone, and q's loads stay in flight until q is staged
  uint4 rk[4], rq[4], rt[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = tid + 256 * u, t = p >> 4;
    const long off = (tok0 + min(t, L - 1)) * DK + (p & 15) * 8;
    rk[u] = *(const uint4 *)(k + off);
    if (MODE == kGiven) rt[u] = *(const uint4 *)(kt_in + off);
  }
  // kOsdn: the chunk's entry d of dimension tid (threads 0-127), loaded here so
  // that its latency passes while the chunk is staged, not on the d chain
  const float d_entry = MODE != kOsdn ? 0.f
                        : poison    ? __uint_as_float(0x7fc00000u)
                                    : ld_wout(&wout[((long)bh * NC + c) * WOUT + min(tid, DK - 1)]);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = tid + 256 * u, t = p >> 4;
    rq[u] = *(const uint4 *)(q + (tok0 + min(t, L - 1)) * DK + (p & 15) * 8);
  }
  // (q's rows past the end are zeroed where q is staged: a write to its
  // registers here would wait for its loads)
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if ((tid + 256 * u) >> 4 >= L) {
      rk[u] = uint4{0, 0, 0, 0};
      if (MODE == kGiven) rt[u] = uint4{0, 0, 0, 0};
    }
  }
  if (GK && tid < DK / 8) *(uint4 *)&Zrow[8 * tid] = uint4{0, 0, 0, 0};
  if (tid < C) {
    const float bv = beta[tok0 + min(tid, L - 1)];
    bs[tid] = tid < L ? ((xf & kGateLogits) ? sigmoid_gate(bv) : bv) : 0.f;
  }
  if (MODE == kOsdn && tid < C) {
    cs[tid] = tid < L ? ld_wout(&wout[((long)bh * NC + c) * WOUT + DK + tid]) : 0.f;
    const float rv = r ? r[tok0 + min(tid, L - 1)] : 1.0f;
    rs[tid] = (r && tid < L) ? ((xf & kGateLogits) ? sigmoid_gate(rv) : rv) : 1.0f;
  }
  // per-token normalisation scales (16 threads per token hold its pieces):
  // kinv = 1 / ||k_t||; XN: ik = 1 / e_k, iq = 1 / e_q with e a power of two >= the
  // chunk's largest |k| (|q|), and the factors kscale = e_k / ||k_t||, qscale =
  // e_q / ||q_t|| that turn the staged rows into unit vectors
  float kscale[4] = {1.f, 1.f, 1.f, 1.f}, qscale[4] = {1.f, 1.f, 1.f, 1.f};
  float kinv[4] = {1.f, 1.f, 1.f, 1.f};
  float ik = 1.f, iq = 1.f;
  if (NORM) {
    float mk = 0.f, mq = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned short *sk8 = (const unsigned short *)&rk[u];
      const unsigned short *sq8 = (const unsigned short *)&rq[u];
      float a = 0.f, b = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = bf2f(sk8[e]), y = bf2f(sq8[e]);
        a = fmaf(x, x, a);
        b = fmaf(y, y, b);
        mk = fmaxf(mk, fabsf(x));
        mq = fmaxf(mq, fabsf(y));
      }
      kinv[u] = kscale[u] = unit_scale(group_sum<16>(a));
      qscale[u] = unit_scale(group_sum<16>(b));
    }
    if (XN) {
      // the chunk's largest |k| and |q| per wave (kOsdn: through Kts, below
      // which its d_32 and q-norm factors lie)
      float *nred = MODE == kOsdn ? (float *)Kts + 256 : nred_;
      mk = wave_max(mk);
      mq = wave_max(mq);
      if (lane == 0) {
        nred[wave] = mk;
        nred[4 + wave] = mq;
      }
      __syncthreads();
      const float ek = pow2_above(fmaxf(fmaxf(nred[0], nred[1]), fmaxf(nred[2], nred[3])));
      const float eq = pow2_above(fmaxf(fmaxf(nred[4], nred[5]), fmaxf(nred[6], nred[7])));
      ik = 1.0f / ek;
      iq = 1.0f / eq;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kscale[u] *= ek;
        qscale[u] *= eq;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if ((tid & 15) == 0) {
        const int t = (tid + 256 * u) >> 4;
        sk[t] = kscale[u];
        sq[t] = qscale[u];
      }
    }
  }
  if (GATED && tid < C) {  // wave 0: an inclusive scan over the chunk's tokens
    const float av = alpha[tok0 + min(tid, L - 1)];
    float incl = fmaxf(flog2(tid < L ? av : 1.0f), -126.f);  // alpha = 0 stays finite
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    lga[tid] = incl;
  }

  // GK: alpha of the chunk for the block products (wave b: rows 16b .. 16b + 15,
  // dimensions 2 lane, 2 lane + 1; rows past the end are 1), issued after the
  // other loads so the waits for those leave them in flight.  They also bring
  // the chunk's alpha into L2 ahead of the diagonal sums, which read it row by row.
  float2 av[GK ? 16 : 1];
  if (GK) {
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int t = 16 * wave + u;
      const float2 a2 = *(const float2 *)(alpha + (tok0 + min(t, L - 1)) * DK + 2 * lane);
      av[u] = t < L ? a2 : float2{1.f, 1.f};
    }
  }

  // write-key scale: a power of two >= max |kt| (given keys), 1 for kt = k
  float ds = 1.0f;
  if (MODE == kGiven) {
    float km = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const unsigned short *s = (const unsigned short *)&rt[u];
#pragma unroll
      for (int e = 0; e < 8; ++e) km = fmaxf(km, fabsf(bf2f(s[e])));
    }
    km = wave_max(km);
    if (lane == 0) red[wave] = km;
    __syncthreads();
    km = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    ds = km > 0.f ? fexp2(ceilf(flog2(km))) : 1.0f;
  }
  float inv = 1.0f / ds;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = tid + 256 * u, t = p >> 4, i0 = (p & 15) * 8;
    *(f16x8 *)&Ks[t * KP + i0] = XN ? cvt8s(rk[u], ik)
                                 : (NORM && MODE == kDeltaNet) ? cvt8s(rk[u], kscale[u])
                                                               : cvt8(rk[u]);
    if (!QT)
      *(f16x8 *)&Qs[t * KP + i0] = t >= L   ? f16x8{0, 0, 0, 0, 0, 0, 0, 0}
                                   : XN     ? cvt8s(rq[u], iq)
                                   : NORM   ? cvt8s(rq[u], qscale[u])
                                            : cvt8(rq[u]);
    if (MODE == kGiven) {
      const unsigned short *s = (const unsigned short *)&rt[u];
      f16x8 hv;
#pragma unroll
      for (int e = 0; e < 8; ++e) hv[e] = h(bf2f(s[e]) * inv);
      *(f16x8 *)&Kts[t * KP + i0] = hv;
    }
    if (GK && MODE == kDeltaNet)
      *(f16x8 *)&Kts[t * KP + i0] = NORM ? cvt8s(rk[u], kscale[u]) : cvt8(rk[u]);
  }
  __syncthreads();

  // the state kernel's per-token factors
  if ((NORM || GATED) && !GK && tid < C) {
    float kf = NORM ? sk[tid] : 1.0f, qf = NORM ? sq[tid] : 1.0f;
    if (GATED) {
      const float gm = fexp2(lga[tid]), lgL = lga[C - 1];
      kf *= gm;
      qf *= gm;
      if (tid == 0) rec_put<PUB>(rec, (int)OFF_GL, fexp2(lgL));
    }
    rec_put<PUB>(rec, (int)OFF_KF + 4 * tid, kf);
    rec_put<PUB>(rec, (int)OFF_QF + 4 * tid, qf);
    if (tid == 0) rec_put<PUB>(rec, (int)OFF_E, float2{ik, iq});  // 1 unless XN
  }

  if (MODE == kOsdn) {
    // The in-chunk recurrence d_{t+1} = r_t d_t + c_t kh_t^2 in two halves at
    // once: threads 0-127 take tokens 0-31 of dimension tid from the entry d,
    // threads 128-255 tokens 32-63 of dimension tid - 128 from d = 0, carrying
    // the product P_t of r over 32 .. t-1 as well; the second half's
    // x_t = d_t kh_t is then P_t kh_t d_32 + e_t kh_t with the first half's
    // d_32.  The keys of a dimension are read first, so no LDS round trip sits
    // on the d chain; x_t stays in registers for the scale and the staging.
    const int dim = tid & (DK - 1), t0h = C / 2 * (tid >> 7);
    // d_32 passes through the start of Kts, which is written only after the
    // barrier that follows its last read (one more array would cost the third
    // workgroup per CU)
    float *dmid = (float *)Kts;
    // (d_t or e_t) kx_t; the second half's P_t kx_t is formed again after the
    // barrier from the keys and r, in the same order (fewer registers held)
    float xb[C / 2];
    {
      f16 kc[C / 2];
#pragma unroll
      for (int t = 0; t < C / 2; ++t) kc[t] = Ks[(t0h + t) * KP + dim];
      float d = t0h ? 0.f : d_entry, pr = 1.f;
#pragma unroll
      for (int t0 = 0; t0 < C / 2; t0 += 4) {
        const float4 c4 = *(const float4 *)&cs[t0h + t0], r4 = *(const float4 *)&rs[t0h + t0];
        const float cv[4] = {c4.x, c4.y, c4.z, c4.w}, rv[4] = {r4.x, r4.y, r4.z, r4.w};
        float sv[4] = {1.f, 1.f, 1.f, 1.f};
        if (NORM) {
          const float4 s4 = *(const float4 *)&sk[t0h + t0];
          sv[0] = s4.x, sv[1] = s4.y, sv[2] = s4.z, sv[3] = s4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // the normalised key is kv * sv; XN stages the write key in the
          // staged keys' frame, d_t kv, and its factor sv enters the products
          const float kv = (float)kc[t0 + e];
          const float kh = NORM ? kv * sv[e] : kv;
          const float kx = XN ? kv : kh;
          xb[t0 + e] = d * kx;
          d = fmaf(cv[e], kh * kh, rv[e] * d);
          pr *= rv[e];
        }
      }
      if (tid < DK) dmid[dim] = d;  // d_32
    }
    __syncthreads();
    // XN: the scores' query factors move from kt's tile (written below) to r's
    // array once the second half below has read r
    const float sqv = (XN && tid < C) ? sq[tid] : 0.f;
    // second half: x_t = (P_t kx_t) d_32 + e_t kx_t (the first half's x is xb)
    float km = 0.f;
    if (t0h) {
      const float dj = dmid[dim];
      float pr = 1.f;
#pragma unroll
      for (int t0 = 0; t0 < C / 2; t0 += 4) {
        const float4 r4 = *(const float4 *)&rs[t0h + t0];
        const float rv[4] = {r4.x, r4.y, r4.z, r4.w};
        float sv[4] = {1.f, 1.f, 1.f, 1.f};
        if (NORM) {
          const float4 s4 = *(const float4 *)&sk[t0h + t0];
          sv[0] = s4.x, sv[1] = s4.y, sv[2] = s4.z, sv[3] = s4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float kv = (float)Ks[(t0h + t0 + e) * KP + dim];
          const float kx = XN ? kv : (NORM ? kv * sv[e] : kv);
          xb[t0 + e] = fmaf(pr * kx, dj, xb[t0 + e]);
          pr *= rv[e];
        }
      }
    }
#pragma unroll
    for (int t = 0; t < C / 2; ++t) km = fmaxf(km, fabsf(xb[t]));
    km = wave_max(km);
    if (lane == 0) red[wave] = km;
    __syncthreads();
    if (XN && tid < C) rs[tid] = sqv;
    km = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    ds = km > 0.f ? fexp2(ceilf(flog2(km))) : 1.0f;
    inv = 1.0f / ds;
#pragma unroll
    for (int t = 0; t < C / 2; ++t) Kts[(t0h + t) * KP + dim] = h(xb[t] * inv);
    __syncthreads();
  }

  // GATED: gamma_L / gamma_t for the S-update operands, over c_t now that the
  // recurrence is done with it
  if (GATED && !GK && tid < C) xdl[tid] = fexp2(lga[C - 1] - lga[tid]);

  if (GK) {
    // (a) the diagonal blocks of A and P term by term.  Wave b takes block b;
    // only the 136 entries on and below the diagonal are summed.  Lane group
    // pr = lane >> 3 (8 lanes, 16 key dimensions each from i0) walks column pr
    // down rows pr .. 15, then column 15 - pr down rows 15 - pr .. 15: 17 steps
    // for every group.  u_i is kt_s,i times the product of alpha_i over s+1 .. t,
    // carried as u <- u alpha_t + z: a step that starts a column takes alpha = 0
    // (a table of zeros) and z = kt_s (its staged row), every other step the
    // row's alpha and z = 0 (a zero row), so the chain needs no select per
    // dimension.  Rows past the end read the last row's alpha: their k and q
    // rows are zero, so their entries are 0 whatever u is.  The 8 lanes of a
    // group add their partial sums.
    const int b = wave, pr = lane >> 3, i0 = 16 * (lane & 7);
#pragma unroll
    for (int x = 0; x < 4; ++x) {  // the entries above the diagonal are 0
      const int pos = lane + 64 * x, tl = pos >> 4, sl = pos & 15;
      if (sl > tl) {
        Adg[(16 * b + tl) * LDF + sl] = 0.f;
        Pdg[(16 * b + tl) * LDF + sl] = 0.f;
      }
    }
    auto row_of = [&](int j) { return j < 16 - pr ? pr + j : j - 1; };
    auto col_of = [&](int j) { return j < 16 - pr ? pr : 15 - pr; };
    auto starts = [&](int j) { return j == 0 || j == 16 - pr; };
    auto aload = [&](int j, float4 (&v)[4]) {
      const float *src = starts(j) ? g_zero16 : alpha + (tok0 + min(16 * b + row_of(j), L - 1)) * DK + i0;
#pragma unroll
      for (int x = 0; x < 4; ++x) v[x] = *(const float4 *)(src + 4 * x);
    };
    float u[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) u[x] = 0.f;
    float4 ab[3][4];  // alpha three steps ahead
    aload(0, ab[0]);
    aload(1, ab[1]);
    aload(2, ab[2]);
#pragma unroll
    for (int j = 0; j < 17; ++j) {
      const int tl = row_of(j), sl = col_of(j), t = 16 * b + tl;
      float al[16];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        al[4 * x] = ab[j % 3][x].x, al[4 * x + 1] = ab[j % 3][x].y;
        al[4 * x + 2] = ab[j % 3][x].z, al[4 * x + 3] = ab[j % 3][x].w;
      }
      if (j + 3 < 17) aload(j + 3, ab[j % 3]);
      const f16 *zp = starts(j) ? &Kts[(16 * b + sl) * KP + i0] : &Zrow[i0];
      const f16x8 z0 = ld8(zp), z1 = ld8(zp + 8);
      const f16x8 k0 = ld8(&Ks[t * KP + i0]), k1 = ld8(&Ks[t * KP + i0 + 8]);
      const f16x8 q0 = ld8(&Qs[t * KP + i0]), q1 = ld8(&Qs[t * KP + i0 + 8]);
      float a = 0.f, pq = 0.f;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const float zx = (float)(x < 8 ? z0[x] : z1[x - 8]);
        u[x] = fmaf(u[x], al[x], zx);
        a = fmaf((float)(x < 8 ? k0[x] : k1[x - 8]), u[x], a);
        pq = fmaf((float)(x < 8 ? q0[x] : q1[x - 8]), u[x], pq);
      }
      a = group_sum<8>(a);
      pq = group_sum<8>(pq);
      if ((lane & 7) == 0) {
        Adg[t * LDF + sl] = tl > sl ? a : 0.f;
        Pdg[t * LDF + sl] = pq;
      }
    }
    // (b) per pair of key dimensions (thread: dimensions i2, i2 + 1 of block
    // blk = wave): the products of alpha over each block, then
    //   g_t = (product over the earlier blocks) * (product from the block start to t)
    //   K (.) G and Q (.) G to the record; the rows of block r >= 1 of k and q
    //   rescaled by the product from the block start to t, and kt_s by the
    //   product from s + 1 to the block end (in place); g_L to the record.
    const int blk = wave, i2 = 2 * lane;
    float2 Bb = {1.f, 1.f};
#pragma unroll
    for (int u = 0; u < 16; ++u) Bb = float2{Bb.x * av[u].x, Bb.y * av[u].y};
    *(float2 *)&Bk[blk * DK + i2] = Bb;
    __syncthreads();  // block products visible; the diagonal sums have read k, q, kt
    float2 Bv[4], G = {1.f, 1.f};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      Bv[x] = *(const float2 *)&Bk[x * DK + i2];
      if (x < blk) G = float2{G.x * Bv[x].x, G.y * Bv[x].y};
    }
    f16 *kg = (f16 *)(rec + OFF_KG), *qg = (f16 *)(rec + OFF_QG);
    // every row is read before any is rewritten in place, so no LDS read waits
    // behind the previous row's stores
    f16x2 k2s[16], q2s[16], t2s[16];
#pragma unroll
    for (int tl = 0; tl < 16; ++tl) {
      const int t = 16 * blk + tl;
      k2s[tl] = *(const f16x2 *)&Ks[t * KP + i2];
      q2s[tl] = *(const f16x2 *)&Qs[t * KP + i2];
      t2s[tl] = *(const f16x2 *)&Kts[t * KP + i2];
    }
    float2 pp = {1.f, 1.f};
#pragma unroll
    for (int tl = 0; tl < 16; ++tl) {
      const int t = 16 * blk + tl;
      pp = float2{pp.x * av[tl].x, pp.y * av[tl].y};
      const f16x2 k2 = k2s[tl], q2 = q2s[tl];
      const float kx = (float)k2[0], ky = (float)k2[1], qx = (float)q2[0], qy = (float)q2[1];
      const float ks = (NORM && MODE == kOsdn) ? sk[t] : 1.f;
      const float gx = G.x * pp.x, gy = G.y * pp.y;
      *(f16x2 *)&kg[t * DK + i2] = f16x2{h((kx * ks) * gx), h((ky * ks) * gy)};
      *(f16x2 *)&qg[t * DK + i2] = f16x2{h(qx * gx), h(qy * gy)};
      if (blk > 0) {
        *(f16x2 *)&Ks[t * KP + i2] = f16x2{h(kx * pp.x), h(ky * pp.y)};
        *(f16x2 *)&Qs[t * KP + i2] = f16x2{h(qx * pp.x), h(qy * pp.y)};
      }
    }
    float2 ss = {1.f, 1.f};  // product over s+1 .. end of the block
#pragma unroll
    for (int tl = 15; tl >= 0; --tl) {
      const int s2 = 16 * blk + tl;
      const f16x2 t2 = t2s[tl];
      *(f16x2 *)&Kts[s2 * KP + i2] = f16x2{h((float)t2[0] * ss.x), h((float)t2[1] * ss.y)};
      ss = float2{ss.x * av[tl].x, ss.y * av[tl].y};
    }
    if (blk == 0)
      *(float2 *)(rec + OFF_GV + 4 * i2) = float2{(Bv[0].x * Bv[1].x) * (Bv[2].x * Bv[3].x),
                                                  (Bv[0].y * Bv[1].y) * (Bv[2].y * Bv[3].y)};
    __syncthreads();
  }

  f16x4 ident;
#pragma unroll
  for (int e = 0; e < 4; ++e) ident[e] = (4 * g + e == c16) ? (f16)1.0f : (f16)0.0f;

  // product tile (rt, ct) of X Kt^T over the 128 key dimensions
  auto gram = [&](const f16 *xs, int rt_, int ct) {
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc = mma32(ld8(&xs[(16 * rt_ + c16) * KP + 32 * kk + 8 * g]),
                  ld8(&Ktp[(16 * ct + c16) * KP + 32 * kk + 8 * g]), acc);
    return acc;
  };
  // GK: tile (rt, ct) below the diagonal: the rescaled rows of xs (times the
  // products over the full blocks between ct and rt, per key dimension) and the
  // rescaled rows of kt
  auto gramk = [&](const f16 *xs, int rt_, int ct) {
    f32x4 acc = zero4();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f16x8 a = ld8(&xs[(16 * rt_ + c16) * KP + 32 * kk + 8 * g]);
      if (rt_ > ct + 1) {
        const int i0 = 32 * kk + 8 * g;
        float m[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
        for (int bb = ct + 1; bb < rt_; ++bb) {
          const float4 b0 = *(const float4 *)&Bk[bb * DK + i0];
          const float4 b1 = *(const float4 *)&Bk[bb * DK + i0 + 4];
          const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) m[j] *= bv[j];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] = h((float)a[j] * m[j]);
      }
      acc = mma32(a, ld8(&Kts[(16 * ct + c16) * KP + 32 * kk + 8 * g]), acc);
    }
    return acc;
  };
  // GK: a diagonal block of A or P in the result layout
  auto diag4 = [&](const float *D, int b_) {
    f32x4 acc;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = D[(16 * b_ + 4 * g + e) * LDF + c16];
    return acc;
  };
  auto beta4 = [&](int rt_) { return *(const f32x4 *)&bs[16 * rt_ + 4 * g]; };
  // kOsdn, NORM stages k as stored: the rows of A take the keys' 1/||k||
  // (XN: e_k / ||k||; also the columns, through colf)
  auto krow4 = [&](int rt_) {
    return (NORM && (MODE == kOsdn || XN)) ? *(const f32x4 *)&sk[16 * rt_ + 4 * g]
                                           : f32x4{1.f, 1.f, 1.f, 1.f};
  };
  // XN: the factor of write key s (column s of A and of the scores)
  auto colf = [&](int s) { return XN ? sk[s] : 1.0f; };
  // GATED: gamma_t / gamma_s for rows t = 16 rt + 4g + e and column s (taken
  // only where s <= t, where it is <= 1)
  auto dec4 = [&](int rt_, int s) {
    if (!GATED) return f32x4{1.f, 1.f, 1.f, 1.f};
    const float4 lt = *(const float4 *)&lga[16 * rt_ + 4 * g];
    const float ls = lga[s];
    return f32x4{fexp2(lt.x - ls), fexp2(lt.y - ls), fexp2(lt.z - ls), fexp2(lt.w - ls)};
  };
  // an entry of A: beta_t ds [gamma_t / gamma_s] (k_t . kt_s) [/ ||k_t||]
  auto a_entry = [&](float b, float dc, float acc, float f) {
    float x = b * ds;
    if (GATED) x *= dc;
    x *= acc;
    if (NORM) x *= f;
    return x;
  };

  // QT: the products of k with kt for A (the diagonal block `wave`, then the
  // off-diagonal jobs wave and wave + 4) into registers; then q into k's tile
  f32x4 aD = zero4(), aO[2] = {zero4(), zero4()};
  if (QT) {
    aD = gram(Ks, wave, wave);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int job = wave + 4 * j;
      if (job < 6) {
        int rt_, ct;
        off_tile(job, rt_, ct);
        aO[j] = gram(Ks, rt_, ct);
      }
    }
    __syncthreads();  // k is no longer read
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = tid + 256 * u, t = p >> 4, i0 = (p & 15) * 8;
      *(f16x8 *)&Qs[t * KP + i0] = t >= L   ? f16x8{0, 0, 0, 0, 0, 0, 0, 0}
                                   : XN     ? cvt8s(rq[u], iq)
                                   : NORM   ? cvt8s(rq[u], qscale[u])
                                            : cvt8(rq[u]);
    }
    __syncthreads();
  }

  // ---- scores P = lower(Q Kt^T) ds, emitted as A operands (transposed tiles)
  for (int idx = wave; idx < 10; idx += 4) {
    int rt_, ct;
    tri_tile(idx, rt_, ct);
    f32x4 acc = !GK ? gram(Qs, rt_, ct) : rt_ == ct ? diag4(Pdg, rt_) : gramk(Qs, rt_, ct);
    if (XN) {  // the query rows' and the write-key columns' factors
      const f32x4 qf = *(const f32x4 *)&(MODE == kOsdn ? rs : sq)[16 * rt_ + 4 * g];
      const float kc = colf(16 * ct + c16);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = (acc[e] * qf[e]) * kc;
    }
    const f32x4 dc = dec4(rt_, 16 * ct + c16);
    f32x4 pv;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      pv[e] = (16 * ct + c16 <= 16 * rt_ + 4 * g + e) ? (GATED ? ds * dc[e] * acc[e] : ds * acc[e])
                                                     : 0.f;
    const f16x4 pt = h4(mma16(h4(pv), ident, zero4()));
    rec_put<PUB>(rec, (int)OFF_P + ((op_index(rt_, ct >> 1) * 64 + lane) * 8 + 4 * (ct & 1)) * 2, pt);
  }
  __syncthreads();  // q is no longer read: its space takes the blocks of A and T

  // ---- A: diagonal block `wave` (then its inverse) and off-diagonal blocks
  {
    const f32x4 acc = GK ? diag4(Adg, wave) : QT ? aD : gram(Ks, wave, wave);
    const f32x4 b4 = beta4(wave), f4 = krow4(wave), dc = dec4(wave, 16 * wave + c16);
    const float kc = colf(16 * wave + c16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * g + e;
      Fd[wave][row][c16] = c16 < row ? a_entry(b4[e], dc[e], acc[e] * kc, f4[e]) : 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int job = wave + 4 * j;
    if (job >= 6) break;
    int rt_, ct;
    off_tile(job, rt_, ct);
    const f32x4 acc = GK ? gramk(Ks, rt_, ct) : QT ? aO[j] : gram(Ks, rt_, ct);
    const f32x4 b4 = beta4(rt_), f4 = krow4(rt_), dc = dec4(rt_, 16 * ct + c16);
    const float kc = colf(16 * ct + c16);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      Aoff[job][4 * g + e][c16] = h(a_entry(b4[e], dc[e], acc[e] * kc, f4[e]));
  }
  wave_lds_sync();
  {
    float x[4];
    tri16_inverse_quad(&Fd[wave][0][0], LDF, lane, x);
#pragma unroll
    for (int j = 0; j < 4; ++j) Tdg[wave][(lane & 3) + 4 * j][lane >> 2] = h(x[j]);
  }

  // the two zero halves of P and T: blocks (0,1) and (2,3)
  if (wave == 0) {
    const f16x4 z = {0, 0, 0, 0};
    rec_put<PUB>(rec, (int)OFF_P + ((op_index(0, 0) * 64 + lane) * 8 + 4) * 2, z);
    rec_put<PUB>(rec, (int)OFF_P + ((op_index(2, 1) * 64 + lane) * 8 + 4) * 2, z);
    rec_put<PUB>(rec, (int)OFF_TM + ((op_index(0, 0) * 64 + lane) * 8 + 4) * 2, z);
    rec_put<PUB>(rec, (int)OFF_TM + ((op_index(2, 1) * 64 + lane) * 8 + 4) * 2, z);
  }

  // ---- write keys as S-update operands: i tiles 2w, 2w+1 (a lane holds tokens
  // 16m + 4g + e of key dimension 16n + c16); GATED: decayed to the chunk end
#pragma unroll
  for (int nn = 0; nn < 2; ++nn) {
    const int n = 2 * wave + nn;
    f16x4 tr[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      f32x4 tv = mma16(ld4(&Ktp[(16 * m + c16) * KP + 16 * n + 4 * g]), ident, zero4());
      if (XN) {  // tokens 16 m + 4 g + e: the write keys' factors
        const f32x4 kf = *(const f32x4 *)&sk[16 * m + 4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) tv[e] *= kf[e];
      }
      if (GATED) {
        const f32x4 xd = *(const f32x4 *)&xdl[16 * m + 4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) tv[e] *= xd[e];
      }
      if (GK && m < 3) {  // kt_s so far carries the product to its block end
        float after = 1.f;
        for (int bb = m + 1; bb < 4; ++bb) after *= Bk[bb * DK + 16 * n + c16];
#pragma unroll
        for (int e = 0; e < 4; ++e) tv[e] *= after;
      }
      tr[m] = h4(tv);
    }
#pragma unroll
    for (int qq = 0; qq < 2; ++qq)
      rec_put<PUB>(rec, (int)OFF_KTF + (((n * 2 + qq) * 64 + lane) * 8) * 2, cat(tr[2 * qq], tr[2 * qq + 1]));
  }
  if (tid == 0) rec_put<PUB>(rec, (int)OFF_DS, ds);
  if (MODE == kDeltaNet) {
    // log rho_t with a_t = ||k_t||^2 from the stored values (16 threads per token)
    float lr = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int p = tid + 256 * u, t = p >> 4;
      const unsigned short *sv = (const unsigned short *)&rk[u];
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = bf2f(sv[e]);
        sq = fmaf(x, x, sq);
      }
      sq = group_sum<16>(sq);
      if (NORM) sq *= kinv[u] * kinv[u];  // of the normalised key
      const float gd = 1.0f - bs[t] * sq;
      if ((p & 15) == 0 && t < L) lr += logf(gd * gd);
    }
    lr = wave_sum(lr);
    if (lane == 0) red[wave] = lr;
  }

  __syncthreads();  // Tdg and Aoff complete
  if (MODE == kDeltaNet && tid == 0)
    rec_put<PUB>(rec, (int)OFF_LR, (red[0] + red[1]) + (red[2] + red[3]));

  // ---- T: the diagonal block of row block `wave` as an A-operand half, then
  // column `wave` below the diagonal: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj
  {
    const int m = wave;
    rec_put<PUB>(rec, (int)OFF_TM + ((op_index(m, m >> 1) * 64 + lane) * 8 + 4 * (m & 1)) * 2,
                 ld4(&Tdg[m][c16][4 * g]));
  }
  if (wave < 3) {
    const int bj = wave;
    f16x4 tcol[4];  // T_{bk, bj} in the result layout (lane: column, rows 4g..4g+3)
#pragma unroll
    for (int e = 0; e < 4; ++e) tcol[bj][e] = Tdg[bj][4 * g + e][c16];
#pragma unroll
    for (int bi = 1; bi < 4; ++bi) {
      if (bi <= bj) continue;
      f32x4 y = zero4();
#pragma unroll
      for (int bk = 0; bk < 3; ++bk)
        if (bk >= bj && bk < bi) {
          const int ofj = bi == 1 ? 0 : bi == 2 ? 1 + bk : 3 + bk;  // off-diagonal index of (bi, bk)
          y = mma16(ld4(&Aoff[ofj][c16][4 * g]), tcol[bk], y);
        }
      const f32x4 z = mma16(ld4(&Tdg[bi][c16][4 * g]), h4(y), zero4());
      f32x4 nz;
#pragma unroll
      for (int e = 0; e < 4; ++e) nz[e] = -z[e];
      tcol[bi] = h4(nz);
      const f16x4 tt = h4(mma16(tcol[bi], ident, zero4()));
      rec_put<PUB>(rec, (int)OFF_TM + ((op_index(bi, bj >> 1) * 64 + lane) * 8 + 4 * (bj & 1)) * 2, tt);
    }
  }
  if (PUB) {  // every wave's record stores complete, then the chunk's flag
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) __hip_atomic_store(pflag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One workgroup of 4 waves per (b, h, chunk), chunk-major, last chunk first,
// heads innermost: the state kernel reads every head's chunk 0 first, which is
// then the freshest data in the caches; with B*H a multiple of 8 a head runs on
// the XCD its state-kernel tiles use.  The grid may cover only the last chunks
// of every head (BHn heads): the others were prepared elsewhere.
template <int MODE, bool NORM, bool GATED, bool GK>
// Four workgroups per CU where the LDS allows it (the two-tile instances) and
// the registers fit a quarter of the file without spilling (not with raw q, k)
__global__ void __launch_bounds__(256, (!GK && !NORM && MODE != kDeltaNet) ? 4 : 1)
chunk_prep(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
           const bf16 *__restrict__ kt_in, const float *__restrict__ beta, int T_, int NC,
           int BHn, unsigned char *__restrict__ ws, const float *__restrict__ r,
           const float *__restrict__ wout, const float *__restrict__ alpha, unsigned xf) {
  __shared__ PrepLds<MODE, NORM, GATED, GK> Ld;
  const int c = NC - 1 - (int)(blockIdx.x / BHn), bh = blockIdx.x % BHn;
  chunk_prep_body<MODE, NORM, GATED, GK, false>(Ld, threadIdx.x, bh, c, false, q, k, kt_in, beta,
                                                T_, NC, ws, r, wout, alpha, xf);
}

// ---------------------------------------------------------------------------
// walk_chunk_pipe: the one-launch walk (the walks in workgroups 0 .. BH-1, the
// others preparing their records) in which the preparing workgroups, once
// their records are done, run chunk_prep for the first NCP chunks of every
// head while the walks finish: the walks leave most of the device idle at
// their end.  A walk publishes its results (device-scope stores, and a flag
// per chunk once a chunk's are complete); a chunk is prepared once its flag is
// set.  The walk records lie in the chunk records' slots (stride REC), with
// their two flags past them: chunk_prep overwrites a slot only after the walk
// has passed its chunk, when nothing reads the walk record or the flags any
// more.  chunk_prep's own launch then covers chunks NCP .. NC-1.  The
// chunk_prep items (chunk-major, heads innermost) continue the walk records'
// sequence of rounds from the next multiple of three: round q of workgroup j
// takes items 3 (NPW q + j) + inst of the whole sequence, so every workgroup
// runs about the same number of rounds.  A round whose items run past the
// last one repeats it (the same bytes written twice, by instances of one
// workgroup, whose flag waits all end before the body's first barrier).  NORM
// and GATED as chunk_prep's (raw q and k, the state gate alpha); the
// per-channel gate, whose chunk_prep needs more LDS, does not take this form.
// ---------------------------------------------------------------------------
template <bool NORM, bool GATED>
using TailLds = PrepLds<kOsdn, NORM, GATED, false>;
template <bool NORM, bool GATED>
constexpr size_t kTailSmem = wd::kPipeSmem > 3 * sizeof(TailLds<NORM, GATED>)
                                 ? wd::kPipeSmem
                                 : 3 * sizeof(TailLds<NORM, GATED>);

template <bool NORM, bool GATED>
__global__ void __launch_bounds__(wd::WT)
walk_chunk_pipe(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                const float *__restrict__ beta, const float *__restrict__ r, float eta,
                unsigned xf, unsigned char *__restrict__ ws, const float *__restrict__ d0, int T_,
                int NC, int NCP, int BH, float *__restrict__ wout, float *__restrict__ d_final,
                float *__restrict__ log_ratio_sum, const float *__restrict__ alpha,
                unsigned long long epoch) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  unsigned long long *flags = (unsigned long long *)(ws + WREC);
  constexpr int fstride = (int)(REC / 8);
  if ((int)blockIdx.x < BH) {
    wd::walk_body<true, true>(smem_raw, blockIdx.x, k, ws, REC, d0, T_, NC, wout, d_final,
                              nullptr, log_ratio_sum, flags, fstride, epoch);
    return;
  }
  const int j = blockIdx.x - BH, NPW = gridDim.x - BH;
  const int q0 =
      wd::pipe_prep(smem_raw, j, NPW, BH, k, beta, r, eta, xf, ws, REC, T_, NC, flags, fstride, epoch);
  const int inst = threadIdx.x >> 8;
  TailLds<NORM, GATED> &Ld = reinterpret_cast<TailLds<NORM, GATED> *>(smem_raw)[inst];
  const int first = (BH * NC + 2) / 3 * 3;  // where the chunk_prep items start in the sequence
  const int total = BH * NCP;
  bool gave_up = false;  // once a wait ran out, later items do not wait
  for (int qr = q0; 3 * (NPW * qr + j) - first < total; ++qr) {
    const int ii = min(3 * (NPW * qr + j) - first + inst, total - 1);
    const int c = ii / BH, bh = ii % BH;
    // the walk past chunk c (a bounded wait; the walk is far ahead by now)
    bool ok = false;
    const unsigned long long *f = &flags[((long)bh * NC + c) * fstride + 1];
    for (int i = 0; !gave_up && i < wd::kPollLimit; ++i) {
      if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    gave_up = !ok;
    // (the thread index through an opaque copy each round, so that the
    // compiler does not hoist the body's lane-dependent addresses out of the
    // loop and keep them live across it)
    int tid = threadIdx.x & 255;
    asm volatile("" : "+v"(tid));
    chunk_prep_body<kOsdn, NORM, GATED, false, true>(Ld, tid, bh, c, !ok, q, k, nullptr, beta, T_,
                                                     NC, ws, r, wout, alpha, xf);
    __syncthreads();  // the next round's staging overwrites this round's LDS
  }
}

// ---------------------------------------------------------------------------
// chunk_state: one workgroup of 12 waves per (b, h, 32 value channels),
// sequential over chunks.  Per 16-channel sub-tile sn:
//   wave sn (the state chain)  K S^T, R = diag(beta)(V - K S^T), X = T R,
//                              S^T += ds Kt^T X; passes X and the new fp16 S^T
//                              to the output wave through LDS
//   wave 2 + sn (the outputs)  Q S^T of chunk c (from the S^T the chain wave
//                              left), then in the next pass O = Q S^T + P X of
//                              chunk c, staged in LDS with the other output
//                              wave's channels and stored 64 bytes a token
//   waves 4-11 (loaders)       global loads of chunk c+2 (GK: c+3), LDS stores of c+1
// The output wave keeps Q S^T and the score operands of chunk c in registers
// so that the loaders may refill that chunk's LDS buffer.  The loaders keep two
// chunks in registers (three with GK), so a chunk's loads are issued one
// chunk (two) before it is stored.
// The roles meet at one barrier, after the first chunk is stored and the first
// S staged; from then on they hand chunks to each other through counters in
// LDS (StateSmem::cnt), each role waiting only for the buffers it reads or is
// about to overwrite, so that no role waits for the slowest of the others each
// chunk.  Each role runs its own loop, so the registers of different roles are
// never live at the same time.
// SCALED (unnormalised q, k or a state gate): q and k are staged as stored and
// the record's per-token factors scale the rows of K S^T and Q S^T in fp32.
// GATED: S decays by the record's gamma_L (the update operands carry the rest).
// GK (per-channel gate): q and k come from the record as K (.) G and Q (.) G
// (fp16), and S decays per key dimension by the record's g_L (kept in the
// factor slot of the LDS record).
// ---------------------------------------------------------------------------
constexpr int ST = 768;        // threads
constexpr int NL = ST - 256;   // loader lanes
// k and q rows in the state kernel's LDS: 256 bytes, no padding, held in the
// paired k order of the 16x16x32 products, so that each operand is one 16-byte
// read.  16-byte chunk 4 kk + g of row t holds k slots 32 kk + 4 g .. +3 and
// 32 kk + 16 + 4 g .. +3, stored at chunk (4 kk + g) ^ (t & 15): the sixteen rows
// one read covers then spread over all banks.
__device__ __forceinline__ int kq_chunk(int t, int chunk) { return t * 128 + 8 * (chunk ^ (t & 15)); }
// value-tile row staged by loader lane lt < 256 (its channels: 8 ((lt >> 4) & 3) .. +7)
__device__ __forceinline__ int vrow(int lt) {
  const int w = lt >> 4, i = lt & 15;
  return 32 * ((w >> 2) & 1) + 16 * (i >> 3) + 8 * (w >> 3) + (i & 7);
}

struct StateSmem {
  f16 K[2][C * 128];  // kq_chunk layout
  f16 Q[2][C * 128];
  uint4 V[2][2][2][64];  // value tile (bf16, exact) as operands [buf][sn][m >> 1][lane]: rows 16 m + c16, 4 channels
  unsigned char rec[2][OFF_END];  // KtF, TmA, PA, ds, factors of the chunk
  float b[2][C];
  f16x8 Sx[2][2][4][64];  // fp16 S^T at a chunk's start [parity][sn][kk][lane], paired order
  f16x8 Xx[2][2][2][64];  // X of a chunk [parity][sn][qq][lane], paired order
  float sig[2][2][2];     // [parity][sn]: the powers of two Sx and Xx are scaled down by
  // a chunk's outputs in bf16 on their way to global memory [token][OSP]:
  // channel 16 sn + j of the tile at slot j (rows of 80 bytes, 16-byte aligned)
  bf16 Ost[C * 40];
  // progress counters (see chunk_state): [0] loader-wave chunk stores, [1 + sn]
  // chunks done by chain wave sn (+1 for the first S), [4 + sn] output passes
  // done by output wave sn, [6] output tiles staged and [7] output tiles read
  // (both output waves)
  int cnt[8];
};
constexpr int OSP = 40;  // row of Ost (bf16)
static_assert(sizeof(StateSmem) <= 160 * 1024, "LDS budget");

// Bounded wait until the LDS counter *p reaches target (every lane reads the
// same word; the value is taken as wave-uniform).  The waves of one workgroup
// hand chunks to each other through these counters: a wave's LDS operations
// reach the LDS in issue order, so data it stored before incrementing a
// counter is in place for any wave that then sees the increment.  The empty
// asm statements keep the compiler from moving LDS accesses across a wait or
// an increment.  The bound (about 2^22 sleeps of 64 cycles) only ensures the
// wave ends if a counter were never reached; the protocol reaches every one.
__device__ __forceinline__ void lds_wait_geq(const int *p, int target) {
  asm volatile("" ::: "memory");
  for (int i = 0; i < (1 << 22); ++i) {
    const int v = __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (v >= target) break;
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");
}
__device__ __forceinline__ void lds_count(int *p, int lane) {
  asm volatile("" ::: "memory");
  if (lane == 0) __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  asm volatile("" ::: "memory");
}

// The state pass of state workgroup b (head and 32-channel tile; see chunk_state).
// PIPE: the chunk records are written by other workgroups of the same launch,
// each announced by pflags[(bh NC + c) pfstride] = epoch once complete; the
// loaders read a record only after its flag (the records' space is written
// once in the launch, so plain loads then see the record).  A loader wave
// whose wait runs out stages NaN keys, so that the outputs turn NaN.
template <bool SCALED, bool GATED, bool GK, bool PIPE>
__device__ __forceinline__ void state_body(
    unsigned char *smem_raw, const int b, const bf16 *__restrict__ q, const bf16 *__restrict__ k,
    const bf16 *__restrict__ v, const float *__restrict__ beta, const float *__restrict__ S0,
    int BH, int T_, int NC, const unsigned char *__restrict__ ws, bf16 *__restrict__ o,
    float *__restrict__ S_final, float *__restrict__ log_ratio_sum, unsigned xf,
    const unsigned long long *__restrict__ pflags, int pfstride, unsigned long long epoch) {
  static_assert(!PIPE || (!GK && !SCALED), "the one-launch forward has the plain records");
  StateSmem &sm = *reinterpret_cast<StateSmem *>(smem_raw);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c16 = lane & 15, g = lane >> 4;
  // (head, 32-channel tile); the four tiles of a head share one XCD (and its L2)
  int bh, tile;
  {
    if ((BH & 7) == 0) {
      bh = 8 * (b >> 5) + (b & 7);
      tile = (b >> 3) & 3;
    } else {
      bh = b >> 2;
      tile = b & 3;
    }
  }
  const int j0 = 32 * tile;  // first channel of the tile

  f16x4 ident;
  bf16x4 identb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ident[e] = (4 * g + e == c16) ? (f16)1.0f : (f16)0.0f;
    identb[e] = (4 * g + e == c16) ? (bf16)1.0f : (bf16)0.0f;
  }

  if (wave >= 4) {
    // ================================ loaders ================================
    // k and q as 2048 pieces of 8 elements, the value tile as 256, the record as
    // OFF_DS/16 + 1 = 1793 pieces of 16 bytes (1825 with the row factors), beta.
    // Loads are unconditional (a masked lane reads a valid address) and masked
    // values are zeroed when stored: a conditional load makes the compiler wait
    // for it at the end of its branch.
    // GK: 32 more pieces, g_L, from OFF_GV into the factor slot (piece 1793 on);
    // SCALED: the factors and the staging scales of raw k and q
    constexpr int RP0 = (int)(OFF_DS / 16) + 1;
    constexpr int RECP = GK ? RP0 + 32 : SCALED ? (int)(OFF_END / 16) : RP0;
    static_assert(RP0 * 16 == (int)OFF_SC, "g_L lands in the factor slot");
    constexpr size_t RB = GK ? RECK : REC;
    constexpr int NKQ = 2048 / NL, NR = (RECP + NL - 1) / NL;
    static_assert(NKQ * NL == 2048, "every lane stages whole pieces of k and q");
    const int lt = tid - 256;
    struct Regs {
      uint4 kq[NKQ], v, r[NR];
      float b;
      float2 e;  // SCALED: 1 / e_k, 1 / e_q
    };
    Regs ra, rb, rc;
    // PIPE: wait until the records of chunks 0 .. cc are all announced (a
    // wave-uniform call).  `ready` counts the chunks from 0 known to be ready;
    // a poll reads the flags of the 64 chunks from there on.  Once the bound
    // ran out the wave stops waiting and stages NaN keys.
    int ready = 0;
    bool bad = false;
    auto await = [&](int cc) {
      if (bad) return;
      const unsigned long long *f = pflags + (long)bh * NC * pfstride;
      for (int i = 0; i < wd::kPollLimit; ++i) {
        if (cc < ready) return;
        const unsigned long long fv =
            __hip_atomic_load(f + (long)min(ready + lane, NC - 1) * pfstride, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long set = __ballot(fv == epoch);
        ready += ~set == 0ull ? 64 : __builtin_ctzll(~set);
        if (cc < ready) return;
        __builtin_amdgcn_s_sleep(8);
      }
      bad = true;
    };
    // chunk cc clamped to the last one: the loads past the end reread it
    auto load = [&](Regs &R, int cc) {
      cc = min(cc, NC - 1);
      if (PIPE) await(cc);
      const long t0 = (long)bh * T_ + (long)cc * C;
      const int L = min(C, T_ - cc * C);
      const unsigned char *rp = ws + ((long)bh * NC + cc) * RB;
#pragma unroll
      for (int u = 0; u < NKQ; ++u) {
        const int p = min(lt + NL * u, 2047), pp = p & 1023, t = min(pp >> 4, L - 1);
        if (GK)  // K (.) G, Q (.) G: fp16 rows of 256 bytes in the record
          R.kq[u] = *(const uint4 *)(rp + (p < 1024 ? OFF_KG : OFF_QG) + t * 256 + (pp & 15) * 16);
        else
          R.kq[u] = *(const uint4 *)((p < 1024 ? k : q) + (t0 + t) * DK + (pp & 15) * 8);
      }
      {
        const int t = min(vrow(lt & 255), L - 1);
        R.v = *(const uint4 *)(v + (t0 + t) * 128 + j0 + ((lt >> 4) & 3) * 8);
      }
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        const int p = min(lt + NL * u, RECP - 1);
        R.r[u] = *(const uint4 *)(rp + ((GK && p >= RP0) ? OFF_GV + (p - RP0) * 16 : p * 16));
      }
      R.b = beta[t0 + min(lt & 63, L - 1)];
      if (SCALED) R.e = *(const float2 *)(rp + OFF_E);
    };
    // chunk cc (< NC) from its register set into LDS buffer cc & 1
    auto stash = [&](const Regs &R, int cc) {
      const int buf = cc & 1, L = min(C, T_ - cc * C);
      const f16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < NKQ; ++u) {
        // piece jp of row t (slots 8 jp .. +7) goes as two halves to chunks
        // 4 kk + 2 (jp & 1) and the next one, in their half (jp >> 1) & 1.  LDS
        // writes are served 16 lanes (128 bytes) a clock: pieces with jp >= 8
        // write their second half first, so that each write of the 16 lanes
        // of a row covers 8 chunks of distinct residue mod 8, all banks once.
        const int p = lt + NL * u, pp = p & 1023, t = pp >> 4, jp = pp & 15;
        const int c0 = 4 * (jp >> 2) + 2 * (jp & 1), hh = 4 * ((jp >> 1) & 1);
        const bool sw = jp >= 8;
        const f16x8 x0 = t < L ? (GK       ? __builtin_bit_cast(f16x8, R.kq[u])
                                  : SCALED ? cvt8s(R.kq[u], p < 1024 ? R.e.x : R.e.y)
                                           : cvt8(R.kq[u]))
                               : z8;
        const f16 qnan = __builtin_bit_cast(f16, (unsigned short)0x7e00);
        const f16x8 x = (PIPE && bad) ? f16x8{qnan, qnan, qnan, qnan, qnan, qnan, qnan, qnan} : x0;
        const f16x4 lo = f16x4{x[0], x[1], x[2], x[3]}, hi = f16x4{x[4], x[5], x[6], x[7]};
        f16 *base = (p < 1024 ? sm.K : sm.Q)[buf];
        *(f16x4 *)&base[kq_chunk(t, c0 + sw) + hh] = sw ? hi : lo;
        *(f16x4 *)&base[kq_chunk(t, c0 + !sw) + hh] = sw ? lo : hi;
      }
      arrived(R.v);  // (the stores below sit in a branch)
      arrived(R.b);
#pragma unroll
      for (int u = 0; u < NR; ++u) arrived(R.r[u]);
      if (lt < 256) {
        // row r, channels 8 q .. +7 of the tile: the operands of sub-tile q >> 1,
        // lanes r % 16 + 16 g for g = 2 (q & 1) and the next, half m & 1.  The
        // 16 lanes of one write cover rows of 8 residues mod 8 and both m parities.
        // The values stay bf16 (exact at any scale).
        const int r = vrow(lt), q = (lt >> 4) & 3, m = r >> 4, g0 = 2 * (q & 1);
        const uint4 x = r < L ? R.v : uint4{0, 0, 0, 0};
        unsigned *vb = (unsigned *)sm.V[buf][q >> 1][m >> 1];
        *(uint2 *)&vb[((r & 15) + 16 * g0) * 4 + 2 * (m & 1)] = uint2{x.x, x.y};
        *(uint2 *)&vb[((r & 15) + 16 * g0 + 16) * 4 + 2 * (m & 1)] = uint2{x.z, x.w};
      }
      uint4 *rd = (uint4 *)sm.rec[buf];
#pragma unroll
      for (int u = 0; u < NR; ++u) {
        const int p = lt + NL * u;
        if (p < RECP) rd[p] = R.r[u];
      }
      if (lt < C)
        sm.b[buf][lt] = lt < L ? ((xf & kGateLogits) ? sigmoid_gate(R.b) : R.b) : 0.f;
    };
    // Chunk cc goes into buffer cc & 1 once every loader wave has stored chunk
    // cc - 1 (no loader wave is then more than one chunk ahead of another, so a
    // count of 8 (cc + 1) means all eight have stored chunk cc), both chain waves
    // are done with chunk cc - 2 and both output waves with their pass over it.
    auto put = [&](const Regs &R, int cc) __attribute__((always_inline)) {
      asm volatile("" ::: "memory");
      for (int i = 0; i < (1 << 22); ++i) {
        const int l = __hip_atomic_load(&sm.cnt[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int h0 = __hip_atomic_load(&sm.cnt[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int h1 = __hip_atomic_load(&sm.cnt[2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int o0 = __hip_atomic_load(&sm.cnt[4], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int o1 = __hip_atomic_load(&sm.cnt[5], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const bool ok = l >= 8 * cc && min(h0, h1) >= cc && min(o0, o1) >= cc - 1;
        if (__builtin_amdgcn_readfirstlane((int)ok)) break;
        __builtin_amdgcn_s_sleep(1);
      }
      asm volatile("" ::: "memory");
      stash(R, cc);
      lds_count(&sm.cnt[0], lane);
    };
    // The loop bodies hold no condition: a store guarded by one would leave
    // the loads in flight differently on its two paths, and the waits after
    // the join would then drain every load.  A store of the chunk past the
    // last (zeros, the last record reread) goes to a buffer no one reads.
    if (!GK) {
      // Entering iteration c the loaders hold chunk c+1 in one register set; they
      // load chunk c+2 into the other (freed by the previous store), then store
      // chunk c+1.  Written for two iterations so that the sets keep fixed names.
      if (NC > 0) {
        load(ra, 0);
        load(rb, 1);
        stash(ra, 0);
      }
      __syncthreads();
      for (int c = 0; c + 1 < NC; c += 2) {
        load(ra, c + 2);
        put(rb, c + 1);
        load(rb, c + 3);
        put(ra, c + 2);
      }
      return;
    }
    // GK (larger records, which miss the last-level cache more often): three
    // register sets.  Entering iteration c the loaders hold chunks c+1 and c+2;
    // they load chunk c+3 into the third set (freed by the previous store), then
    // store chunk c+1, so every load has two iterations to arrive.
    if (NC > 0) {
      load(ra, 0);
      load(rb, 1);
      load(rc, 2);
      stash(ra, 0);
    }
    __syncthreads();
    int c = 0;
    for (; c + 2 < NC; c += 3) {
      load(ra, c + 3);
      put(rb, c + 1);
      load(rb, c + 4);
      put(rc, c + 2);
      load(rc, c + 5);
      put(ra, c + 3);
    }
    // the last one or two chunks (c, c+1): chunk c+1 still to store
    if (c + 1 < NC) put(rb, c + 1);
  } else if (wave < 2) {
    // ============================== state chain ==============================
    const int sn = wave;
    const int jcol = j0 + 16 * sn + c16;
    f32x4 Sacc[8];  // S^T tiles: rows i = 16 i8 + 4g + e, column jcol
    f16x8 Sb[4];    // S^T / ss in the paired k order
    float ss = 1.f; // ss: a power of two >= max |S| of the wave's channels
    // the fp16 copy of S^T for the products, divided by ss (exact scaling), into
    // LDS for the output wave with its scale
    auto stage_S = [&](int parity) {
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
        sm.Sx[parity][sn][kk][lane] = Sb[kk];
      }
      if (lane == 0) sm.sig[parity][sn][0] = ss;
    };
    // chunk 0 is stored and the first S staged before the barrier below
    if (tid == 0) {
      sm.cnt[0] = 8;
      sm.cnt[1] = sm.cnt[2] = 1;
      sm.cnt[4] = sm.cnt[5] = sm.cnt[6] = sm.cnt[7] = 0;
    }
#pragma unroll
    for (int i8 = 0; i8 < 8; ++i8) Sacc[i8] = zero4();
    if (S0) {
#pragma unroll
      for (int i8 = 0; i8 < 8; ++i8) {
        const float4 s4 = *(const float4 *)(S0 + ((long)bh * 128 + jcol) * DK + 16 * i8 + 4 * g);
        Sacc[i8] = f32x4{s4.x, s4.y, s4.z, s4.w};
      }
    }
    stage_S(0);
    __syncthreads();

    for (int c = 0; c < NC; ++c) {
      const int cb = c & 1;
      lds_wait_geq(&sm.cnt[0], 8 * (c + 1));  // chunk c stored by every loader wave
      const f16 *Kc = sm.K[cb];
      const f16x8 *KtF = (const f16x8 *)(sm.rec[cb] + OFF_KTF);
      const f16x8 *TmA = (const f16x8 *)(sm.rec[cb] + OFF_TM);
      const float ds = *(const float *)(sm.rec[cb] + OFF_DS);
      // K S^T, then R = diag(beta)(V - K S^T) with the values turned into the
      // result layout (exactly: bf16 through the identity), then R / sr in fp16
      // with sr a power of two >= max |R| of the wave's channels
      f32x4 rf[4];
      // every operand read is issued before the first product, so that the
      // products do not wait on LDS latency one read at a time
      f16x8 ka[16];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ka[4 * m + kk] = ld8(&Kc[kq_chunk(16 * m + c16, 4 * kk + g)]);
      const uint4 Vv[2] = {sm.V[cb][sn][0][lane], sm.V[cb][sn][1][lane]};
      __builtin_amdgcn_sched_barrier(0);
      f32x4 ks[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        ks[m] = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) ks[m] = mma32(ka[4 * m + kk], Sb[kk], ks[m]);
      }
      // the operands of T R, on their way while R and its scale are formed
      f16x8 tm[6];
#pragma unroll
      for (int x = 0; x < 6; ++x) tm[x] = TmA[x * 64 + lane];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 a = ks[m];
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] *= ss;
        if (SCALED) {
          const f32x4 s4 = *(const f32x4 *)(sm.rec[cb] + OFF_KF + 4 * (16 * m + 4 * g));
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] *= s4[e];
        }
        const uint4 &vp = Vv[m >> 1];
        const bf16x4 vin = __builtin_bit_cast(bf16x4, (m & 1) ? uint2{vp.z, vp.w} : uint2{vp.x, vp.y});
        const f32x4 vv = mma16bf(vin, identb, zero4());
        const f32x4 b4 = *(const f32x4 *)&sm.b[cb][16 * m + 4 * g];
#pragma unroll
        for (int e = 0; e < 4; ++e) rf[m][e] = b4[e] * (vv[e] - a[e]);
      }
      // the S update's operands, on their way while R's scale and X are formed
      f16x8 kf[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) kf[x] = KtF[x * 64 + lane];
      __builtin_amdgcn_sched_barrier(0);
      float mr = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) mr = fmaxf(mr, fabsf(rf[m][e]));
      const float sr = pow2_above(wave_max(mr)), isr = pow2_inv(sr);
      f16x4 rr[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) rr[m][e] = h(rf[m][e] * isr);
      const f16x8 Rb[2] = {cat(rr[0], rr[1]), cat(rr[2], rr[3])};
      // X / sr = T (R / sr)
      f32x4 X[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f32x4 acc = zero4();
#pragma unroll
        for (int qq = 0; qq <= (m >> 1); ++qq) acc = mma32(tm[op_index(m, qq)], Rb[qq], acc);
        X[m] = acc;
      }
      const f16x8 Xb[2] = {cat(h4(X[0]), h4(X[1])), cat(h4(X[2]), h4(X[3]))};
      // X of chunk c - 2 and S at the start of chunk c - 1, in the slots written
      // below, are read by the output wave's pass c - 1
      lds_wait_geq(&sm.cnt[4 + sn], c);
      sm.Xx[cb][sn][0][lane] = Xb[0];
      sm.Xx[cb][sn][1][lane] = Xb[1];
      if (lane == 0) sm.sig[cb][sn][1] = sr;
      const float gL = GATED ? *(const float *)(sm.rec[cb] + OFF_GL) : 1.0f;
      // S^T <- gamma_L S^T + ds sr Kt^T (X / sr) (GK: row i of S^T decays by g_L[i])
      const float dsr = ds * sr;
#pragma unroll
      for (int i8 = 0; i8 < 8; ++i8) {
        f32x4 u = zero4();
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) u = mma32(kf[i8 * 2 + qq], Xb[qq], u);
        f32x4 gv = {gL, gL, gL, gL};
        if (GK) gv = *(const f32x4 *)(sm.rec[cb] + OFF_SC + 4 * (16 * i8 + 4 * g));
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Sacc[i8][e] = fmaf(dsr, u[e], (GATED || GK) ? gv[e] * Sacc[i8][e] : Sacc[i8][e]);
      }
      stage_S(cb ^ 1);
      lds_count(&sm.cnt[1 + sn], lane);
    }

    if (S_final) {
#pragma unroll
      for (int i8 = 0; i8 < 8; ++i8)
        *(float4 *)(S_final + ((long)bh * 128 + jcol) * DK + 16 * i8 + 4 * g) =
            float4{Sacc[i8][0], Sacc[i8][1], Sacc[i8][2], Sacc[i8][3]};
    }
    if (log_ratio_sum && tile == 0 && wave == 0) {
      // the chunks' sums of log rho_t, in a fixed order
      float acc = 0.f;
      for (int c = lane; c < NC; c += 64)
        acc += *(const float *)(ws + ((long)bh * NC + c) * (GK ? RECK : REC) + OFF_LR);
      acc = wave_sum(acc);
      if (lane == 0) log_ratio_sum[bh] = acc;
    }
  } else {
    // ================================ outputs ================================
    const int sn = wave - 2;
    f32x4 O[4];     // Q S^T of the chunk whose outputs are pending
    f16x8 Pr[6];    // its score operands
    __syncthreads();
    for (int it = 0; it <= NC; ++it) {
      // X of chunk it - 1 and S at the start of chunk it, from chain wave sn
      lds_wait_geq(&sm.cnt[1 + sn], it + 1);
      if (it > 0) {
        // O = Q S^T + P X of chunk it - 1, stored as bf16 through an identity
        // transpose (a lane then holds 4 consecutive channels of one token)
        const int c = it - 1;
        const long tok0 = (long)bh * T_ + (long)c * C;
        const int L = min(C, T_ - c * C);
        const f16x8 Xb[2] = {sm.Xx[c & 1][sn][0][lane], sm.Xx[c & 1][sn][1][lane]};
        // X is stored divided by sr: O = sr (Q S^T / sr + P (X / sr)).  The
        // four tiles are formed before any is stored, so that their products
        // overlap.  Both output waves stage their 16 channels in LDS; each then
        // stores 32 tokens of all 32 channels, 64 contiguous bytes a token (half
        // the write requests of 32-byte pieces)
        const float sr = sm.sig[c & 1][sn][1], isr = pow2_inv(sr);
        bf16 *stg = sm.Ost;
        f32x4 ot[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
          for (int e = 0; e < 4; ++e) O[m][e] *= isr;
#pragma unroll
          for (int qq = 0; qq <= (m >> 1); ++qq) O[m] = mma32(Pr[op_index(m, qq)], Xb[qq], O[m]);
#pragma unroll
          for (int e = 0; e < 4; ++e) O[m][e] *= sr;
          const bf16x4 ob = {(bf16)O[m][0], (bf16)O[m][1], (bf16)O[m][2], (bf16)O[m][3]};
          ot[m] = mma16bf(ob, identb, zero4());
        }
        // both output waves have read the staging of chunk c - 1 (count 2 (it - 1))
        lds_wait_geq(&sm.cnt[7], 2 * (it - 1));
#pragma unroll
        for (int m = 0; m < 4; ++m)
          *(bf16x4 *)&stg[(16 * m + c16) * OSP + 16 * sn + 4 * g] =
              bf16x4{(bf16)ot[m][0], (bf16)ot[m][1], (bf16)ot[m][2], (bf16)ot[m][3]};
        lds_count(&sm.cnt[6], lane);
        lds_wait_geq(&sm.cnt[6], 2 * it);  // both have staged chunk c
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int t = 32 * sn + 16 * j + (lane >> 2);
          const uint4 ov = *(const uint4 *)&stg[t * OSP + 8 * (lane & 3)];
          if (t < L) *(uint4 *)(o + (tok0 + t) * 128 + j0 + 8 * (lane & 3)) = ov;
        }
        lds_count(&sm.cnt[7], lane);
      }
      if (it < NC) {
        // Q S^T of chunk it from the S^T its chain wave left, and its scores
        lds_wait_geq(&sm.cnt[0], 8 * (it + 1));  // chunk it stored by every loader wave
        const int cb = it & 1;
        f16x8 Sb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) Sb[kk] = sm.Sx[cb][sn][kk][lane];
        const float ss = sm.sig[cb][sn][0];  // Sb holds S^T / ss
        const f16 *Qc = sm.Q[cb];
        f16x8 qa[16];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) qa[4 * m + kk] = ld8(&Qc[kq_chunk(16 * m + c16, 4 * kk + g)]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          f32x4 a = zero4();
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) a = mma32(qa[4 * m + kk], Sb[kk], a);
#pragma unroll
          for (int e = 0; e < 4; ++e) a[e] *= ss;
          if (SCALED) {
            const f32x4 s4 = *(const f32x4 *)(sm.rec[cb] + OFF_QF + 4 * (16 * m + 4 * g));
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] *= s4[e];
          }
          O[m] = a;
        }
        const f16x8 *PA = (const f16x8 *)(sm.rec[cb] + OFF_P);
#pragma unroll
        for (int x = 0; x < 6; ++x) Pr[x] = PA[x * 64 + lane];
      }
      lds_count(&sm.cnt[4 + sn], lane);
    }
  }
}

template <bool SCALED, bool GATED, bool GK>
__global__ void __launch_bounds__(ST)
chunk_state(const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
            const float *__restrict__ beta, const float *__restrict__ S0, int BH, int T_, int NC,
            const unsigned char *__restrict__ ws, bf16 *__restrict__ o,
            float *__restrict__ S_final, float *__restrict__ log_ratio_sum, unsigned xf) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  state_body<SCALED, GATED, GK, false>(smem_raw, blockIdx.x, q, k, v, beta, S0, BH, T_, NC, ws, o,
                                       S_final, log_ratio_sum, xf, nullptr, 0, 0);
}

// ---------------------------------------------------------------------------
// walk_state_pipe: the plain forward in one launch, for few heads (B*H at most
// an eighth of the compute units), where the walks, sequential over long
// sequences, would otherwise leave most of the device idle and the state pass
// after them would occupy only half of it.  The grid is the resident one
// (NRES workgroups, one per CU) followed by the 4 B*H state workgroups:
//   - workgroups 0 .. BH-1 walk (as in walk_pipe) and publish their results;
//   - the next NRES - BH prepare the walk's records (pipe_prep), which never
//     waits; then the first NRES - 5 BH of them run chunk_prep for every chunk
//     (chunk-major, three chunks a round, each once the walk has passed it),
//     publishing each record with device-scope stores and a flag, while the
//     other 4 B*H end, freeing their compute units;
//   - the state workgroups, dispatched after the resident ones onto the
//     compute units so freed, run the state pass (state_body), each chunk
//     once its record's flag is set.
// The walks wait only for the preparing workgroups, which never wait while
// they prepare the records; every other wait is for a workgroup dispatched
// earlier, and every wait is bounded.  So the launch needs only more of its
// workgroups resident at once than there are walks.
// Workspace: the chunk records (stride REC, as the split forward), wout, the
// walk's records (stride WREC), then three flags per chunk (the walk record
// ready, the walk past the chunk, the chunk record ready); each region is
// written once in a launch, so plain loads of a record after its flag see it.
// ---------------------------------------------------------------------------
constexpr size_t kStatePipeSmem =
    kTailSmem<false, false> > sizeof(StateSmem) ? kTailSmem<false, false> : sizeof(StateSmem);

__global__ void __launch_bounds__(wd::WT)
walk_state_pipe(const bf16 *__restrict__ q, const bf16 *__restrict__ k,
                const bf16 *__restrict__ v, const float *__restrict__ beta,
                const float *__restrict__ r, float eta, unsigned xf,
                unsigned char *__restrict__ ws, unsigned char *__restrict__ wrec,
                const float *__restrict__ d0, const float *__restrict__ S0, int T_, int NC,
                int BH, float *__restrict__ wout, float *__restrict__ d_final,
                float *__restrict__ log_ratio_sum, bf16 *__restrict__ o,
                float *__restrict__ S_final, unsigned long long *__restrict__ flags,
                unsigned long long epoch) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  constexpr int fstride = 3;
  const int NRES = (int)gridDim.x - 4 * BH, b = blockIdx.x;
  if (b < BH) {
    wd::walk_body<true, true>(smem_raw, b, k, wrec, WREC, d0, T_, NC, wout, d_final, nullptr,
                              log_ratio_sum, flags, fstride, epoch);
    return;
  }
  if (b >= NRES) {
    static_assert(ST == wd::WT, "the state pass runs in the walk's workgroup size");
    state_body<false, false, false, true>(smem_raw, b - NRES, q, k, v, beta, S0, BH, T_, NC, ws,
                                          o, S_final, nullptr, xf, flags + 2, fstride, epoch);
    return;
  }
  const int j = b - BH, NPW = NRES - BH;
  wd::pipe_prep(smem_raw, j, NPW, BH, k, beta, r, eta, xf, wrec, WREC, T_, NC, flags, fstride,
                epoch);
  const int PT = NPW - 4 * BH;  // the workgroups that go on with chunk_prep
  if (j >= PT) return;
  const int inst = threadIdx.x >> 8;
  TailLds<false, false> &Ld = reinterpret_cast<TailLds<false, false> *>(smem_raw)[inst];
  const int total = BH * NC;
  bool gave_up = false;  // once a wait ran out, later items do not wait
  // round m of workgroup j: items 3 m + inst, m = j, j + PT, ...
  for (int m = j; 3 * m < total; m += PT) {
    const int ii = min(3 * m + inst, total - 1);
    const int c = ii / BH, bh = ii % BH;
    // the walk past chunk c (a bounded wait)
    bool ok = false;
    const unsigned long long *f = &flags[((long)bh * NC + c) * fstride + 1];
    for (int i = 0; !gave_up && i < wd::kPollLimit; ++i) {
      if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch) {
        ok = true;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
    gave_up = !ok;
    // (the thread index through an opaque copy each round, so that the
    // compiler does not hoist the body's lane-dependent addresses out of the
    // loop and keep them live across it)
    int tid = threadIdx.x & 255;
    asm volatile("" : "+v"(tid));
    chunk_prep_body<kOsdn, false, false, false, true, true>(
        Ld, tid, bh, c, !ok, q, k, nullptr, beta, T_, NC, ws, r, wout, nullptr, xf,
        &flags[((long)bh * NC + c) * fstride + 2], epoch);
    __syncthreads();  // the next round's staging overwrites this round's LDS
  }
}

}  // namespace

size_t split_workspace_bytes(int B, int H, int T, bool gate_channels) {
  const long nc = (T + C - 1) / C;
  return (size_t)B * H * nc * (gate_channels ? RECK : REC);
}

namespace {

template <bool SCALED, bool GATED, bool GK>
hipError_t launch_state_t(const ChunkArgs &a, int NC, const void *ws, float *log_ratio_sum,
                          hipStream_t s) {
  const int BH = a.B * a.H;
  const size_t shm = sizeof(StateSmem);
  hipError_t e = hipFuncSetAttribute((const void *)chunk_state<SCALED, GATED, GK>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((chunk_state<SCALED, GATED, GK>), dim3((unsigned)(BH * 4)), dim3(ST), shm, s,
                     (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v, a.beta, a.S0, BH,
                     a.T, NC, (const unsigned char *)ws, (bf16 *)a.o, a.S_final, log_ratio_sum,
                     a.xf);
  return hipGetLastError();
}

bool per_channel(const float *alpha, unsigned xf) { return alpha && (xf & kGateChannels); }

// the record carries row factors when q, k arrive unnormalised or a gate is
// given; with the per-channel gate it carries K (.) G, Q (.) G and g_L instead
hipError_t launch_state(const ChunkArgs &a, int NC, const void *ws, float *log_ratio_sum,
                        hipStream_t s) {
  if (per_channel(a.alpha, a.xf)) return launch_state_t<false, false, true>(a, NC, ws, log_ratio_sum, s);
  if (a.alpha) return launch_state_t<true, true, false>(a, NC, ws, log_ratio_sum, s);
  if (a.xf & kNormQK) return launch_state_t<true, false, false>(a, NC, ws, log_ratio_sum, s);
  return launch_state_t<false, false, false>(a, NC, ws, log_ratio_sum, s);
}

template <int MODE, bool NORM, bool GATED, bool GK>
void launch_prep_t(int BH, int NC, int nck, hipStream_t s, const void *q, const void *k,
                   const void *kt, const float *beta, int T, unsigned char *rec, const float *r,
                   const float *wout, const float *alpha, unsigned xf) {
  if (nck <= 0) return;
  hipLaunchKernelGGL((chunk_prep<MODE, NORM, GATED, GK>), dim3((unsigned)(BH * nck)), dim3(256), 0,
                     s, (const bf16 *)q, (const bf16 *)k, (const bf16 *)kt, beta, T, NC, BH, rec, r,
                     wout, alpha, xf);
}

// chunk_prep over the last nck chunks (all by default) of every head; kGiven
// takes no input transforms
template <int MODE>
hipError_t launch_prep(int BH, int NC, hipStream_t s, const void *q, const void *k,
                       const void *kt, const float *beta, int T, unsigned char *rec,
                       const float *r, const float *wout, const float *alpha, unsigned xf,
                       int nck = -1) {
  if (NC <= 0) return hipSuccess;
  if (nck < 0) nck = NC;
  constexpr bool TX = MODE != kGiven;  // instances with the input transforms
  const bool norm = TX && (xf & kNormQK);
  if (per_channel(alpha, xf)) {
    if (norm)
      launch_prep_t<MODE, TX, false, true>(BH, NC, nck, s, q, k, kt, beta, T, rec, r, wout, alpha, xf);
    else
      launch_prep_t<MODE, false, false, true>(BH, NC, nck, s, q, k, kt, beta, T, rec, r, wout, alpha, xf);
  } else if (norm && alpha) {
    launch_prep_t<MODE, TX, true, false>(BH, NC, nck, s, q, k, kt, beta, T, rec, r, wout, alpha, xf);
  } else if (norm) {
    launch_prep_t<MODE, TX, false, false>(BH, NC, nck, s, q, k, kt, beta, T, rec, r, wout, alpha, xf);
  } else if (alpha) {
    launch_prep_t<MODE, false, true, false>(BH, NC, nck, s, q, k, kt, beta, T, rec, r, wout, alpha, xf);
  } else {
    launch_prep_t<MODE, false, false, false>(BH, NC, nck, s, q, k, kt, beta, T, rec, r, wout, alpha, xf);
  }
  return hipGetLastError();
}

}  // namespace

// Heads up to which the forward may run in one launch (walk_state_pipe): an
// eighth of MI355X's 256 compute units.  The launch itself also checks the
// device's count.
constexpr int kStatePipeHeads = 32;

size_t split_forward_workspace_bytes(int B, int H, int T, bool gate_channels) {
  // the walk's records live in the space the chunk records take later; with
  // few heads they get their own space after wout, then three flags per chunk
  // (walk_state_pipe)
  const size_t nc = (size_t)((T + C - 1) / C), BH = (size_t)B * H;
  size_t n = BH * nc * ((gate_channels ? RECK : REC) + WOUT * sizeof(float));
  if (!gate_channels && BH <= (size_t)kStatePipeHeads) n += BH * nc * (WREC + 3 * sizeof(unsigned long long));
  return n;
}

// walk_prep, the walk's sequential pass, chunk_prep forming the write keys
// from the walk's results, the state kernel -- in that order on one stream.
// (Running chunk_prep of finished segments beside the walk on a second stream
// was measured: the cross-stream waits and the sharing of CUs ate the overlap.)
// How many of every head's first chunks walk_chunk_pipe prepares: what its
// preparing workgroups can do between finishing the walk's records and the
// walks' end.  In units of a round of preparation (three chunks per
// workgroup, about 8 us on MI355X; the walk takes about 1.05 us a chunk and
// about 10 us to start), less one round of margin.
int tail_chunks(int BH, int NC, int cus) {
#ifdef OSDN_TAIL_CHUNKS
  return min(OSDN_TAIL_CHUNKS, max(NC - 2, 0));
#else
  const int npw = cus - BH;
  const double round_us = 8.0, walk_us = 10.0 + 1.05 * NC;
  const double prep_rounds = (double)BH * NC / (3.0 * npw);
  const double tail_rounds = walk_us / round_us - prep_rounds - 1.0;
  if (tail_rounds <= 0) return 0;
  return min((int)(tail_rounds * 3.0 * npw / BH), max(NC - 2, 0));
#endif
}

template <bool NORM, bool GATED>
hipError_t launch_walk_chunk_pipe(const FusedArgs &a, unsigned char *rec, float *wout, int NC,
                                  int ncp, int BH, int cus, hipStream_t s) {
  constexpr size_t shm = kTailSmem<NORM, GATED>;
  hipError_t e = hipFuncSetAttribute((const void *)walk_chunk_pipe<NORM, GATED>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((walk_chunk_pipe<NORM, GATED>), dim3((unsigned)cus), dim3(wd::WT), shm, s,
                     (const bf16 *)a.q, (const bf16 *)a.k, a.beta, a.r, a.eta, a.xf, rec, a.d0,
                     a.T, NC, ncp, BH, wout, a.d_final, a.log_ratio_sum, a.alpha, next_epoch());
  return hipGetLastError();
}

hipError_t launch_split_forward(const FusedArgs &a, void *ws, hipStream_t s) {
  const int BH = a.B * a.H;
  if (BH == 0) return hipSuccess;
  const int NC = (a.T + C - 1) / C;
  unsigned char *rec = (unsigned char *)ws;
  const size_t rb = per_channel(a.alpha, a.xf) ? RECK : REC;
  float *wout = (float *)(rec + (size_t)BH * NC * rb);
  static_assert(WREC <= REC && REC <= RECK, "walk records fit in the chunk records' space");
  ChunkArgs ca{a.q, a.k, nullptr, a.v, a.beta, a.alpha, a.S0, a.B, a.H, a.T, a.dk, a.dv, a.chunk,
               a.dtype, a.o, a.S_final, a.xf};
  if (a.precond_off) {  // the plain delta rule (Gated DeltaNet with alpha): kt = k
    hipError_t e = launch_prep<kDeltaNet>(BH, NC, s, a.q, a.k, nullptr, a.beta, a.T, rec, nullptr,
                                          nullptr, a.alpha, a.xf);
    if (e != hipSuccess) return e;
    return launch_state(ca, NC, ws, a.log_ratio_sum, s);
  }
  // the gate leaves the preconditioner walk unchanged
  ScanArgs sa{a.k, a.beta, a.r, a.d0, a.eta, a.B, a.H, a.T, a.dk, a.dtype, 0, nullptr,
              a.d_final, nullptr, nullptr, a.log_ratio_sum, a.xf};
  // The walk's records take the chunk records' slots (stride REC), each with
  // its ready flag and its walked flag past it: chunk_prep overwrites a slot
  // only once the walk is done with it.
  static_assert(WREC % 8 == 0 && REC - WREC >= 16, "the flags fit past a walk record");
  unsigned long long *flags = (unsigned long long *)(rec + WREC);
  const int cus = device_cus();
  if (NC > 0 && !a.alpha && !(a.xf & kNormQK) && BH <= kStatePipeHeads && 8 * BH <= cus) {
    // the whole forward in one launch (the workspace has the space for it)
    unsigned char *wr = (unsigned char *)(wout + (size_t)BH * NC * WOUT);
    unsigned long long *fl = (unsigned long long *)(wr + (size_t)BH * NC * WREC);
    hipError_t e = hipFuncSetAttribute((const void *)walk_state_pipe,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)kStatePipeSmem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(walk_state_pipe, dim3((unsigned)(cus + 4 * BH)), dim3(wd::WT),
                       kStatePipeSmem, s, (const bf16 *)a.q, (const bf16 *)a.k, (const bf16 *)a.v,
                       a.beta, a.r, a.eta, a.xf, rec, wr, a.d0, a.S0, a.T, NC, BH, wout,
                       a.d_final, a.log_ratio_sum, (bf16 *)a.o, a.S_final, fl, next_epoch());
    return hipGetLastError();
  }
  const bool one_launch = NC > 0 && 2 * BH <= cus;
  const int ncp = one_launch && !per_channel(a.alpha, a.xf) ? tail_chunks(BH, NC, cus) : 0;
  hipError_t e;
  if (ncp > 0) {
    const bool norm = (a.xf & kNormQK) != 0, gated = a.alpha != nullptr;
    e = norm ? (gated ? launch_walk_chunk_pipe<true, true>(a, rec, wout, NC, ncp, BH, cus, s)
                      : launch_walk_chunk_pipe<true, false>(a, rec, wout, NC, ncp, BH, cus, s))
             : (gated ? launch_walk_chunk_pipe<false, true>(a, rec, wout, NC, ncp, BH, cus, s)
                      : launch_walk_chunk_pipe<false, false>(a, rec, wout, NC, ncp, BH, cus, s));
  } else {
    e = launch_walk(sa, rec, REC, wout, s, flags, (int)(REC / 8));
  }
  if (e != hipSuccess) return e;
  e = launch_prep<kOsdn>(BH, NC, s, a.q, a.k, nullptr, a.beta, a.T, rec, a.r, wout, a.alpha, a.xf,
                         NC - ncp);
  if (e != hipSuccess) return e;
  return launch_state(ca, NC, ws, nullptr, s);
}

hipError_t launch_split_chunk(const ChunkArgs &a, bool given, void *ws, hipStream_t s) {
  const int BH = a.B * a.H;
  if (BH == 0) return hipSuccess;
  const int NC = (a.T + C - 1) / C;
  unsigned char *rec = (unsigned char *)ws;
  const unsigned xf = a.xf & kGateChannels;  // the only flag the given-keys pass takes
  hipError_t e = given ? launch_prep<kGiven>(BH, NC, s, a.q, a.k, a.k_tilde, a.beta, a.T, rec,
                                             nullptr, nullptr, a.alpha, xf)
                       : launch_prep<kDeltaNet>(BH, NC, s, a.q, a.k, nullptr, a.beta, a.T, rec,
                                                nullptr, nullptr, a.alpha, xf);
  if (e != hipSuccess) return e;
  ChunkArgs b = a;
  b.xf = xf;
  return launch_state(b, NC, ws, nullptr, s);
}

}  // namespace osdn
