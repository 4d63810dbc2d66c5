// Device code of the preconditioner walk shared by the launches that run it
// (walk.hip) and by the forward pipeline that runs the walk together with
// the chunk-parallel pass (chunk_split.hip): the per-chunk preparation of the
// walk's records and the sequential walk itself.  Everything here is inline,
// a template or constexpr, so that every translation unit may include it.
#pragma once

#include "device.h"
#include "mfma.h"
#include "walk.h"

namespace osdn {
namespace wd {

constexpr int C = 64;
constexpr int DK = 128;
constexpr int KP = 136;  // padded row (halves) of [64][128] tiles in LDS
constexpr int FP = 68;   // padded row (floats) of [64][64] fp32 tiles in LDS
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The maximum over each aligned group of 8 lanes (DPP); every lane of the
// group receives it.
__device__ __forceinline__ float group_max8(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  return v;
}

// ---------------------------------------------------------------------------
// walk_prep: the record of one (b, h, chunk), formed by 4 waves (tid 0..255
// of the caller's 256 threads).  Every thread of the workgroup takes part in
// the same barriers, so several instances may share a workgroup as long as
// each runs this once per round.  COH: the record is written with device-scope
// stores (sc1), which reach memory without an L2 writeback, so that another
// workgroup of the same launch can read it with device-scope loads once a
// flag says it is complete; `store` false computes without writing.
// ---------------------------------------------------------------------------
struct alignas(16) PrepSmem {
  // The fp16 squared keys are needed only for the key gram; (I + M)^-1 reuses
  // their space.
  float F[C * FP];                // key gram G, then M (strictly lower)
  unsigned char KM[C * KP * 2];   // fp16 p_t / e_t^2, then (I + M)^-1 [64][FP]
  float Yw[3][16][17];            // per-wave staging of a block sum
  float bs[C], al[C], nn[C], lg[C + 4];
  float ss[C];  // 1 / ||k_t||^2 for unnormalised keys, else 1
  float e2[C];  // e_t^2: the square of row t's staging scale
};
static_assert(C * KP * 2 >= C * FP * 4, "the inverse fits in the keys' space");

// a buffer resource over n bytes at p (raw buffer: offsets in bytes; accesses
// past n read zero and write nothing)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_over(const void *p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, n, 0x00020000);
}
constexpr int kSc1 = 16;  // cache policy of a device-scope (sc1) buffer access

// The global loads of one chunk (prep_load), apart from the rest so that a
// caller can issue the next chunk's while it works on this one: beta and r of
// token `lane` (the log-gate scan needs only these), beta of the two rows the
// thread stages, then their keys: row t = (tid >> 3) + 32 u, keys 8 (tid & 7)
// + 64 j .. +7 for j = 0, 1 (the 8 threads of a row read, and write to LDS,
// 128 contiguous bytes per j).  Rows past the end reread the last row and are
// zeroed when staged.
struct PrepIn {
  float pb, pr, rb[2];
  uint4 rk[2][2];
};

__device__ __forceinline__ PrepIn prep_load(const int tid, const int bh, const int c,
                                            const bf16 *__restrict__ k,
                                            const float *__restrict__ beta,
                                            const float *__restrict__ r, int T_) {
  PrepIn in;
  const long tok0 = (long)bh * T_ + (long)c * C;
  const int L = min(C, T_ - c * C);
  const int tb = min(tid & 63, L - 1);
  in.pb = beta[tok0 + tb];
  in.pr = r ? r[tok0 + tb] : 1.0f;
#pragma unroll
  for (int u = 0; u < 2; ++u) in.rb[u] = beta[tok0 + min((tid >> 3) + 32 * u, L - 1)];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = min((tid >> 3) + 32 * u, L - 1);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      in.rk[u][j] = *(const uint4 *)(k + (tok0 + t) * DK + 8 * (tid & 7) + 64 * j);
  }
  return in;
}

// staged(): called by every thread right after the barrier that ends the
// staging.  COH: every wave's earlier global stores are complete at that
// barrier (a caller writes the previous chunk's flag from staged()).
template <bool COH, typename Staged>
__device__ __forceinline__ void prep_chunk(PrepSmem &sm, const PrepIn &in, const int tid,
                                           const int bh, const int c, const bool store,
                                           const float *__restrict__ r, float eta, int T_, int NC,
                                           unsigned xf, unsigned char *__restrict__ wrec,
                                           size_t rstride, Staged &&staged) {
  float *F = sm.F;
  float(*Yw)[16][17] = sm.Yw;
  float *bs = sm.bs, *al = sm.al, *nn = sm.nn, *lg = sm.lg, *ss = sm.ss, *e2 = sm.e2;
  f16 *Ph = (f16 *)sm.KM;
  float *Mi = (float *)sm.KM;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c16 = lane & 15, g = lane >> 4;
  const int L = min(C, T_ - c * C);
  float pb = in.pb, pr = in.pr;
  const float *rb = in.rb;
  const uint4(*rk)[2] = in.rk;
  if (xf & kGateLogits) {
    pb = sigmoid_gate(pb);
    pr = sigmoid_gate(pr);
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

  // stage p_t = k_t (.) k_t of the stored keys divided by e_t^2, with e_t a
  // power of two >= the row's largest |k|, in fp16: (k / e_t)^2 is exact in
  // fp32 (8 significant bits squared), so this is the one rounding the fp16
  // product of two fp16 copies of k / e_t would make, done once per row
  // instead of once per gram tile.  Entry (t, s) of the key gram then carries
  // 1 / (e_t^2 e_s^2), put back in fp32 when M is formed.  n_t from the stored
  // bf16 values (8 threads per token), and alpha_t with it.  Unnormalised keys
  // enter through the fp32 factor 1 / n_t on p_t (the normalised key's p is
  // p_t / n_t).
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int t = (tid >> 3) + 32 * u, i0 = 8 * (tid & 7);
    const bool ok = t < L;
    float x[16], sq = 0.f, mk = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const unsigned short *s = (const unsigned short *)&rk[u][j];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[8 * j + e] = bf2f(s[e]);
        sq = fmaf(x[8 * j + e], x[8 * j + e], sq);
        mk = fmaxf(mk, fabsf(x[8 * j + e]));
      }
    }
    sq = group_sum<8>(ok ? sq : 0.f);
    const float er = pow2_above(group_max8(mk));
    const float ie = pow2_inv(er);
    const f16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f16x8 ph;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = x[8 * j + e] * ie;
        ph[e] = h(y * y);
      }
      *(f16x8 *)&Ph[t * KP + i0 + 64 * j] = ok ? ph : z8;  // a padded row stages zeros
    }
    if ((tid & 7) == 0) {
      const float sc = (xf & kNormQK) ? (sq > 0.f ? 1.0f / sq : 0.f) : 1.0f;
      const float bt = ok ? ((xf & kGateLogits) ? sigmoid_gate(rb[u]) : rb[u]) : 0.f;
      const float n = sq * sc;  // ||k_t||^2 of the key the recurrence sees
      ss[t] = sc;
      nn[t] = n;
      al[t] = n > 0.f ? eta * bt / n : 0.f;
      e2[t] = er * er;
    }
  }
  if (COH) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  staged();

  // lower tiles of the key gram G = P P^T with P = k (.) k in fp16, turned into
  // M in the result registers: M_ts = beta_t alpha_s R_{t,s} s_t s_s e_t^2 e_s^2 G_ts
  // for s < t, zero on and above the diagonal.  Wave w forms tiles w, w + 4 and
  // w + 8 of the ten; waves 2 and 3 run a third pass on tile 9 whose entries
  // go to their own rows of Yw (unused until the off-diagonal blocks), so that
  // every pass is the same branch-free code: each tile's vectors are read
  // before its products and the next tile's operands while its entries are
  // formed.
  {
    f16x8 opa[4], opb[4];
    auto read_ops = [&](int job) {
      int rt, ct;
      tri_tile(min(job, 9), rt, ct);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        opa[kk] = ld8(&Ph[(16 * rt + c16) * KP + 32 * kk + 8 * g]);
        opb[kk] = ld8(&Ph[(16 * ct + c16) * KP + 32 * kk + 8 * g]);
      }
    };
    read_ops(wave);
#pragma unroll
    for (int pass = 0; pass < 3; ++pass) {
      const int job = wave + 4 * pass;
      int rt, ct;
      tri_tile(min(job, 9), rt, ct);
      const int s = 16 * ct + c16, t0 = 16 * rt + 4 * g;
      const float als = al[s], lgs = lg[s + 1], sss = ss[s], e2s = e2[s];
      const float4 b4 = *(const float4 *)&bs[t0], l4 = *(const float4 *)&lg[t0];
      const float4 s4 = *(const float4 *)&ss[t0], x4 = *(const float4 *)&e2[t0];
      f32x4 acc = zero4();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mma32(opa[kk], opb[kk], acc);
      if (pass < 2) read_ops(job + 4);
      const float bt[4] = {b4.x, b4.y, b4.z, b4.w}, lt[4] = {l4.x, l4.y, l4.z, l4.w};
      const float st[4] = {s4.x, s4.y, s4.z, s4.w}, et[4] = {x4.x, x4.y, x4.z, x4.w};
      float *dst = job < 10 ? &F[t0 * FP + s] : &Yw[wave - 2][0][0] + 4 * lane;
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // (above the diagonal R may overflow: not stored)
        const float m = bt[e] * als * fexp2(lt[e] - lgs) * (st[e] * sss) * ((et[e] * e2s) * acc[e]);
        dst[job < 10 ? e * FP : e] = s < t0 + e ? m : 0.f;
      }
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

  // the record: the inverse's ten 16x16 blocks on and below the diagonal (the
  // walk reads no other; piece q: block q >> 6, row (q >> 2) & 15, columns
  // 4 (q & 3) .. +3), then the vectors
  if (!store) return;
  unsigned char *rec = wrec + ((long)bh * NC + c) * rstride;
  const __amdgpu_buffer_rsrc_t rr = rsrc_over(rec, (int)WREC);
  auto put = [&](float v, size_t off) {
    if (COH)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rr, (int)off, 0, kSc1);
    else
      *(float *)(rec + off) = v;
  };
  for (int q = tid; q < 640; q += 256) {
    int bi, bj;
    tri_tile(q >> 6, bi, bj);
    const int row = 16 * bi + ((q >> 2) & 15), col = 16 * bj + 4 * (q & 3);
    const float4 m = *(const float4 *)&Mi[row * FP + col];
    const size_t off = W_MINV + 4 * (size_t)(row * C + col);
    if (COH)
      __builtin_amdgcn_raw_buffer_store_b128(
          u32x4{__float_as_uint(m.x), __float_as_uint(m.y), __float_as_uint(m.z), __float_as_uint(m.w)},
          rr, (int)off, 0, kSc1);
    else
      *(float4 *)(rec + off) = m;
  }
  if (tid < C) {
    const int t = tid;
    put(bs[t] * fexp2(lg[t]), W_U + 4 * t);
    put(al[t], W_A + 4 * t);
    put(t < L ? fexp2(lg[C] - lg[t + 1]) * al[t] : 0.f, W_WA + 4 * t);
    put(ss[t], W_S + 4 * t);
  }
  if (tid == 0) put(fexp2(lg[C]), W_GL);
}


// ---------------------------------------------------------------------------
// walk: one workgroup of 12 waves per (b, h), sequential over the chunks from
// the entry d0 (ones if none is given), three barriers per chunk.  Waves 0-3
// run the chain, reading p_t = k_t (.) k_t in fp32 from LDS:
//   A  b_t = <d, p_t> (4 threads per token), rhs_t = 1 - u_t s_t b_t
//   B  g = (I + M)^-1 rhs (4 threads per token); c_t, w_t = R_{L,t} alpha_t s_t g_t
//   C  d <- Gamma_L d + sum_t w_t p_t: wave v takes dimensions 32 v .. +31, its
//      two lane halves one half of the tokens each, joined by a lane-half swap;
//      lane l < 32 keeps d of its dimension in a register; then log rho_t
// Waves 4-11 keep the chain fed: they load the keys and the record four
// chunks ahead (four register sets: a load has over two iterations to
// arrive) and square the keys into p (fp32) as they store them, so that none
// of this sits on the chain.
// ---------------------------------------------------------------------------
constexpr int PS = 144;  // row (floats) of p in LDS: 16 dwords past a multiple of 64
                         // spreads the 16-byte reads of phase A over all banks
constexpr int WT = 768;  // threads: the chain (waves 0-3), the loaders (waves 4-11)
constexpr int NLD = WT - 256;  // loader lanes
// Column of key dimension i in a row of p: 16-byte halves of each 32-byte piece
// swapped in the pieces whose index has bit 2 set.  The loaders then store the
// first half of every piece with one instruction and the 8 lanes of each LDS
// write clock still cover distinct banks.
__device__ __forceinline__ int p_slot(int i) { return i ^ ((i >> 3) & 4); }

struct alignas(16) WalkSmem {
  float P[2][C * PS];        // p_t = k_t (.) k_t
  float Mi[2][C * FP];       // (I + M)^-1
  float vec[2][4][C];        // u = beta Gamma, alpha, R_{L,t} alpha, the 1/||k||^2 factor
  float gL[2][4];            // Gamma_L
  float pad[4];              // where loader lanes without a record piece store
  float d[DK];               // entry d of the chunk in the pass
  float rhs[C], w[C], g[C];
  int bad;                   // set if a record never became ready (PIPE)
};

// Bound on the polls of a record's ready flag (each a memory round trip plus
// a sleep: about a third of a second in all); the protocol sets every flag
// within the time the records take to prepare.  A wave gives up at most once.
constexpr int kPollLimit = 1 << 18;

// The walk of head bh; the record of chunk c at wrec + (bh NC + c) rstride.
// PIPE: the records are written by other workgroups of the same launch while
// the walk runs; flags[(bh NC + c) fstride] holds `epoch` once the record of
// chunk c is complete, and the records are read with device-scope loads (see
// prep_chunk).  PUB: the walk's results (wout) are written with device-scope
// stores for other workgroups of the launch, and flags[(bh NC + c) fstride +
// 1] is set to `epoch` once those of chunk c are complete.
template <bool PIPE, bool PUB>
__device__ __forceinline__ void walk_body(unsigned char *smem_raw, const int bh,
                                          const bf16 *__restrict__ k,
                                          const unsigned char *__restrict__ wrec, size_t rstride,
                                          const float *__restrict__ d0, int T_, int NC,
                                          float *__restrict__ wout, float *__restrict__ d_final,
                                          float *__restrict__ log_ratio,
                                          float *__restrict__ log_ratio_sum,
                                          unsigned long long *__restrict__ flags, int fstride,
                                          unsigned long long epoch) {
  WalkSmem &sm = *reinterpret_cast<WalkSmem *>(smem_raw);
  const int tid = threadIdx.x;
  if (PIPE) {
    if (tid == 0) sm.bad = 0;
    __syncthreads();
  }

  if (tid >= 256) {
    // ================================ loaders ================================
    // a chunk: 1024 pieces of 8 keys (2 per lane) and the record as 705
    // pieces of 16 bytes: the inverse's ten 16x16 blocks on and below the
    // diagonal (piece q: block q >> 6, row (q >> 2) & 15, columns 4 (q & 3)
    // .. +3), then 64 of the vectors and Gamma_L.  The blocks above the
    // diagonal are zero in both LDS buffers from the start and never written.
    const int lt = tid - 256;
    constexpr int NMI = 640, RP = NMI + 65;
    constexpr int NRP = (RP + NLD - 1) / NLD;
    struct Regs {
      uint4 k[2], rr[NRP];
    };
    Regs ra, rb, rc, rd;
    // Piece q's byte offsets in the record and in the WalkSmem of buffer buf
    // (the pad past the last piece).  Arithmetic only: the loaders take no
    // divergent branch, whose two paths would leave the loads in flight
    // differently and make the waits after them drain every load.
    auto rec_off = [&](int q) {
      int bi, bj;
      tri_tile(min(q >> 6, 9), bi, bj);
      const int mi = (int)W_MINV + 4 * ((16 * bi + ((q >> 2) & 15)) * C + 16 * bj + 4 * (q & 3));
      return q < NMI ? mi : (int)W_U + 16 * (q - NMI);  // the vectors, then Gamma_L
    };
    auto lds_off = [&](int q, int buf) {
      int bi, bj;
      tri_tile(min(q >> 6, 9), bi, bj);
      const int v = q - NMI;  // 16 pieces per vector
      const int mi = (int)offsetof(WalkSmem, Mi) +
                     4 * (buf * C * FP + (16 * bi + ((q >> 2) & 15)) * FP + 16 * bj + 4 * (q & 3));
      const int ve = (int)offsetof(WalkSmem, vec) + 4 * (buf * 4 * C + (v >> 4) * C + (v & 15) * 4);
      const int gv = (int)offsetof(WalkSmem, gL) + 16 * buf;
      return q < NMI ? mi : q < RP - 1 ? ve : q == RP - 1 ? gv : (int)offsetof(WalkSmem, pad);
    };
    // chunk cc clamped to the last one: loads past it reread it
    auto load = [&](Regs &R, int cc) {
      cc = min(cc, NC - 1);
      const bf16 *kc = k + ((long)bh * T_ + (long)cc * C) * DK;  // uniform base, 32-bit offsets
      const int L = min(C, T_ - cc * C);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = lt + NLD * u, tt = min(p >> 4, L - 1);
        R.k[u] = *(const uint4 *)(kc + tt * DK + (p & 15) * 8);
      }
      const unsigned char *rs = wrec + ((long)bh * NC + cc) * rstride;
      const __amdgpu_buffer_rsrc_t rr = rsrc_over(rs, (int)WREC);
#pragma unroll
      for (int u = 0; u < NRP; ++u) {
        const int off = rec_off(min(lt + NLD * u, RP - 1));
        if (PIPE) {
          const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rr, off, 0, kSc1);
          R.rr[u] = uint4{x.x, x.y, x.z, x.w};
        } else {
          R.rr[u] = *(const uint4 *)(rs + off);
        }
      }
    };
    // PIPE: wait until the records of chunks 0 .. cc are all ready (a
    // wave-uniform call).  `ready` counts the chunks from 0 known to be
    // ready; each poll reads the flags of the 64 chunks from there on.  false
    // if the bound ran out, then and in every later call.
    int ready = 0;
    bool gave_up = false;
    auto await = [&](int cc) {
      cc = min(cc, NC - 1);
      if (gave_up) return false;
      const int lane = tid & 63;
      const unsigned long long *f = flags + (long)bh * NC * fstride;
      for (int i = 0; i < kPollLimit; ++i) {
        if (cc < ready) return true;
        const unsigned long long v =
            __hip_atomic_load(f + (long)min(ready + lane, NC - 1) * fstride, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
        const unsigned long long set = __ballot(v == epoch);
        ready += ~set == 0ull ? 64 : __builtin_ctzll(~set);
        if (cc < ready) return true;
        __builtin_amdgcn_s_sleep(8);
      }
      gave_up = true;
      return false;
    };
    // the record of chunk cc into LDS buffer cc & 1.  PIPE: once a record was
    // missing, the lane that stores Gamma_L overwrites it with NaN, so that d
    // and everything after it turn NaN (a branch around an LDS store only:
    // one around a loaded register would make the loads' waits drain them).
    auto stash_rec = [&](const Regs &R, int cc) {
      const int buf = cc & 1;
#pragma unroll
      for (int u = 0; u < NRP; ++u)
        *(uint4 *)(smem_raw + lds_off(lt + NLD * u, buf)) = R.rr[u];
      static_assert(NRP == 2 && RP - 1 >= NLD, "Gamma_L is the second piece of one lane");
      if (PIPE && lt == RP - 1 - NLD && sm.bad != 0) sm.gL[buf][0] = __uint_as_float(0x7fc00000u);
    };
    // piece u of the keys of chunk cc (tokens 32 u .. +31), squared, into LDS
    // buffer cc & 1 (rows past the end zero), in the p_slot layout
    auto stash_p = [&](const Regs &R, int cc, int u) {
      const int buf = cc & 1, L = min(C, T_ - cc * C);
      const int p = lt + NLD * u, tt = p >> 4, i0 = (p & 15) * 8;
      const unsigned short *s = (const unsigned short *)&R.k[u];
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = bf2f(s[e]);
        x[e] = tt < L ? y * y : 0.f;
      }
      float *row = &sm.P[buf][tt * PS];
      *(float4 *)(row + p_slot(i0)) = float4{x[0], x[1], x[2], x[3]};
      *(float4 *)(row + p_slot(i0 + 4)) = float4{x[4], x[5], x[6], x[7]};
    };
    // one iteration, its work spread so that no window outlasts the chain's
    // phase: the record of chunk c+1 and half its keys (window A), the other
    // half (window B), the loads of chunk c+4 into the set that held chunk c
    // (window C).  The loaders store nothing to global memory: a store would
    // share the load counter, whose waits then could no longer count the
    // loads in flight and would drain them.
    // (Unconditional: past the last chunk the stores put the last chunk's
    // reread record and zero keys into a buffer that only the chain's idle
    // iterations read.  A conditional iteration would leave the loads in
    // flight differently on its two paths, and the waits after them would
    // then drain every load.)
    // PIPE: loader wave 4 alone makes sure that chunk c+4's record is ready
    // before the barrier after which all loaders load it (a poll waits for
    // the wave's loads in flight; the other loader waves keep theirs).
    auto iteration = [&](int c, Regs &free_, const Regs &next) {
      stash_rec(next, c + 1);
      stash_p(next, c + 1, 0);
      __syncthreads();
      stash_p(next, c + 1, 1);
      if (PIPE && (tid >> 6) == 4 && !await(c + 4)) sm.bad = 1;
      __syncthreads();
      load(free_, c + 4);
      __syncthreads();
    };
    // zeros into the six blocks above the diagonal of both buffers (768 pieces)
    for (int i = lt; i < 2 * 6 * 64; i += NLD) {
      int bi, bj;
      off_tile((i >> 6) % 6, bj, bi);  // (bj, bi) below the diagonal: (bi, bj) above it
      *(float4 *)&sm.Mi[i / 384][(16 * bi + ((i >> 2) & 15)) * FP + 16 * bj + 4 * (i & 3)] =
          float4{0.f, 0.f, 0.f, 0.f};
    }
    if (NC > 0) {
      // PIPE: every loader wave waits for the first four records itself
      if (PIPE && !await(3)) sm.bad = 1;
      load(ra, 0);
      load(rb, 1);
      load(rc, 2);
      load(rd, 3);
      stash_rec(ra, 0);
      stash_p(ra, 0, 0);
      stash_p(ra, 0, 1);
    }
    __syncthreads();
    for (int c = 0; c < NC; c += 4) {
      iteration(c, ra, rb);
      iteration(c + 1, rb, rc);
      iteration(c + 2, rc, rd);
      iteration(c + 3, rd, ra);
    }
    if (PUB) __syncthreads();  // the chain's last barrier
    return;
  }

  // ================================= chain ==================================
  // The operands from the chunk's LDS buffers (p, the inverse, the per-token
  // factors) are read into registers ahead of their phase, right after an
  // earlier phase's own reads (B's and C's in phase A, which has time to
  // spare while the loaders store, the next chunk's A in phase C): a phase
  // then waits only for the vector it contracts with (d, rhs or w), which the
  // previous phase wrote.
  // PUB: device-scope stores of the results, and the flag that says chunk cc's
  // are complete
  auto put_out = [&](float *p, float v) {
    if (PUB)
      __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *p = v;
  };
  auto walked = [&](int cc) {
    __hip_atomic_store(&flags[((long)bh * NC + cc) * fstride + 1], epoch, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  };
  const int t = tid >> 2, part = tid & 3;       // phases A and B
  const int wv = tid >> 6, l = tid & 63;
  const int dim = 32 * wv + (l & 31), half = l >> 5;  // phase C
  float dreg = 0.f;  // lanes l < 32: d of dimension dim, entry value of the chunk in the pass
  if (half == 0) {
    dreg = d0 ? d0[(long)bh * DK + dim] : 1.0f;
    if (NC > 0) put_out(&wout[(long)bh * NC * WOUT + dim], dreg);
    sm.d[dim] = dreg;
  }
  float pa[32];    // A: p_t at dimensions 4 (part + 4 j) .. +3
  float mr[16];    // B: row t of (I + M)^-1, columns 16 part .. +15
  float pcol[32];  // C: p of tokens 8 j + 4 half + e at dimension dim
  float ut = 0.f, sta = 0.f;            // A: u_t, s_t
  float wa = 0.f, stb = 0.f, at = 0.f;  // B: R_{L,t} alpha_t, s_t, alpha_t
  float gl = 0.f;                       // C: Gamma_L
  float lr_acc = 0.f;  // wave 0: sum of log rho_t over token tid
  auto read_a = [&](int cb) {
    const float *pr = &sm.P[cb][t * PS];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 p4 = *(const float4 *)(pr + p_slot(4 * (part + 4 * j)));
      pa[4 * j] = p4.x, pa[4 * j + 1] = p4.y, pa[4 * j + 2] = p4.z, pa[4 * j + 3] = p4.w;
    }
    ut = sm.vec[cb][0][t];
    sta = sm.vec[cb][3][t];
  };
  auto read_b = [&](int cb) {
    const float *mrow = &sm.Mi[cb][t * FP + 16 * part];
#pragma unroll
    for (int j = 0; j < 16; j += 4) {
      const float4 m4 = *(const float4 *)(mrow + j);
      mr[j] = m4.x, mr[j + 1] = m4.y, mr[j + 2] = m4.z, mr[j + 3] = m4.w;
    }
    wa = sm.vec[cb][2][t];
    stb = sm.vec[cb][3][t];
    at = sm.vec[cb][1][t];
  };
  // tokens 8 j + 4 half + e of C's operand for j in [j0, j0 + 4)
  auto read_c = [&](int cb, int j0) {
    const float *pc = &sm.P[cb][p_slot(dim)];
#pragma unroll
    for (int j = j0; j < j0 + 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) pcol[4 * j + e] = pc[(8 * j + 4 * half + e) * PS];
    gl = sm.gL[cb][0];
  };
  __syncthreads();
  if (NC > 0) read_a(0);

  // whole groups of four chunks, as the loaders run; past the last chunk an
  // iteration changes no d and stores nothing
  const int NC4 = (NC + 3) & ~3;
  for (int c = 0; c < NC4; ++c) {
    const int cb = c & 1;
    // PUB: chunk c-1 issued at least two stores per wave (its c_t and the next
    // entry d), so once at most two are pending those of chunk c-2 are
    // complete; the flag goes out after the barrier that follows
    if (PUB && c >= 2 && c < NC) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    // A
    {
      float4 dv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) dv[j] = *(const float4 *)&sm.d[4 * (part + 4 * j)];
      __builtin_amdgcn_sched_barrier(0);
      read_b(cb);
      read_c(cb, 0);
      read_c(cb, 4);
      __builtin_amdgcn_sched_barrier(0);
      float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        b0 = fmaf(dv[j].x, pa[4 * j], b0);
        b1 = fmaf(dv[j].y, pa[4 * j + 1], b1);
        b2 = fmaf(dv[j].z, pa[4 * j + 2], b2);
        b3 = fmaf(dv[j].w, pa[4 * j + 3], b3);
        b0 = fmaf(dv[j + 1].x, pa[4 * j + 4], b0);
        b1 = fmaf(dv[j + 1].y, pa[4 * j + 5], b1);
        b2 = fmaf(dv[j + 1].z, pa[4 * j + 6], b2);
        b3 = fmaf(dv[j + 1].w, pa[4 * j + 7], b3);
      }
      const float b = group_sum<4>((b0 + b1) + (b2 + b3));
      if (part == 0) sm.rhs[t] = 1.0f - ut * (sta * b);
    }
    __syncthreads();
    if (PUB && tid == 0 && c >= 2 && c < NC) walked(c - 2);
    // B
    {
      float4 rv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) rv[j] = *(const float4 *)&sm.rhs[16 * part + 4 * j];
      float ga = 0.f, gb = 0.f, gc = 0.f, gd = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ga = fmaf(mr[4 * j], rv[j].x, ga);
        gb = fmaf(mr[4 * j + 1], rv[j].y, gb);
        gc = fmaf(mr[4 * j + 2], rv[j].z, gc);
        gd = fmaf(mr[4 * j + 3], rv[j].w, gd);
      }
      const float gt = group_sum<4>((ga + gb) + (gc + gd));
      if (part == 0) {
        sm.w[t] = wa * gt * stb;
        sm.g[t] = gt;
        if (c < NC) put_out(&wout[((long)bh * NC + c) * WOUT + DK + t], at * gt);
      }
    }
    __syncthreads();
    // C: tokens 8 j + 4 half + e of dimension dim
    {
      float4 wv4[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) wv4[j] = *(const float4 *)&sm.w[8 * j + 4 * half];
      __builtin_amdgcn_sched_barrier(0);
      read_a(cb ^ 1);  // past the last chunk: a stale buffer, never used
      __builtin_amdgcn_sched_barrier(0);
      float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        a0 = fmaf(wv4[j].x, pcol[4 * j], a0);
        a1 = fmaf(wv4[j].y, pcol[4 * j + 1], a1);
        a2 = fmaf(wv4[j].z, pcol[4 * j + 2], a2);
        a3 = fmaf(wv4[j].w, pcol[4 * j + 3], a3);
      }
      const float a = (a0 + a1) + (a2 + a3);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a),
                                                       false, false);
      const float sum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      if (half == 0 && c < NC) {
        dreg = fmaf(gl, dreg, sum);
        sm.d[dim] = dreg;
        if (c + 1 < NC) put_out(&wout[((long)bh * NC + c + 1) * WOUT + dim], dreg);  // next entry d
      }
      // log rho_t = log g_t^2 of the chunk (g from phase B), wave 0; the
      // hardware logarithm (about one ulp of log2)
      if (tid < C && tid < min(C, T_ - c * C)) {
        const float gt = sm.g[tid];
        const float lr = __logf(gt * gt);
        lr_acc += lr;
        if (log_ratio) log_ratio[(long)bh * T_ + (long)c * C + tid] = lr;
      }
    }
    __syncthreads();
  }
  if (PUB) {  // the last two chunks' flags (the loaders meet this barrier too)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      for (int cc = max(NC - 2, 0); cc < NC; ++cc) walked(cc);
  }
  if (log_ratio_sum && tid < 64) {
    const float s = wave_sum(lr_acc);
    if (tid == 0) log_ratio_sum[bh] = s;
  }

  if (d_final && half == 0) d_final[(long)bh * DK + dim] = dreg;
}

// The LDS of a one-launch walk: the walk's, or three preparing instances'
constexpr size_t kPipeSmem = sizeof(WalkSmem) > 3 * sizeof(PrepSmem) ? sizeof(WalkSmem)
                                                                       : 3 * sizeof(PrepSmem);

// The preparing workgroup j of NPW in a launch whose first BH workgroups walk:
// three chunks at a time (one per 256 threads, in lockstep), in the order the
// walks read them: chunk-major from chunk 0, heads innermost, workgroup j
// taking rounds j, j + NPW, ... of 3 NPW chunks.  A finished record is
// announced by writing `epoch` (a value no earlier call used) to
// flags[(bh NC + c) fstride].  It never waits for anything.  Returns the
// number of rounds it ran (a caller may go on with rounds of other items).
__device__ __forceinline__ int pipe_prep(unsigned char *smem_raw, const int j, const int NPW,
                                          const int BH, const bf16 *__restrict__ k,
                                          const float *__restrict__ beta,
                                          const float *__restrict__ r, float eta, unsigned xf,
                                          unsigned char *__restrict__ wrec, size_t rstride, int T_,
                                          int NC, unsigned long long *__restrict__ flags,
                                          int fstride, unsigned long long epoch) {
  // instance inst takes waves 4 inst .. +3; its wave roles are rotated by
  // inst, so that the waves with the most work in the inverse's later levels
  // (roles 0 and 1) of the three instances sit on different SIMDs (waves w,
  // w + 4 and w + 8 of a workgroup share one)
  const int inst = threadIdx.x >> 8;
  const int it = ((((threadIdx.x >> 6) & 3) + inst) & 3) * 64 + (threadIdx.x & 63);
  PrepSmem &ps = reinterpret_cast<PrepSmem *>(smem_raw)[inst];
  const int total = BH * NC;
  // Round q takes chunks 3 (NPW q + j) + inst: chunk-major, heads innermost.
  auto item_of = [&](int q) { return 3 * (NPW * q + j) + inst; };
  auto busy = [&](int q) { return 3 * (NPW * q + j) < total; };
  auto locate = [&](int item, int &bh_, int &c_) {
    const int ii = min(item, total - 1);  // past the last chunk: reread it, store nothing
    c_ = ii / BH;
    bh_ = ii % BH;
  };
  int bh, c, pbh = 0, pc = 0;
  bool pvalid = false;  // the previous round's chunk, whose flag is still to be written
  locate(item_of(0), bh, c);
  PrepIn cur = prep_load(it, bh, c, k, beta, r, T_), nxt;
  int rounds = 0;
  for (int q = 0; busy(q); ++q, ++rounds) {
    const int item = item_of(q);
    const bool valid = item < total;
    locate(item, bh, c);
    // Once this round's staging is done, the previous round's record stores
    // are complete (prep_chunk waits for them before that barrier): its flag
    // goes out, and the next round's loads.
    prep_chunk<true>(ps, cur, it, bh, c, valid, r, eta, T_, NC, xf, wrec, rstride, [&] {
      if (pvalid && it == 0)
        __hip_atomic_store(&flags[((long)pbh * NC + pc) * fstride], epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      int nbh, ncc;
      locate(item_of(q + 1), nbh, ncc);
      nxt = prep_load(it, nbh, ncc, k, beta, r, T_);
    });
    cur = nxt;
    // the record's stores read the inverse and the vectors from LDS, which the
    // next round's staging overwrites: every wave is past them first.  The
    // first round's flags go out at once: the walks are waiting for them.
    if (q == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (q == 0) {
      if (valid && it == 0)
        __hip_atomic_store(&flags[((long)bh * NC + c) * fstride], epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
      pvalid = valid;
      pbh = bh;
      pc = c;
    }
  }
  // the last round's flag
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (pvalid && it == 0)
    __hip_atomic_store(&flags[((long)pbh * NC + pc) * fstride], epoch, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  return rounds;
}

}  // namespace wd
}  // namespace osdn
