// Layout of the preconditioner walk's scratch records (walk.hip), shared with
// the chunk-parallel pass that reads the walk's results (chunk_split.hip).
#pragma once

#include <stddef.h>

namespace osdn {

// Per (b, h, chunk of 64 tokens), written by walk_prep and read by walk:
//   W_MINV  fp32 [64][64]  (I + M)^-1, row-major; only its ten 16x16 blocks on
//                          and below the diagonal are written (and read)
//   W_U     fp32 [64]      beta_t Gamma_t
//   W_A     fp32 [64]      alpha_t = eta beta_t / n_t (0 if n_t = 0)
//   W_WA    fp32 [64]      R_{L,t} alpha_t (0 past the end of the sequence)
//   W_S     fp32 [64]      1 / ||k_t||^2 when the keys come unnormalised, else 1:
//                          p_t of the normalised key is W_S[t] (k_t (.) k_t)
//   W_GL    fp32           Gamma_L
constexpr size_t WREC = 17664;
constexpr size_t W_MINV = 0, W_U = 16384, W_A = 16640, W_WA = 16896, W_S = 17152, W_GL = 17408;

// Per (b, h, chunk), written by walk: the chunk's entry preconditioner d [128]
// then c_t = alpha_t g_t [64], fp32.
constexpr int WOUT = 192;

}  // namespace osdn
