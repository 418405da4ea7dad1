// Chunked prefill of the CCQ read step on a Gated DeltaNet backbone (gfx950): the kernels.  Included
// by ccq_prefill_gdn.hip (main kernel, scans, launch) and ccq_prefill_gdn_summary.hip (segment
// summary), which the build compiles with different scheduler settings.
//
// Method (gist.science summary of arXiv 2606.01294, §2 "理论推导", §2 "机制", §2 "集成"):
// the cleaned query qc_t = q_t - lambda_t Sigma_t q_t replaces q_t in the read o_t = S_t qc_t,
// the write rule is left as it is.  The Gated DeltaNet write rule (standard definition) is
//   S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  alpha_t = exp(g_t), scalar.
//
// Chunk algebra (rows i = 0..63 of a chunk, carry S0; gamma_i = prod_{j<=i} alpha_j inside the
// chunk, Gam_ij = gamma_i / gamma_j).  With delta_t = beta_t (v_t - alpha_t S_{t-1} k_t) the rule
// reads S_t = alpha_t S_{t-1} + delta_t k_t^T, so S_i = gamma_i S0 + sum_{j<=i} Gam_ij delta_j k_j^T
// and the deltas of a chunk solve a unit lower-triangular system:
//   (I + A) Delta = X,   A_ij = beta_i Gam_ij k_i . k_j (j < i),   X = diag(beta) (V - diag(gamma) K S0^T)
//   O   = diag(gamma) Qc S0^T + (tril_incl(Qc K^T) * Gam) Delta
//   S_L = gamma_L S0 + Delta^T diag(gamma_L / gamma) K
// The CCQ statistics part (gate, Q K^T, Q C0, cleaned query) is the rule-independent code in
// ccq_prefill_common.hpp; C0 += K^T K, m0 += sum k, n0 += L as for every rule.
//
// Segments.  S_L is affine in S0: S_L = S0 M_c + b_c with M_c = gamma_L I - W^T diag(gamma_L /
// gamma) K (W = (I + A)^{-1} diag(beta gamma) K) and b_c the S_L of a zero S0.  A run of chunks
// therefore maps S_in to S_in M_seg + dS_seg, where dS_seg is the run's S from zero and M_seg
// is the same recurrence applied to a d_k x d_k state that starts at I with v = 0 (then X and
// b_c carry no v term).  With more than one segment per chain, gdn_summary_kernel computes
// (dS, dC, dksum) and M for every segment but the last, gdn_scan_state_kernel chains
// S_in[p+1] = S_in[p] M_p + dS_p in fp32, gdn_scan_sum_kernel adds up C and ksum, and the
// main kernel runs every segment from its carry-in.
//
// Kernel layout.  One workgroup of D/16 waves per (chain, segment); wave w owns the 16 value
// channels [16w, 16w + 16): its tiles of C and S^T live in MFMA accumulators (as in the GLA
// kernel), and so do its columns of X and Delta, held as Delta[j][v] tiles (token rows).  The
// triangular system is solved in fp32 by 16-token blocks: the inverses of the four diagonal
// blocks (I + A_bb)^{-1} come from forward substitution (one lane per column), then every wave
// runs Delta_b = (I + A_bb)^{-1} (X_b - sum_{b' < b} A_bb' Delta_b') on its own columns with
// fp32 MFMAs, the off-diagonal blocks of A read from LDS.  Products on bf16 operands with fp32
// accumulation: K S0^T, Qc S0^T, the intra term and the carry update; the intra matrix Qc K^T
// takes qc as bf16 hi + lo.
#pragma once

#include "ccq_internal.hpp"
#include "ccq_prefill_common.hpp"

namespace ccq {

// Workspace slot of one (chain, segment): S [D][D] | C [D][D] | ksum [D] | M [D][D], fp32.
__host__ __device__ static inline size_t gdn_slot_floats(int d) { return 3 * (size_t)d * d + d; }

template <int D, typename T>
struct GdnSmem {
  using C_ = Cfg<D, T>;
  T Qs[kL][C_::PQ];        // q rows
  T Ks[2][kL][C_::PQ];     // k rows of chunk c in Ks[c % 2]; the other half receives chunk c + 1
  T Vs[kL][C_::PQ];        // v rows
  T Qa[kL][C_::PQ];        // cleaned query (hi part for bf16)
  T Qalo[C_::LO][C_::PQ];  // bf16 only: lo part of the cleaned query
  T Pm[kL][C_::PT];        // tril(Q K^T - c 1^T), then M = tril(Qc K^T) * Gam
  T Wt[4][C_::PQ];         // w_lambda hi, lo; key sum hi, lo
  float As[kL][kL + 4];    // A_ij = beta_i Gam_ij k_i . k_j below the diagonal (lower tiles only)
  float Tb[4][16][16 + 4]; // (I + A_bb)^{-1} of the four diagonal 16-token blocks
  float m0[D], m1[D];
  float lgam[kL], beta[kL];  // chunk-local log gamma_i, beta_i
  float gam[kL], gdec[kL];   // gamma_i = e^{lgam_i} and gamma_L / gamma_i = e^{lgam_L - lgam_i}
  f32x4 tok[kL];             // lambda, 1/n, sq/n^2, gate logit + b
};

// ---------------------------------------------------------------- steps shared by the kernels

// Wave 1: chunk-local log gamma (inclusive scan over lanes = tokens), beta, and the per-token
// factors gamma_i and gamma_L / gamma_i into LDS (formed once here rather than by every lane
// that scales by them).
template <int D, typename T>
__device__ __forceinline__ void gdn_gates(GdnSmem<D, T>& sm, float sg, float sb, int lane) {
  float x = sg;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  sm.lgam[lane] = x;
  sm.beta[lane] = sb;
  sm.gam[lane] = __expf(x);
  sm.gdec[lane] = __expf(__shfl(x, kL - 1, 64) - x);
}

// A = beta Gam (K K^T) below the diagonal, lower 16x16 tiles idx = i0, i0 + step, ... < 10.
template <int D, typename T>
__device__ __forceinline__ void gdn_build_A(GdnSmem<D, T>& sm, const T (*Ks)[Cfg<D, T>::PQ], int i0, int step,
                                            int lane) {
  using C_ = Cfg<D, T>;
  constexpr int NK = C_::NK, PQ = C_::PQ;
  const int g = lane >> 4, l16 = lane & 15;
  for (int idx = i0; idx < 10; idx += step) {
    const int ti = tri_row(idx), tj = tri_col(idx);
    f32x4 acc = zero4();  // k_j . k_i at j = 16 tj + 4 g + r, i = 16 ti + l16
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const Frag<T> A = lds_frag<T, KORD_CONTIG>(&Ks[0][0], PQ, 16 * tj, 32 * kk, lane);
      const Frag<T> B = lds_frag<T, KORD_CONTIG>(&Ks[0][0], PQ, 16 * ti, 32 * kk, lane);
      mma(acc, A, B);
    }
    const int i = 16 * ti + l16, j0 = 16 * tj + 4 * g;
    const float lgi = sm.lgam[i], bi = sm.beta[i];
    const f32x4 lgj = *reinterpret_cast<const f32x4*>(&sm.lgam[j0]);
    f32x4 av;
#pragma unroll
    for (int r = 0; r < 4; ++r) av[r] = (j0 + r < i) ? bi * __expf(lgi - lgj[r]) * acc[r] : 0.f;
    *reinterpret_cast<f32x4*>(&sm.As[i][j0]) = av;
  }
}

// Key sums m1 = m0 + sum_t k_t: 2D threads (rel = 0 .. 2D - 1), two per channel, 32 tokens each.
template <int D, typename T>
__device__ __forceinline__ void gdn_key_sums(GdnSmem<D, T>& sm, const T (*Ks)[Cfg<D, T>::PQ], int rel) {
  const int c = rel >> 1, half = rel & 1;
  float s = 0.f;
#pragma unroll 8
  for (int t = 32 * half; t < 32 * half + 32; ++t) s += to_f32(Ks[t][c]);
  s += __shfl_xor(s, 1, 64);
  if (half == 0) sm.m1[c] = sm.m0[c] + s;
}

// One wave: (I + A_bb)^{-1} for the four diagonal blocks in fp32.  Lane (block, i) holds row i
// of A_bb and of the inverse T, starting from T_i = e_i; for each pivot k the 16 lanes of a
// block receive row k of T (final by then) and the rows below it apply T_i -= A_ik T_k, which
// is forward substitution of T (I + A_bb) = I row by row.  About 20 registers per lane.
template <int D, typename T>
__device__ __forceinline__ void gdn_diag_inverse(GdnSmem<D, T>& sm, int lane) {
  const int blk = lane >> 4, i = lane & 15, base = 16 * blk;
  float trow[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) trow[j] = (j == i) ? 1.f : 0.f;
#pragma unroll
  for (int k = 0; k < 15; ++k) {
    const float coef = (i > k) ? sm.As[base + i][base + k] : 0.f;
#pragma unroll
    for (int j = 0; j <= k; ++j) {  // row k of T is zero right of column k
      const float tk = __shfl(trow[j], k, 16);
      trow[j] -= coef * tk;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<f32x4*>(&sm.Tb[blk][i][4 * q]) = f32x4{trow[4 * q], trow[4 * q + 1], trow[4 * q + 2], trow[4 * q + 3]};
}

// One wave: (I + A_bb)^{-1} of diagonal block blk in fp32 with MFMAs.  N = A_bb is strictly lower
// triangular, so N^16 = 0 and (I + N)^{-1} = sum_k (-N)^k = (I - N)(I + N^2)(I + N^4)(I + N^8): three
// squarings and three products, 24 v_mfma_f32_16x16x4_f32 in a chain four products deep, instead of a
// 15-step forward substitution.  Every product takes its B operand straight from the accumulators of
// the previous one (element r of lane (g, l) is X[4 g + r][l], the B layout of k-slice r) and its A
// operand from LDS: the powers are written to Tb[blk] (which receives the inverse at the end) and to an
// upper block of As, which the kernels never use (A is strictly lower triangular).  The LDS traffic
// stays inside the wave, whose LDS instructions complete in order, so no barrier is needed.
__device__ __forceinline__ void diag_block_inverse_mfma(float (*As)[kL + 4], float (*Tb)[16][20], int blk, int lane) {
  const int g = lane >> 4, l = lane & 15, base = 16 * blk;
  constexpr int PA = kL + 4;
  const float* N = &As[base][base];
  float* s1 = &Tb[blk][0][0];                                              // pitch 20
  // upper blocks (0,1) (0,2) (0,3) (1,2) for blocks 0..3
  float* s2 = &As[blk == 3 ? 16 : 0][blk == 3 ? 32 : 16 * (blk + 1)];      // pitch PA
  auto mm = [&](const float* X, int px, const f32x4& y, f32x4 acc) {        // acc + X Y
#pragma unroll
    for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[l * px + 4 * g + r], y[r], acc, 0, 0, 0);
    return acc;
  };
  auto put = [&](float* X, int px, const f32x4& v) {
#pragma unroll
    for (int r = 0; r < 4; ++r) X[(4 * g + r) * px + l] = v[r];
  };
  f32x4 n1, e;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    n1[r] = N[(4 * g + r) * PA + l];
    e[r] = (4 * g + r == l ? 1.f : 0.f) - n1[r];  // I - N
  }
  const f32x4 n2 = mm(N, PA, n1, zero4());
  put(s1, 20, n2);
  e = mm(s1, 20, e, e);                     // (I - N)(I + N^2)
  const f32x4 n4 = mm(s1, 20, n2, zero4());
  put(s2, PA, n4);
  e = mm(s2, PA, e, e);                     // ... (I + N^4)
  const f32x4 n8 = mm(s2, PA, n4, zero4());
  put(s1, 20, n8);
  e = mm(s1, 20, e, e);                     // ... (I + N^8)
  put(s1, 20, e);
}
template <int D, typename T>
__device__ __forceinline__ void gdn_diag_inverse_mfma(GdnSmem<D, T>& sm, int blk, int lane) {
  diag_block_inverse_mfma(sm.As, sm.Tb, blk, lane);
}

// X = beta (V - gamma K S0^T) on the wave's 16 state rows (WITH_V false: V = 0).  X[b][r] at
// token 16 b + 4 g + r, state row cw + l16; stile(t) is the tile S^T[16 t + 4 g + r][cw + l16].
template <int D, typename T, bool WITH_V, typename STile>
__device__ __forceinline__ void gdn_rhs(const GdnSmem<D, T>& sm, const T (*Ks)[Cfg<D, T>::PQ], STile stile, int cw,
                                        int lane, f32x4 (&X)[4]) {
  using C_ = Cfg<D, T>;
  constexpr int NK = C_::NK, PQ = C_::PQ;
  const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int b = 0; b < 4; ++b) X[b] = zero4();
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const Frag<T> Bs = acc_frag<T>(stile(2 * kk), stile(2 * kk + 1));  // S0^T, own columns
#pragma unroll
    for (int b = 0; b < 4; ++b) mma(X[b], lds_frag<T, KORD_ACC>(&Ks[0][0], PQ, 16 * b, 32 * kk, lane), Bs);
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int j0 = 16 * b + 4 * g;
    const f32x4 gm = *reinterpret_cast<const f32x4*>(&sm.gam[j0]);
    const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[j0]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = WITH_V ? to_f32(sm.Vs[j0 + r][cw + l16]) : 0.f;
      X[b][r] = bt[r] * (v - gm[r] * X[b][r]);
    }
  }
}

// Delta = (I + A)^{-1} X by 16-token blocks on the wave's columns:
//   Delta_b = T_b (X_b - sum_{b' < b} A_bb' Delta_b'),  T_b = (I + A_bb)^{-1}  (in sm.Tb),
// fp32 operands (A and T from LDS, Delta in the accumulators).
// fp32 tiles: v_mfma_f32_16x16x4_f32, one K-slice of 4 per instruction.
template <int D, typename T>
__device__ __forceinline__ void gdn_solve_f32(const GdnSmem<D, T>& sm, const f32x4 (&X)[4], int lane, f32x4 (&Dl)[4]) {
  const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    f32x4 Z = X[b];
#pragma unroll
    for (int bp = 0; bp < b; ++bp) {
      const f32x4 a4 = *reinterpret_cast<const f32x4*>(&sm.As[16 * b + l16][16 * bp + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) Z = __builtin_amdgcn_mfma_f32_16x16x4f32(-a4[r], Dl[bp][r], Z, 0, 0, 0);
    }
    const f32x4 t4 = *reinterpret_cast<const f32x4*>(&sm.Tb[b][l16][4 * g]);
    Dl[b] = zero4();
#pragma unroll
    for (int r = 0; r < 4; ++r) Dl[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(t4[r], Z[r], Dl[b], 0, 0, 0);
  }
}

// bf16 hi + lo split of 8 fp32 values (x0 then x1, negated when NEG) into a KORD_ACC fragment
// pair: elements 0..3 from x0, 4..7 from x1.
template <bool NEG>
__device__ __forceinline__ void split_hl(const f32x4& x0, const f32x4& x1, Frag<__bf16>& h, Frag<__bf16>& l) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float v = NEG ? -(e < 4 ? x0[e] : x1[e - 4]) : (e < 4 ? x0[e] : x1[e - 4]);
    h.v[e] = (__bf16)v;
    l.v[e] = (__bf16)(v - (float)h.v[e]);
  }
}

// The same for NR right-hand sides at once on bf16 tiles: every product is three
// v_mfma_f32_16x16x32_bf16 on hi + lo splits of its fp32 operands (hi.hi + hi.lo + lo.hi, about
// 16 significant bits, against 8 for a plain bf16 product), with two 16-token blocks of the
// reduction per instruction: a third of the matrix-core time of the fp32 form.  The systems
// share the split A and T fragments, and their chains interleave.  KORD_ACC pairs: A's element
// e of lane (g, i) is A[16 b + i][16 p0 + 4 g + e] (e < 4) or [16 p1 + 4 g + e - 4]; Delta's is
// Delta[16 p0 + 4 g + e][i] or [16 p1 + 4 g + e - 4][i], exactly the accumulator rows of blocks
// p0 and p1.
template <int D, typename T, int NR>
__device__ __forceinline__ void gdn_solve_n(const GdnSmem<D, T>& sm, const f32x4 (&X)[NR][4], int lane,
                                            f32x4 (&Dl)[NR][4]) {
  if constexpr (sizeof(T) != 2) {
#pragma unroll
    for (int r = 0; r < NR; ++r) gdn_solve_f32<D, T>(sm, X[r], lane, Dl[r]);
  } else {
    const int g = lane >> 4, l16 = lane & 15;
    Frag<T> Bh[NR][2], Bl[NR][2];  // Delta pairs (0, 1) and (2, -), hi and lo, as blocks complete
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        Bh[r][p].v = bf16x8{};
        Bl[r][p].v = bf16x8{};
      }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f32x4 Z[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) Z[r] = X[r][b];
#pragma unroll
      for (int pr = 0; 2 * pr < b; ++pr) {  // block pairs with a block before b: -A_b,pair Delta_pair
        const int p0 = 2 * pr, p1 = 2 * pr + 1;
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(&sm.As[16 * b + l16][16 * p0 + 4 * g]);
        const f32x4 a1 = p1 < b ? *reinterpret_cast<const f32x4*>(&sm.As[16 * b + l16][16 * p1 + 4 * g]) : zero4();
        Frag<T> Ah, Al;
        split_hl<true>(a0, a1, Ah, Al);
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          mma(Z[r], Ah, Bh[r][pr]);
          mma(Z[r], Ah, Bl[r][pr]);
          mma(Z[r], Al, Bh[r][pr]);
        }
      }
      Frag<T> Th, Tl;
      split_hl<false>(*reinterpret_cast<const f32x4*>(&sm.Tb[b][l16][4 * g]), zero4(), Th, Tl);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        Frag<T> zh, zl;
        split_hl<false>(Z[r], zero4(), zh, zl);
        Dl[r][b] = zero4();
        mma(Dl[r][b], Th, zh);
        mma(Dl[r][b], Th, zl);
        mma(Dl[r][b], Tl, zh);
        if (b < 3) {  // into half b % 2 of pair b / 2
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = Dl[r][b][e];
            const __bf16 hv = (__bf16)v;
            Bh[r][b / 2].v[4 * (b % 2) + e] = hv;
            Bl[r][b / 2].v[4 * (b % 2) + e] = (__bf16)(v - (float)hv);
          }
        }
      }
    }
  }
}

template <int D, typename T>
__device__ __forceinline__ void gdn_solve(const GdnSmem<D, T>& sm, const f32x4 (&X)[4], int lane, f32x4 (&Dl)[4]) {
  gdn_solve_n<D, T, 1>(sm, *reinterpret_cast<const f32x4(*)[1][4]>(&X), lane, *reinterpret_cast<f32x4(*)[1][4]>(&Dl));
}

// S^T = gamma_L S^T + K^T diag(gamma_L / gamma) Delta on the wave's state tiles.
template <int D, typename T, typename STileM>
__device__ __forceinline__ void gdn_state_update(const GdnSmem<D, T>& sm, const T (*Ks)[Cfg<D, T>::PQ],
                                                 STileM stile, const f32x4 (&Dl)[4], int lane) {
  using C_ = Cfg<D, T>;
  constexpr int NA = C_::NA, PQ = C_::PQ;
  const int g = lane >> 4;
  const float gL = sm.gam[kL - 1];
#pragma unroll
  for (int t = 0; t < NA; ++t) stile(t) *= gL;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    f32x4 d0 = Dl[2 * kk], d1 = Dl[2 * kk + 1];
    d0 *= *reinterpret_cast<const f32x4*>(&sm.gdec[32 * kk + 4 * g]);
    d1 *= *reinterpret_cast<const f32x4*>(&sm.gdec[32 * kk + 16 + 4 * g]);
    const Frag<T> Bd = acc_frag<T>(d0, d1);  // diag(gamma_L / gamma) Delta, own columns
#pragma unroll
    for (int t = 0; t < NA; ++t) mma(stile(t), tr_frag_acc<T>(&Ks[0][0], PQ, 32 * kk, 16 * t, lane), Bd);
  }
}

// C += K^T K on the wave's tiles.
template <int D, typename T>
__device__ __forceinline__ void gdn_cov_update(const T (*Ks)[Cfg<D, T>::PQ], f32x4 (&Cacc)[Cfg<D, T>::NA], int cw,
                                               int lane) {
  using C_ = Cfg<D, T>;
  constexpr int NA = C_::NA, PQ = C_::PQ;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const Frag<T> Bk = tr_frag<T>(&Ks[0][0], PQ, 32 * kk, cw, lane);  // K[t][own channel]
#pragma unroll
    for (int t = 0; t < NA; ++t) mma(Cacc[t], tr_frag<T>(&Ks[0][0], PQ, 32 * kk, 16 * t, lane), Bk);
  }
}

// ---------------------------------------------------------------- main kernel

// CC: this instantiation writes the carry at every chunk start (FwdArgs::chunk_carry).
template <int D, typename T, bool CC>
__global__ __launch_bounds__(4 * D) void gdn_main_kernel(FwdArgs a) {
  using C_ = Cfg<D, T>;
  constexpr int NW = C_::NW, NA = C_::NA, NK = C_::NK;
  constexpr int PQ = C_::PQ, PT = C_::PT;
  constexpr bool kSplit = sizeof(T) == 2;
  __shared__ GdnSmem<D, T> sm;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, and known to be so
  const int cw = 16 * w;  // this wave's 16 channels
  const int P = a.segments, cps = a.chunks_per_segment;
  const int chain = blockIdx.x / P, seg = blockIdx.x % P;
  const int h = chain % a.H;
  const int nchunks = (a.T + kL - 1) / kL;
  const int cbeg = seg * cps;
  const int cend = min(nchunks, cbeg + cps);
  const size_t tok0 = (size_t)chain * (size_t)a.T;
  const T* qg = static_cast<const T*>(a.q);
  const T* kg = static_cast<const T*>(a.k);
  const T* vg = static_cast<const T*>(a.v);
  const T* gg = static_cast<const T*>(a.log_alpha);
  const T* bg = static_cast<const T*>(a.beta);

  // ---- carry in: the segment's slot for segments 1.., else the caller's carry (or zeros)
  // the caller's C0 / C_out may be the packed upper triangle (the workspace slots never are)
  const bool cpacked = (a.flags & kFlagPackedCov) != 0;
  constexpr size_t kTri = (size_t)D * (D + 1) / 2;
  const float* Sin = nullptr;
  const float* Cin = nullptr;
  const float* min_ = nullptr;
  bool cin_packed = false;
  if (P > 1 && (seg > 0 || a.snapshot)) {  // slot 0 holds a copy of the caller's carry when the carry out overlaps it
    const float* slot = static_cast<const float*>(a.workspace) + ((size_t)chain * P + seg) * gdn_slot_floats(D);
    Sin = slot;
    Cin = slot + (size_t)D * D;
    min_ = slot + 2 * (size_t)D * D;
  } else if (a.S0 != nullptr) {
    Sin = a.S0 + (size_t)chain * D * D;
    cin_packed = cpacked;
    Cin = a.C0 + (size_t)chain * (cpacked ? kTri : (size_t)D * D);
    min_ = a.ksum0 + (size_t)chain * D;
  }
  f32x4 Cacc[NA], Sacc[NA];
  {
    const int row = cw + l16;
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      const int col = 16 * t + 4 * g;
      Sacc[t] = Sin ? *reinterpret_cast<const f32x4*>(Sin + (size_t)row * D + col) : zero4();
      if (Cin == nullptr)
        Cacc[t] = zero4();
      else if (cin_packed)
        Cacc[t] = ld_packed4<D>(Cin, row, col);
      else
        Cacc[t] = *reinterpret_cast<const f32x4*>(Cin + (size_t)row * D + col);
    }
  }
  vm_wait_all();
  int64_t nb = (int64_t)cbeg * kL;
  if (a.n0 != nullptr)
    nb += a.snapshot ? reinterpret_cast<const int64_t*>(static_cast<const char*>(a.workspace) +
                                                         fwd_count_offset((size_t)a.B * a.H, P,
                                                                          gdn_slot_floats(D) * sizeof(float)))[chain]
                     : a.n0[chain];
  const float b_lam = a.b_lambda[h];
  if (tid < D) {
    const int c = tid;
    const float m = min_ ? min_[c] : 0.f;
    sm.m0[c] = m;
    const float wv = a.w_lambda[(size_t)h * D + c];
    const T whi = (T)wv, mhi = (T)m;
    sm.Wt[0][c] = whi;
    sm.Wt[1][c] = (T)(wv - (float)whi);
    sm.Wt[2][c] = mhi;
    sm.Wt[3][c] = (T)(m - (float)mhi);
  }
  for (int e = tid; e < kL * PT; e += 64 * NW) (&sm.Pm[0][0])[e] = (T)0.f;

  // ---- chunk tiles go straight from HBM to LDS (no registers involved): k of the next chunk
  // at the start of a chunk (it has its own buffer), q and v once the cleaned query and X
  // are formed.  Wave 1 keeps the per-token log alpha and beta of the next chunk in registers
  // (lane = token).  Rows past the end of the sequence are zeroed (beta = 0 then makes their
  // deltas zero).
  auto chunk_len = [&](int c) { return min(kL, a.T - c * kL); };
  auto dma_rows = [&](T (*dst)[PQ], const T* src, int c, int ln) {
    dma_tile<D, T, PQ>(dst, src + (tok0 + (size_t)c * kL) * D, chunk_len(c), w, NW, ln);
  };
  // wave 1: the raw log alpha and beta of token `lane` of the next chunk (token 0 again past the
  // end).  They stay as loaded until the chunk top, after its wait, where tokens past the end
  // read zero: anything done with them here would wait for the tile loads issued just before.
  T sg = T(0.f), sb = T(0.f);
  auto load_gates = [&](int c, int ln) {
    if (w == 1) {
      const size_t i = tok0 + (size_t)c * kL + (ln < chunk_len(c) ? ln : 0);
      sg = gg[i];
      sb = bg[i];
    }
  };
  auto put_gates = [&](int c, int ln) {
    const bool ok = ln < chunk_len(c);
    gdn_gates<D, T>(sm, ok ? to_f32(sg) : 0.f, ok ? to_f32(sb) : 0.f, ln);
  };
  if (cbeg < cend) {
    dma_rows(sm.Qs, qg, cbeg, lane);
    dma_rows(sm.Ks[cbeg & 1], kg, cbeg, lane);
    dma_rows(sm.Vs, vg, cbeg, lane);
    load_gates(cbeg, lane);
  }

  for (int ch = cbeg; ch < cend; ++ch) {
    // lane-derived values come from the lane index recomputed (and made opaque) every chunk, so
    // the compiler recomputes LDS addresses per chunk instead of holding them in registers across
    // the loop (where they spill, and every reload waits behind the in-flight tile loads)
    int lane_opaque;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_opaque));
    const int lane = lane_opaque, g = lane >> 4, l16 = lane & 15;
    (void)g;
    (void)l16;
    const int t0 = ch * kL;
    const int Lc = min(kL, a.T - t0);
    T (*Ks)[PQ] = sm.Ks[ch & 1];

    // ---- this chunk's tiles have landed; gates; rows past the end of the sequence zeroed
    vm_wait_all();
    if (w == 1) put_gates(ch, lane);
    if (CC) {  // the carry at this chunk's start, for the chunked backward
      put_carry_row<D, T, NA>(a, chain, ch, 0, cw + l16, g, Sacc);
      put_carry_row<D, T, NA>(a, chain, ch, 1, cw + l16, g, Cacc);
      if (tid < D) put_carry_ksum<D, T>(a, chain, ch, tid, sm.m0[tid]);
    }
    lds_barrier();
    if (Lc < kL) {
      zero_tail<D, T, PQ>(sm.Qs, Lc, tid, 64 * NW);
      zero_tail<D, T, PQ>(Ks, Lc, tid, 64 * NW);
      zero_tail<D, T, PQ>(sm.Vs, Lc, tid, 64 * NW);
      lds_barrier();
    }
    if (a.flags & kFlagNormalizeKeys) {
      normalize_rows<D, T, PQ>(Ks, tid, 64 * NW);
      lds_barrier();
    }
    if (ch + 1 < cend) dma_rows(sm.Ks[(ch + 1) & 1], kg, ch + 1, lane);

    // ---- gate and Gram rows (waves 0..3) and Q C0 (every wave); A = beta Gam (K K^T) below
    // the diagonal and the key sums (the other waves at d = 128, all of them at d = 64)
    ccq_gram_rows<D, T, NW>(sm, Ks, w, lane, nb, b_lam);
    {
      constexpr int kw0 = (NW >= 8) ? 4 : 0, kws = NW - kw0;
      if (w >= kw0) gdn_build_A<D, T>(sm, Ks, w - kw0, kws, lane);
      if (tid >= 2 * D) gdn_key_sums<D, T>(sm, Ks, tid - 2 * D);
    }
    f32x4 R[1][4];
    ccq_query_carry<D, T, 1, false>(sm, [&](int, int t) -> const f32x4& { return Cacc[t]; }, lane, R);
    lds_barrier();

    // ---- inverses of the diagonal blocks (the last four waves, one block each), cleaned query
    // (the inverse waves carry the longer path here: they take issue priority until the barrier)
    if (w >= NW - 4) __builtin_amdgcn_s_setprio(2);
    if (w >= NW - 4) gdn_diag_inverse_mfma<D, T>(sm, w - (NW - 4), lane);
    ccq_clean_query<D, T, 1, kSplit>(sm, Ks, sm.Qalo, R, cw, lane, [](int, int, int) { return 1.0f; });
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();
    if (ch + 1 < cend) dma_rows(sm.Qs, qg, ch + 1, lane);  // q of this chunk is no longer read

    // ---- X = beta (V - gamma K S0^T) and Delta on the wave's columns; M = tril(Qc K^T) * Gam
    // on the lower tiles -> Pm
    f32x4 X[4];
    gdn_rhs<D, T, true>(sm, Ks, [&](int t) -> const f32x4& { return Sacc[t]; }, cw, lane, X);

    for (int idx = w; idx < 10; idx += NW) {
      const int ti = tri_row(idx), tj = tri_col(idx);
      f32x4 acc = zero4();  // qc_i . k_j at j = 16 tj + 4 g + r, i = 16 ti + l16
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const Frag<T> A = lds_frag<T, KORD_CONTIG>(&Ks[0][0], PQ, 16 * tj, 32 * kk, lane);
        mma(acc, A, lds_frag<T, KORD_CONTIG>(&sm.Qa[0][0], PQ, 16 * ti, 32 * kk, lane));
        if constexpr (kSplit) mma(acc, A, lds_frag<T, KORD_CONTIG>(&sm.Qalo[0][0], PQ, 16 * ti, 32 * kk, lane));
        __builtin_amdgcn_sched_barrier(0);  // one K step of operands live at a time
      }
      const int i = 16 * ti + l16, j0 = 16 * tj + 4 * g;
      const float lgi = sm.lgam[i];
      const f32x4 lgj = *reinterpret_cast<const f32x4*>(&sm.lgam[j0]);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = (j0 + r <= i) ? acc[r] * __expf(lgi - lgj[r]) : 0.f;
      st4<T>(&sm.Pm[i][j0], acc);
    }
    f32x4 Dl[4];  // Delta[b][r] at token 16 b + 4 g + r, value channel cw + l16 (fp32)
    gdn_solve<D, T>(sm, X, lane, Dl);
    lds_barrier();
    if (ch + 1 < cend) {  // v of this chunk is no longer read
      dma_rows(sm.Vs, vg, ch + 1, lane);
      load_gates(ch + 1, lane);
    }

    // ---- O^T for the wave's 16 value rows: gamma * S0 Qc^T + Delta^T M^T
    f32x4 O[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) O[ti] = zero4();
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const Frag<T> A = acc_frag<T>(Sacc[2 * kk], Sacc[2 * kk + 1]);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) mma(O[ti], A, lds_frag<T, KORD_ACC>(&sm.Qa[0][0], PQ, 16 * ti, 32 * kk, lane));
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) O[ti] *= sm.gam[16 * ti + l16];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const Frag<T> A = acc_frag<T>(Dl[2 * kk], Dl[2 * kk + 1]);  // Delta^T, own rows
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        if (kk == 1 && ti < 2) continue;  // tokens 32..63 never precede tokens 0..31
        mma(O[ti], A, lds_frag<T, KORD_ACC>(&sm.Pm[0][0], PT, 16 * ti, 32 * kk, lane));
      }
    }
    T* og = static_cast<T*>(a.o);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      const int i = 16 * ti + l16;
      if (i < Lc) st4<T>(og + (tok0 + t0 + i) * D + cw + 4 * g, O[ti]);
    }

    // ---- carry update: C += K^T K;  S^T = gamma_L S0^T + K^T diag(gamma_L / gamma) Delta
    gdn_cov_update<D, T>(Ks, Cacc, cw, lane);
    gdn_state_update<D, T>(sm, Ks, [&](int t) -> f32x4& { return Sacc[t]; }, Dl, lane);
    if (tid < D) {
      const float m = sm.m1[tid];
      sm.m0[tid] = m;
      const T mhi = (T)m;
      sm.Wt[2][tid] = mhi;
      sm.Wt[3][tid] = (T)(m - (float)mhi);
    }
    nb += Lc;
    lds_barrier();
  }

  // ---- carry out (last segment)
  if (seg == P - 1 && a.S_out != nullptr) {
    float* Sout = a.S_out + (size_t)chain * D * D;
    float* Cout = a.C_out + (size_t)chain * (cpacked ? kTri : (size_t)D * D);
    const int row = cw + l16;
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      const int col = 16 * t + 4 * g;
      *reinterpret_cast<f32x4*>(Sout + (size_t)row * D + col) = Sacc[t];
      if (cpacked)
        st_packed4<D>(Cout, row, col, Cacc[t]);
      else
        *reinterpret_cast<f32x4*>(Cout + (size_t)row * D + col) = Cacc[t];
    }
    if (tid < D) a.ksum_out[(size_t)chain * D + tid] = sm.m0[tid];
    if (tid == 0) a.n_out[chain] = nb;
  }
}

// ---------------------------------------------------------------- segment summaries

// Workgroup (chain, segment p < P-1): runs the segment from a zero carry, (dS, dC, dksum), and
// the transition recurrence (state starting at I, v = 0), M_p, side by side, sharing the
// staged keys, A and the diagonal inverses; writes both to slot p.  Summary segments are
// whole chunks.
// WITH_C: the workgroup also accumulates dC = sum K^T K (otherwise csum_body does, beside it).
template <int D, typename T, bool WITH_C>
__device__ __forceinline__ void gdn_summary_body(const FwdArgs& a, GdnSmem<D, T>& sm, int bid) {
  using C_ = Cfg<D, T>;
  constexpr int NW = C_::NW, NA = C_::NA, PQ = C_::PQ;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cw = 16 * w;
  const int P = a.segments, cps = a.chunks_per_segment;
  const int chain = bid / (P - 1), seg = bid % (P - 1);
  const int nchunks = (a.T + kL - 1) / kL;
  const int cbeg = seg * cps;
  const int cend = min(nchunks, cbeg + cps);
  const size_t tok0 = (size_t)chain * (size_t)a.T;
  const T* kg = static_cast<const T*>(a.k);
  const T* vg = static_cast<const T*>(a.v);
  const T* gg = static_cast<const T*>(a.log_alpha);
  const T* bg = static_cast<const T*>(a.beta);

  // states: S from zero, M from the identity; C from zero
  f32x4 Sacc[NA], Macc[NA], Cacc[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    Sacc[t] = zero4();
    Cacc[t] = zero4();
#pragma unroll
    for (int r = 0; r < 4; ++r) Macc[t][r] = (cw + l16 == 16 * t + 4 * g + r) ? 1.f : 0.f;
  }
  if (tid < D) sm.m0[tid] = 0.f;

  auto chunk_len = [&](int c) { return min(kL, a.T - c * kL); };
  auto dma_rows = [&](T (*dst)[PQ], const T* src, int c, int ln) {
    dma_tile<D, T, PQ>(dst, src + (tok0 + (size_t)c * kL) * D, chunk_len(c), w, NW, ln);
  };
  // wave 1: the raw log alpha and beta of token `lane` of the next chunk (token 0 again past the
  // end).  They stay as loaded until the chunk top, after its wait, where tokens past the end
  // read zero: anything done with them here would wait for the tile loads issued just before.
  T sg = T(0.f), sb = T(0.f);
  auto load_gates = [&](int c, int ln) {
    if (w == 1) {
      const size_t i = tok0 + (size_t)c * kL + (ln < chunk_len(c) ? ln : 0);
      sg = gg[i];
      sb = bg[i];
    }
  };
  auto put_gates = [&](int c, int ln) {
    const bool ok = ln < chunk_len(c);
    gdn_gates<D, T>(sm, ok ? to_f32(sg) : 0.f, ok ? to_f32(sb) : 0.f, ln);
  };
  if (cbeg < cend) {
    dma_rows(sm.Ks[cbeg & 1], kg, cbeg, lane);
    dma_rows(sm.Vs, vg, cbeg, lane);
    load_gates(cbeg, lane);
  }

  for (int ch = cbeg; ch < cend; ++ch) {
    // the lane index recomputed, opaque to the compiler, every chunk (as in the main kernel)
    int lane_opaque;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_opaque));
    const int lane = lane_opaque;
    T (*Ks)[PQ] = sm.Ks[ch & 1];
    vm_wait_all();
    if (w == 1) put_gates(ch, lane);
    lds_barrier();
    if (a.flags & kFlagNormalizeKeys) {
      normalize_rows<D, T, PQ>(Ks, tid, 64 * NW);
      lds_barrier();
    }
    if (ch + 1 < cend) dma_rows(sm.Ks[(ch + 1) & 1], kg, ch + 1, lane);

    gdn_build_A<D, T>(sm, Ks, w, NW, lane);
    if (tid >= 2 * D) gdn_key_sums<D, T>(sm, Ks, tid - 2 * D);
    lds_barrier();

    if (w >= NW - 4) __builtin_amdgcn_s_setprio(2);  // the inverse waves' longer path, to the barrier
    if (w >= NW - 4) gdn_diag_inverse_mfma<D, T>(sm, w - (NW - 4), lane);
    f32x4 XSM[2][4];  // right-hand sides of the S and M recurrences
    gdn_rhs<D, T, true>(sm, Ks, [&](int t) -> const f32x4& { return Sacc[t]; }, cw, lane, XSM[0]);
    gdn_rhs<D, T, false>(sm, Ks, [&](int t) -> const f32x4& { return Macc[t]; }, cw, lane, XSM[1]);
    __builtin_amdgcn_s_setprio(0);
    lds_barrier();
    if (ch + 1 < cend) {
      dma_rows(sm.Vs, vg, ch + 1, lane);
      load_gates(ch + 1, lane);
    }

    {
      f32x4 Dl[2][4];
      gdn_solve_n<D, T, 2>(sm, XSM, lane, Dl);
      gdn_state_update<D, T>(sm, Ks, [&](int t) -> f32x4& { return Sacc[t]; }, Dl[0], lane);
      gdn_state_update<D, T>(sm, Ks, [&](int t) -> f32x4& { return Macc[t]; }, Dl[1], lane);
    }
    if constexpr (WITH_C) gdn_cov_update<D, T>(Ks, Cacc, cw, lane);
    if (tid < D) sm.m0[tid] = sm.m1[tid];
    lds_barrier();
  }

  float* slot = static_cast<float*>(a.workspace) + ((size_t)chain * P + seg) * gdn_slot_floats(D);
  const int row = cw + l16;
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    const size_t o = (size_t)row * D + 16 * t + 4 * g;
    *reinterpret_cast<f32x4*>(slot + o) = Sacc[t];
    if constexpr (WITH_C) *reinterpret_cast<f32x4*>(slot + (size_t)D * D + o) = Cacc[t];
    *reinterpret_cast<f32x4*>(slot + 2 * (size_t)D * D + D + o) = Macc[t];
  }
  if (tid < D) slot[2 * (size_t)D * D + tid] = sm.m0[tid];
}

template <int D, typename T>
__global__ __launch_bounds__(4 * D) void gdn_summary_kernel(FwdArgs a) {
  __shared__ GdnSmem<D, T> sm;
  gdn_summary_body<D, T, true>(a, sm, blockIdx.x);
}

// The summary in two roles of one launch (as gla_summary_split_kernel): summary workgroups without
// dC, and dC workgroups on the compute units the summary leaves idle.
template <int D, typename T>
union GdnSplitSmem {
  GdnSmem<D, T> s;
  CSumSmem<D, T> c;
};
template <int D, typename T>
__global__ __launch_bounds__(4 * D) void gdn_summary_split_kernel(FwdArgs a) {
  __shared__ GdnSplitSmem<D, T> sm;
  const int nS = a.B * a.H * (a.segments - 1);
  if ((int)blockIdx.x < nS)
    gdn_summary_body<D, T, false>(a, sm.s, blockIdx.x);
  else
    csum_body<D, T>(a, sm.c, blockIdx.x - nS, gridDim.x - nS, gdn_slot_floats(D));
}

// ---------------------------------------------------------------- scans over segments

// S part, in fp32: slot p holds dS_p and M_p (p < P-1) and receives S_in[p] (1 <= p <= P-1):
//   S_in[0] = S0 (or 0),  S_in[p+1] = S_in[p] M_p + dS_p.  The main kernel's segment 0 reads the
// caller's carry itself, so slot 0 keeps its summary -- unless the carry out overlaps the carry
// in: then slot 0 receives S_in[0] as well.
// Workgroup (16-row block rb of S, chain), D/32 waves: wave w computes the two 16x16 output
// tiles at columns 32 w .. 32 w + 31 with fp32 MFMAs (v_mfma_f32_16x16x4_f32, one K-slice of 4
// per instruction), the A operand (rows of S_in[p]) and B operand (M_p) read from LDS, eight
// K-slices of operands at a time.  The running rows live in the accumulators: lane (g, l)
// holds rows 4 g + r, column n0 + 16 t + l.
template <int D>
__global__ __launch_bounds__(2 * D) void gdn_scan_state_kernel(FwdArgs a) {
  constexpr int NT = 2 * D, KB = 8;
  __shared__ float Ss[16][D + 4];
  __shared__ float Ms[D][D + 4];
  const int rb = blockIdx.x, chain = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int P = a.segments;
  const size_t slot_f = gdn_slot_floats(D);
  float* base = static_cast<float*>(a.workspace) + (size_t)chain * P * slot_f;
  const int n0 = 32 * w;
  auto elem = [&](int t, int r) { return (size_t)(16 * rb + 4 * g + r) * D + n0 + 16 * t + l16; };
  f32x4 run[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) run[t][r] = (a.S0 != nullptr) ? a.S0[(size_t)chain * D * D + elem(t, r)] : 0.f;
  for (int p = 0; p < P; ++p) {
    float* slot = base + (size_t)p * slot_f;
    f32x4 dS[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        dS[t][r] = (p < P - 1) ? slot[elem(t, r)] : 0.f;
        // segment 0 reads the caller's carry itself unless the carry out overlaps it
        if (p > 0 || a.snapshot) slot[elem(t, r)] = run[t][r];
      }
    if (p == P - 1) break;
    // M_p: every load in flight before the first LDS store
    constexpr int NV = D * D / 4 / NT;
    const float* M = slot + 2 * (size_t)D * D + D;
    f32x4 mv[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) mv[v] = *reinterpret_cast<const f32x4*>(M + 4 * (size_t)(tid + NT * v));
    __syncthreads();  // the previous step's reads of Ss and Ms are done
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int e = 4 * (tid + NT * v);
      *reinterpret_cast<f32x4*>(&Ms[e / D][e % D]) = mv[v];
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) Ss[4 * g + r][n0 + 16 * t + l16] = run[t][r];
    __syncthreads();
    run[0] = dS[0];
    run[1] = dS[1];
    for (int k0 = 0; k0 < D / 4; k0 += KB) {
      float av[KB], b0[KB], b1[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int kk = k0 + u;
        av[u] = Ss[l16][4 * kk + g];
        b0[u] = Ms[4 * kk + g][n0 + l16];
        b1[u] = Ms[4 * kk + g][n0 + 16 + l16];
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        run[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], b0[u], run[0], 0, 0, 0);
        run[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], b1[u], run[1], 0, 0, 0);
      }
    }
  }
}

// C and ksum part: additive exclusive scan, one thread per float of the C | ksum region (slot 0
// not written, as for S).
template <int D>
__global__ __launch_bounds__(256) void gdn_scan_sum_kernel(FwdArgs a) {
  const int chain = blockIdx.y;
  const int P = a.segments;
  const size_t f = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (f >= (size_t)D * D + D) return;
  const size_t slot_f = gdn_slot_floats(D);
  if (a.snapshot && f == 0) {  // the caller's token count, for every segment of the main kernel
    int64_t* counts = reinterpret_cast<int64_t*>(static_cast<char*>(a.workspace) +
                                                 fwd_count_offset((size_t)a.B * a.H, P, slot_f * sizeof(float)));
    counts[chain] = a.n0 != nullptr ? a.n0[chain] : 0;
  }
  float* base = static_cast<float*>(a.workspace) + (size_t)chain * P * slot_f + (size_t)D * D;
  float run = 0.f;
  if (a.S0 != nullptr) {
    if (f >= (size_t)D * D)
      run = a.ksum0[(size_t)chain * D + (f - (size_t)D * D)];
    else if (a.flags & kFlagPackedCov)
      run = a.C0[(size_t)chain * D * (D + 1) / 2 + packed_index((int)f / D, (int)f % D, D)];
    else
      run = a.C0[(size_t)chain * D * D + f];
  }
  for (int p = 0; p < P; ++p) {
    float* v = base + (size_t)p * slot_f + f;
    const float d = (p < P - 1) ? *v : 0.f;
    if (p > 0 || a.snapshot) *v = run;
    run += d;
  }
}

}  // namespace ccq
