// Chunked prefill of the CCQ read step on a Gated DeltaNet backbone (gfx950).
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
// Kernel layout.  One workgroup of D/16 waves per chain; wave w owns the 16 value channels
// [16w, 16w + 16): its tiles of C and S^T live in MFMA accumulators (as in the GLA kernel), and
// so do its columns of X and Delta, held as Delta[j][v] tiles (token rows).  The triangular
// system is solved in fp32 by 16-token blocks: the inverses of the four diagonal blocks
// (I + A_bb)^{-1} come from forward substitution (one lane per column), then every wave runs
// Delta_b = (I + A_bb)^{-1} (X_b - sum_{b' < b} A_bb' Delta_b') on its own columns with fp32
// MFMAs, the off-diagonal blocks of A read from LDS.  Products on bf16 operands with fp32
// accumulation: K S0^T, Qc S0^T, the intra term and the carry update; the intra matrix
// Qc K^T takes qc as bf16 hi + lo.
#include "ccq_internal.hpp"
#include "ccq_prefill_common.hpp"

namespace ccq {

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
  f32x4 tok[kL];             // lambda, 1/n, sq/n^2, gate logit + b
};

template <int D, typename T>
__global__ __launch_bounds__(4 * D) void gdn_main_kernel(FwdArgs a) {
  using C_ = Cfg<D, T>;
  constexpr int NW = C_::NW, NA = C_::NA, NK = C_::NK;
  constexpr int PQ = C_::PQ, PT = C_::PT;
  constexpr bool kSplit = sizeof(T) == 2;
  __shared__ GdnSmem<D, T> sm;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int cw = 16 * w;        // this wave's 16 channels
  const int chain = blockIdx.x;
  const int h = chain % a.H;
  const int nchunks = (a.T + kL - 1) / kL;
  const size_t tok0 = (size_t)chain * (size_t)a.T;
  const T* qg = static_cast<const T*>(a.q);
  const T* kg = static_cast<const T*>(a.k);
  const T* vg = static_cast<const T*>(a.v);
  const T* gg = static_cast<const T*>(a.log_alpha);
  const T* bg = static_cast<const T*>(a.beta);

  // ---- carry in
  f32x4 Cacc[NA], Sacc[NA];
  {
    const int row = cw + l16;
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      const int col = 16 * t + 4 * g;
      Sacc[t] = a.S0 ? *reinterpret_cast<const f32x4*>(a.S0 + (size_t)chain * D * D + (size_t)row * D + col) : zero4();
      Cacc[t] = a.C0 ? *reinterpret_cast<const f32x4*>(a.C0 + (size_t)chain * D * D + (size_t)row * D + col) : zero4();
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  int64_t nb = (a.n0 != nullptr) ? a.n0[chain] : 0;
  const float b_lam = a.b_lambda[h];
  if (tid < D) {
    const int c = tid;
    const float m = a.ksum0 ? a.ksum0[(size_t)chain * D + c] : 0.f;
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
  auto dma_rows = [&](T (*dst)[PQ], const T* src, int c) {
    dma_tile<D, T, PQ>(dst, src + (tok0 + (size_t)c * kL) * D, chunk_len(c), w, NW, lane);
  };
  float sg = 0.f, sb = 0.f;
  auto load_gates = [&](int c) {
    if (w == 1) {
      const bool ok = lane < chunk_len(c);
      const size_t i = tok0 + (size_t)c * kL + (ok ? lane : 0);
      const float x = ldf(gg, i), y = ldf(bg, i);
      sg = ok ? x : 0.f;
      sb = ok ? y : 0.f;
    }
  };
  if (nchunks > 0) {
    dma_rows(sm.Qs, qg, 0);
    dma_rows(sm.Ks[0], kg, 0);
    dma_rows(sm.Vs, vg, 0);
    load_gates(0);
  }

  for (int ch = 0; ch < nchunks; ++ch) {
    const int t0 = ch * kL;
    const int Lc = min(kL, a.T - t0);
    T (*Ks)[PQ] = sm.Ks[ch & 1];

    // ---- this chunk's tiles have landed; chunk-local log gamma by an inclusive scan over the
    // lanes of wave 1; rows past the end of the sequence are zeroed
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (w == 1) {
      float x = sg;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      sm.lgam[lane] = x;
      sm.beta[lane] = sb;
    }
    lds_barrier();
    if (Lc < kL) {
      zero_tail<D, T, PQ>(sm.Qs, Lc, tid, 64 * NW);
      zero_tail<D, T, PQ>(Ks, Lc, tid, 64 * NW);
      zero_tail<D, T, PQ>(sm.Vs, Lc, tid, 64 * NW);
      lds_barrier();
    }
    if (ch + 1 < nchunks) dma_rows(sm.Ks[(ch + 1) & 1], kg, ch + 1);

    // ---- gate and Gram rows (waves 0..3); A = beta Gam (K K^T) below the diagonal and the key
    // sums (the other waves at d = 128, all of them at d = 64)
    ccq_gram_rows<D, T, NW>(sm, Ks, w, lane, nb, b_lam);
    {
      constexpr int kw0 = (NW >= 8) ? 4 : 0, kws = NW - kw0;
      if (w >= kw0) {
        for (int idx = w - kw0; idx < 10; idx += kws) {
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
      if (tid >= 2 * D) {  // key sums: two threads per channel, 32 tokens each
        const int c = (tid - 2 * D) >> 1, half = tid & 1;
        float s = 0.f;
#pragma unroll 8
        for (int t = 32 * half; t < 32 * half + 32; ++t) s += to_f32(Ks[t][c]);
        s += __shfl_xor(s, 1, 64);
        if (half == 0) sm.m1[c] = sm.m0[c] + s;
      }
    }
    lds_barrier();

    // ---- inverses of the diagonal blocks (last wave: lane = (block, column)), cleaned query,
    // X = beta (V - gamma K S0^T) for the wave's value channels
    if (w == NW - 1) {
      const int blk = lane >> 4, c = l16, base = 16 * blk;
      float tcol[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
        for (int jj = 0; jj < (i + 3) / 4; ++jj) {
          const f32x4 a4 = *reinterpret_cast<const f32x4*>(&sm.As[base + i][base + 4 * jj]);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * jj + e < i) acc -= a4[e] * tcol[4 * jj + e];
        }
        tcol[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.Tb[blk][i][c] = tcol[i];
    }
    f32x4 R[1][4];
    ccq_query_carry<D, T, 1>(sm, [&](int, int t) -> const f32x4& { return Cacc[t]; }, lane, R);
    ccq_clean_query<D, T, 1, kSplit>(sm, Ks, sm.Qalo, R, cw, lane, [](int, int, int) { return 1.0f; });
    f32x4 X[4];  // X[b][r] at token 16 b + 4 g + r, value channel cw + l16
#pragma unroll
    for (int b = 0; b < 4; ++b) X[b] = zero4();
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const Frag<T> Bs = acc_frag<T>(Sacc[2 * kk], Sacc[2 * kk + 1]);  // S0^T, own columns
#pragma unroll
      for (int b = 0; b < 4; ++b) mma(X[b], lds_frag<T, KORD_ACC>(&Ks[0][0], PQ, 16 * b, 32 * kk, lane), Bs);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int j0 = 16 * b + 4 * g;
      const f32x4 lg = *reinterpret_cast<const f32x4*>(&sm.lgam[j0]);
      const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[j0]);
#pragma unroll
      for (int r = 0; r < 4; ++r) X[b][r] = bt[r] * (to_f32(sm.Vs[j0 + r][cw + l16]) - __expf(lg[r]) * X[b][r]);
    }
    lds_barrier();
    if (ch + 1 < nchunks) {  // q and v of this chunk are no longer read
      dma_rows(sm.Qs, qg, ch + 1);
      dma_rows(sm.Vs, vg, ch + 1);
      load_gates(ch + 1);
    }

    // ---- M = tril(Qc K^T) * Gam on the lower tiles -> Pm; Delta on the wave's columns
    for (int idx = w; idx < 10; idx += NW) {
      const int ti = tri_row(idx), tj = tri_col(idx);
      f32x4 acc = zero4();  // qc_i . k_j at j = 16 tj + 4 g + r, i = 16 ti + l16
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const Frag<T> A = lds_frag<T, KORD_CONTIG>(&Ks[0][0], PQ, 16 * tj, 32 * kk, lane);
        mma(acc, A, lds_frag<T, KORD_CONTIG>(&sm.Qa[0][0], PQ, 16 * ti, 32 * kk, lane));
        if constexpr (kSplit) mma(acc, A, lds_frag<T, KORD_CONTIG>(&sm.Qalo[0][0], PQ, 16 * ti, 32 * kk, lane));
      }
      const int i = 16 * ti + l16, j0 = 16 * tj + 4 * g;
      const float lgi = sm.lgam[i];
      const f32x4 lgj = *reinterpret_cast<const f32x4*>(&sm.lgam[j0]);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = (j0 + r <= i) ? acc[r] * __expf(lgi - lgj[r]) : 0.f;
      st4<T>(&sm.Pm[i][j0], acc);
    }
    f32x4 Dl[4];  // Delta[b][r] at token 16 b + 4 g + r, value channel cw + l16 (fp32)
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
    lds_barrier();

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
    for (int ti = 0; ti < 4; ++ti) O[ti] *= __expf(sm.lgam[16 * ti + l16]);
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
    const float lgL = sm.lgam[kL - 1];
    const float gL = __expf(lgL);
#pragma unroll
    for (int t = 0; t < NA; ++t) Sacc[t] *= gL;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const Frag<T> Bk = tr_frag<T>(&Ks[0][0], PQ, 32 * kk, cw, lane);  // K[t][own channel]
      f32x4 d0 = Dl[2 * kk], d1 = Dl[2 * kk + 1];
      const f32x4 lg0 = *reinterpret_cast<const f32x4*>(&sm.lgam[32 * kk + 4 * g]);
      const f32x4 lg1 = *reinterpret_cast<const f32x4*>(&sm.lgam[32 * kk + 16 + 4 * g]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        d0[r] *= __expf(lgL - lg0[r]);
        d1[r] *= __expf(lgL - lg1[r]);
      }
      const Frag<T> Bd = acc_frag<T>(d0, d1);  // diag(gamma_L / gamma) Delta, own columns
#pragma unroll
      for (int t = 0; t < NA; ++t) {
        mma(Cacc[t], tr_frag<T>(&Ks[0][0], PQ, 32 * kk, 16 * t, lane), Bk);
        mma(Sacc[t], tr_frag_acc<T>(&Ks[0][0], PQ, 32 * kk, 16 * t, lane), Bd);
      }
    }
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

  // ---- carry out
  if (a.S_out != nullptr) {
    float* Sout = a.S_out + (size_t)chain * D * D;
    float* Cout = a.C_out + (size_t)chain * D * D;
    const int row = cw + l16;
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      const int col = 16 * t + 4 * g;
      *reinterpret_cast<f32x4*>(Sout + (size_t)row * D + col) = Sacc[t];
      *reinterpret_cast<f32x4*>(Cout + (size_t)row * D + col) = Cacc[t];
    }
    if (tid < D) a.ksum_out[(size_t)chain * D + tid] = sm.m0[tid];
    if (tid == 0) a.n_out[chain] = nb;
  }
}

template <int D, typename T>
static hipError_t launch_gdn_t(const FwdArgs& a, hipStream_t s) {
  if (a.events != nullptr) {
    for (int i = 0; i < 3; ++i)
      if (hipEventRecord(static_cast<hipEvent_t>(a.events[i]), s) != hipSuccess) return hipErrorLaunchFailure;
  }
  hipLaunchKernelGGL((gdn_main_kernel<D, T>), dim3((unsigned)(a.B * a.H)), dim3(4 * D), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.events == nullptr) return e;
  return hipEventRecord(static_cast<hipEvent_t>(a.events[3]), s);
}

hipError_t launch_gdn(const FwdArgs& a, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.d == 128) return launch_gdn_t<128, __bf16>(a, s);
    if (a.d == 64) return launch_gdn_t<64, __bf16>(a, s);
  } else {
    if (a.d == 64) return launch_gdn_t<64, float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
