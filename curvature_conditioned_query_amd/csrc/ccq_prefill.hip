// Chunked prefill of the CCQ read step on a GLA backbone (gfx950).
//
// Method (gist.science summary of arXiv 2606.01294, "不要阅读一切：一种基于曲率条件的线性注意力
// 查询"): §2 "理论推导" gives Sigma_t = Cbar_t - mu_t mu_t^T from the running mean and
// second moment of the keys; §2 "机制" gives q_clean = q_t - lambda_t Sigma_t q_t with
// lambda_t = sigmoid(W_lambda q_t + b_lambda) and says the statistics are kept by the same
// recurrent or chunked mechanism as the backbone state; §2 "集成" leaves the write rule
// unchanged and reads o_t = S_t q_clean.  The GLA write rule is
// S_t = S_{t-1} diag(alpha_t) + v_t k_t^T with alpha_t = exp(g_t) per key channel.
//
// Chunk algebra (rows i = 0..63 of a chunk, carry S0, C0 = sum k k^T, m0 = sum k, n0),
// obtained by unrolling the per-token recurrence inside the chunk:
//   s_i  = m0 + sum_{j<=i} k_j,  n_i = n0 + i + 1,  sq_i = s_i . q_i = m0 . q_i + sum_{j<=i} P_ij
//   with P = Q K^T, row i of Q C0 + tril_incl(P) K is C_i q_i, and
//   u_i  = C_i q_i / n_i - s_i sq_i / n_i^2                                  (row i = Sigma_i q_i)
//        = (Q C0 + tril_incl(P - c 1^T) K)_i / n_i - m0 sq_i / n_i^2,  c_i = sq_i / n_i
//   qc_i = q_i - lambda_i u_i
//   B_i  = sum_{j<=i} g_j  (per channel, chunk-local)
//   O    = (Qc * e^B) S0^T + tril_incl((Qc * e^B)(K * e^-B)^T) V
//   S_L  = (S0 + V^T (K * e^-B)) diag(e^{B_63})
//   C0 += K^T K;  m0 += sum_j k_j;  n0 += L
// The intra-chunk decay is factored with the chunk start as reference, so e^{-B} stays
// finite while B > -80 inside a chunk (the documented precondition).
//
// Kernel layout.  One workgroup of D/16 waves per (chain, segment) -- 8 waves at d = 128,
// two per SIMD, so one wave's vector and LDS work overlaps the other's matrix work.
// Wave w owns the 16 channels [16w, 16w + 16) of d:
//  - both fp32 carries live in its MFMA accumulators: tile a of C holds C[16a+4g+r][16w+l]
//    and tile a of S holds S^T[16a+4g+r][16w+l] (l = lane % 16, g = lane / 16, r =
//    element).  Read as an A operand, a pair of such tiles is S (resp. C, which is
//    symmetric) restricted to the wave's rows, so the carry feeds the read-side MFMAs
//    straight from registers and never leaves them inside a chain;
//  - every chunk tile sits in LDS row-major ([token][channel]); operands whose contraction
//    runs over tokens (K^T, V^T, (K e^-B)^T) are read with the gfx950 transposing LDS read
//    (ds_read_b64_tr_b16), so no transposed copy is ever written;
//  - the next chunk's q, k, v and log decay go straight from HBM to LDS
//    (global_load_lds_dwordx4), each as soon as the buffer it lands in is free, so no
//    registers hold prefetched rows;
//  - the cumulative decay over tokens is an MFMA against a lower-triangular ones fragment,
//    channel selection an MFMA against an identity fragment (exact: x * 1 + 0).
#include "ccq_internal.hpp"
#include "ccq_prefill_common.hpp"

#include <type_traits>

namespace ccq {

// Workspace slot of one (chain, segment): S [D][D] | C [D][D] | ksum [D] | log decay [D], fp32.
size_t fwd_slot_bytes(int d) { return (size_t)(2 * d * d + 2 * d) * sizeof(float); }

template <int D, typename T>
struct Smem {
  using C_ = Cfg<D, T>;
  T Qs[kL][C_::PQ];     // q rows
  T Gs[kL][C_::PQ];     // log decay rows
  // Chunk c keeps its k rows in X[c % 2] and v rows in Y[c % 2]; the other halves receive the
  // next chunk's k and v (in the first chunk of a sequence they hold the bf16 low parts of
  // k e^-B and q_clean e^B until the intra-chunk attention is formed).
  T X[2][kL][C_::PQ];
  T Y[2][kL][C_::PQ];
  T Kp[kL][C_::PQ];     // k * e^-B rows (hi part for bf16)
  T Qa[kL][C_::PQ];     // q_clean * e^B rows (hi part for bf16)
  T Pm[kL][C_::PT];     // tril(Q K^T - c 1^T), then the masked intra-chunk attention matrix
  T Wt[4][C_::PQ];      // w_lambda hi, lo; key sum hi, lo (B operand of q . [w, m0])
  float m0[D], m1[D], eBL[D];
  f32x4 tok[kL];        // per token: lambda, 1/n, sq/n^2, gate logit + b
};

// Full read (o for every token) of one (chain, segment) from the segment's carry-in, carry
// out at the end of the chain.
// CC: this instantiation writes the carry at every chunk start (FwdArgs::chunk_carry); the one
// without it carries no trace of that code.
template <int D, typename T, bool CC>
__global__ __launch_bounds__(4 * D) void gla_main_kernel(FwdArgs a) {
  using C_ = Cfg<D, T>;
  constexpr int NW = C_::NW, NA = C_::NA, NK = C_::NK;
  constexpr int PQ = C_::PQ, PT = C_::PT;
  constexpr bool kSplit = sizeof(T) == 2;  // hi/lo operands for the intra term
  __shared__ Smem<D, T> sm;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int cw = 16 * w;       // this wave's 16 channels
  const int hb = w & 1;        // which half of its 32-channel block
  const int cb = cw - 16 * hb; // first channel of the block
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
  float* slots = static_cast<float*>(a.workspace);
  const size_t slot_f = 2 * (size_t)D * D + 2 * D;

  // ---- carry in
  // the caller's C0 / C_out may be the packed upper triangle (the workspace slots never are)
  const bool cpacked = (a.flags & kFlagPackedCov) != 0;
  constexpr size_t kTri = (size_t)D * (D + 1) / 2;
  f32x4 Cacc[NA], Sacc[NA];
  const float* Sin = nullptr;
  const float* Cin = nullptr;
  const float* min_ = nullptr;
  bool cin_packed = false;
  // segment 0 starts from the caller's carry (or zeros) itself, unless the carry out overlaps
  // it: then the scan has copied it into slot 0
  if (P > 1 && (seg > 0 || a.snapshot)) {
    const float* slot = slots + ((size_t)chain * P + seg) * slot_f;
    Sin = slot;
    Cin = slot + (size_t)D * D;
    min_ = slot + 2 * (size_t)D * D;
  } else if (a.S0 != nullptr) {
    Sin = a.S0 + (size_t)chain * D * D;
    cin_packed = cpacked;
    Cin = a.C0 + (size_t)chain * (cpacked ? kTri : (size_t)D * D);
    min_ = a.ksum0 + (size_t)chain * D;
  }
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
  // the carry-in loads complete here, so nothing in the chunk loop waits on them
  vm_wait_all();
  int64_t nb = (int64_t)cbeg * kL;  // tokens before this chunk (count base)
  if (a.n0 != nullptr)
    nb += a.snapshot ? reinterpret_cast<const int64_t*>(reinterpret_cast<const char*>(a.workspace) +
                                                          fwd_count_offset((size_t)a.B * a.H, P, slot_f * sizeof(float)))[chain]
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

  // ---- chunk tiles go straight from HBM to LDS (no registers involved), each as soon as the
  // previous chunk has finished reading the buffer it lands in: log decay after the gate and
  // Gram rows, q after the cleaned query, k and v at the start of the previous chunk (after its
  // intra-chunk attention when that chunk splits its operands into hi + lo).
  auto chunk_len = [&](int ch) { return min(kL, a.T - ch * kL); };
  const DmaPlan<D, T, PQ, NW> plan(w, lane);
  auto dma_rows = [&](T (*dst)[PQ], const T* g, int ch) {
    plan.load(dst, g + (tok0 + (size_t)ch * kL) * D, chunk_len(ch), w);
  };
  if (cbeg < cend) {
    dma_rows(sm.Qs, qg, cbeg);
    dma_rows(sm.Gs, gg, cbeg);
    dma_rows(sm.X[cbeg & 1], kg, cbeg);
    dma_rows(sm.Y[cbeg & 1], vg, cbeg);
  }

  if (CC && cbeg < cend) {  // the carry at the segment's first chunk, for the backward
    put_carry_row<D, T, NA>(a, chain, cbeg, 0, cw + l16, g, Sacc);
    put_carry_row<D, T, NA>(a, chain, cbeg, 1, cw + l16, g, Cacc);
    if (tid < D) put_carry_ksum<D, T>(a, chain, cbeg, tid, sm.m0[tid]);  // this thread's own m0 entry
  }
  const Frag<T> Ih = ident_frag<T>(hb, lane);

  // One chunk.  bf16: the intra-chunk attention takes hi + lo operands in the first chunk of a
  // sequence read from an empty state, where an output is one or a few possibly cancelling
  // products and nothing else; in every later chunk single bf16 operands, like every other
  // product here, so the next chunk's k and v stream in from the start of the chunk.  That
  // first chunk runs its own copy of the body, so the loop carries no registers for the split.
  auto chunk = [&](const int ch, auto split_tag) {
    constexpr bool split = kSplit && decltype(split_tag)::value;
    const int t0 = ch * kL;
    const int Lc = min(kL, a.T - t0);

    T (*Ks)[PQ] = sm.X[ch & 1];
    T (*Vs)[PQ] = sm.Y[ch & 1];
    T (*Klo)[PQ] = sm.X[(ch + 1) & 1];   // split chunks only
    T (*Qalo)[PQ] = sm.Y[(ch + 1) & 1];  // split chunks only

    // ---- this chunk's tiles have landed (own loads, then everyone's); rows past the end of
    // the sequence are zeroed
    vm_wait_all();
    lds_barrier();
    if (Lc < kL) {
      zero_tail<D, T, PQ>(sm.Qs, Lc, tid, 64 * NW);
      zero_tail<D, T, PQ>(sm.Gs, Lc, tid, 64 * NW);
      zero_tail<D, T, PQ>(Ks, Lc, tid, 64 * NW);
      zero_tail<D, T, PQ>(Vs, Lc, tid, 64 * NW);
      lds_barrier();
    }
    if (a.flags & kFlagNormalizeKeys) {
      normalize_rows<D, T, PQ>(Ks, tid, 64 * NW);
      lds_barrier();
    }
    if (!split && ch + 1 < cend) {
      dma_rows(sm.X[(ch + 1) & 1], kg, ch + 1);
      dma_rows(sm.Y[(ch + 1) & 1], vg, ch + 1);
    }

    // ---- own channels: cumulative decay (4 consecutive channels per lane), k e^-B, key sum,
    // chunk decay.  BT[ti][r] = B at token 16 ti + l16, channel cw + 4g + r.
    f32x4 BT[4];
    {
      f32x4 GT[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        GT[ti] = zero4();  // log alpha at token 16 ti + 4 g + r, channel cw + l16
        mma(GT[ti], lds_frag<T, KORD_CONTIG>(&sm.Gs[0][0], PQ, 16 * ti, cb, lane), Ih);
      }
      const Frag<T> Ga = acc_frag<T>(GT[0], GT[1]);
      const Frag<T> Gb = acc_frag<T>(GT[2], GT[3]);
      f32x4 ks = zero4();
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        BT[ti] = zero4();
        mma(BT[ti], Ga, ltri_frag<T>(ti, 0, lane));
        if (ti >= 2) mma(BT[ti], Gb, ltri_frag<T>(ti, 1, lane));
        f32x4 KC = zero4();  // k at token 16 ti + l16, channel cw + 4g + r
        mma(KC, Ih, lds_frag<T, KORD_CONTIG>(&Ks[0][0], PQ, 16 * ti, cb, lane));
        ks += KC;
        f32x4 kp;
#pragma unroll
        for (int r = 0; r < 4; ++r) kp[r] = KC[r] * __expf(-BT[ti][r]);
        const int t = 16 * ti + l16;
        if constexpr (kSplit) {
          const bf16x4 kh = to_bf16x4(kp);
          *reinterpret_cast<bf16x4*>(&sm.Kp[t][cw + 4 * g]) = kh;
          if (split) {
            f32x4 kl;
#pragma unroll
            for (int r = 0; r < 4; ++r) kl[r] = kp[r] - (float)kh[r];
            st4<T>(&Klo[t][cw + 4 * g], kl);
          }
        } else {
          st4<T>(&sm.Kp[t][cw + 4 * g], kp);
        }
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) ks[r] += __shfl_xor(ks[r], off, 64);
      }
      const int c = cw + 4 * g;
      if (l16 == 0) *reinterpret_cast<f32x4*>(&sm.m1[c]) = *reinterpret_cast<const f32x4*>(&sm.m0[c]) + ks;
      if (l16 == 15) {  // token 63
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sm.eBL[c + r] = __expf(BT[3][r]);
        }
      }
    }
    // gate and Gram rows on waves 0..3 while every wave forms Q C0 for its channels
    ccq_gram_rows<D, T, NW>(sm, Ks, w, lane, nb, b_lam);
    f32x4 R[1][4];
    ccq_query_carry<D, T, 1>(sm, [&](int, int t) -> const f32x4& { return Cacc[t]; }, lane, R);
    lds_barrier();
    if (ch + 1 < cend) dma_rows(sm.Gs, gg, ch + 1);

    ccq_clean_query<D, T, 1, split>(sm, Ks, Qalo, R, cw, lane,
                                    [&](int, int ti, int r) { return __expf(BT[ti][r]); });
    // C += K^T K for the wave's channels: Q C0 is formed, so the statistic carry moves on here,
    // beside the cleaned query, rather than in the output phase
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const Frag<T> Bk = tr_frag<T>(&Ks[0][0], PQ, 32 * kk, cw, lane);  // K[t][own channel]
#pragma unroll
      for (int t0_ = 0; t0_ < NA; t0_ += 4) {
        Frag<T> Ak[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) Ak[u] = tr_frag<T>(&Ks[0][0], PQ, 32 * kk, 16 * (t0_ + u), lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) mma(Cacc[t0_ + u], Ak[u], Bk);
      }
    }
    lds_barrier();
    if (ch + 1 < cend) dma_rows(sm.Qs, qg, ch + 1);

    // ---- O^T for the wave's 16 value rows, first part: S0 (Qc e^B)^T (needs only the cleaned
    // query, so it runs beside the intra-chunk attention)
    f32x4 O[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) O[ti] = zero4();
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      Frag<T> Bq[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) Bq[ti] = lds_frag<T, KORD_ACC>(&sm.Qa[0][0], PQ, 16 * ti, 32 * kk, lane);
      const Frag<T> A = acc_frag<T>(Sacc[2 * kk], Sacc[2 * kk + 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) mma(O[ti], A, Bq[ti]);
    }

    // ---- intra-chunk attention (Qc e^B)(K e^-B)^T on the lower tiles -> Pm (masked)
    {
      constexpr bool kLo = split;
      for (int idx = w; idx < 10; idx += NW) {
        const int ti = tri_row(idx), tj = tri_col(idx);
        f32x4 acc = zero4();
        Frag<T> Af[NK], Bf[NK], Alf[NK], Blf[NK];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          Af[kk] = lds_frag<T, KORD_CONTIG>(&sm.Kp[0][0], PQ, 16 * tj, 32 * kk, lane);
          Bf[kk] = lds_frag<T, KORD_CONTIG>(&sm.Qa[0][0], PQ, 16 * ti, 32 * kk, lane);
          if constexpr (kLo) {
            Alf[kk] = lds_frag<T, KORD_CONTIG>(&Klo[0][0], PQ, 16 * tj, 32 * kk, lane);
            Blf[kk] = lds_frag<T, KORD_CONTIG>(&Qalo[0][0], PQ, 16 * ti, 32 * kk, lane);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          mma(acc, Af[kk], Bf[kk]);
          if constexpr (kLo) {
            mma(acc, Af[kk], Blf[kk]);
            mma(acc, Alf[kk], Bf[kk]);
          }
        }
        const int i = 16 * ti + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = (16 * tj + 4 * g + r <= i) ? acc[r] : 0.f;
        st4<T>(&sm.Pm[i][16 * tj + 4 * g], acc);
      }
    }
    lds_barrier();
    if (split && ch + 1 < cend) {  // the low parts are consumed: their buffers take the next k, v
      dma_rows(sm.X[(ch + 1) & 1], kg, ch + 1);
      dma_rows(sm.Y[(ch + 1) & 1], vg, ch + 1);
    }

    // ---- O^T, second part: + V^T A^T
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const Frag<T> A = tr_frag<T>(&Vs[0][0], PQ, 32 * kk, cw, lane);  // V^T, own rows
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        if (kk == 1 && ti < 2) continue;
        const Frag<T> B = lds_frag<T, KORD_CONTIG>(&sm.Pm[0][0], PT, 16 * ti, 32 * kk, lane);
        mma(O[ti], A, B);
      }
    }
    T* og = static_cast<T*>(a.o);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      const int i = 16 * ti + l16;
      if (i < Lc) st4<T>(og + (tok0 + t0 + i) * D + cw + 4 * g, O[ti]);
    }

    // ---- carry update: S^T = diag(e^{B_63}) (S^T + (K e^-B)^T V)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const Frag<T> Bv = tr_frag<T>(&Vs[0][0], PQ, 32 * kk, cw, lane);  // V[t][own channel]
#pragma unroll
      for (int t0_ = 0; t0_ < NA; t0_ += 4) {
        Frag<T> Ap[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) Ap[u] = tr_frag<T>(&sm.Kp[0][0], PQ, 32 * kk, 16 * (t0_ + u), lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) mma(Sacc[t0_ + u], Ap[u], Bv);
      }
    }
#pragma unroll
    for (int t = 0; t < NA; ++t) Sacc[t] *= *reinterpret_cast<const f32x4*>(&sm.eBL[16 * t + 4 * g]);
    if (tid < D) {
      const float m = sm.m1[tid];
      sm.m0[tid] = m;
      const T mhi = (T)m;
      sm.Wt[2][tid] = mhi;
      sm.Wt[3][tid] = (T)(m - (float)mhi);
    }
    nb += Lc;
    lds_barrier();
    if (CC && ch + 1 < cend) {  // the carry at the next chunk's start, for the backward
      put_carry_row<D, T, NA>(a, chain, ch + 1, 0, cw + l16, g, Sacc);
      put_carry_row<D, T, NA>(a, chain, ch + 1, 1, cw + l16, g, Cacc);
      if (tid < D) put_carry_ksum<D, T>(a, chain, ch + 1, tid, sm.m0[tid]);
    }
  };
  int ch = cbeg;
  if (kSplit && ch < cend && nb == 0) chunk(ch++, std::true_type{});
  for (; ch < cend; ++ch) chunk(ch, std::false_type{});

  // ---- carry out (last segment of the chain)
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

// Records the caller's timing event `i` (if any) on the stream.
static hipError_t record_event(const FwdArgs& a, int i, hipStream_t s) {
  if (a.events == nullptr) return hipSuccess;
  return hipEventRecord(static_cast<hipEvent_t>(a.events[i]), s);
}

template <int D, typename T>
static hipError_t launch_gla(const FwdArgs& a, hipStream_t s) {
  const int chains = a.B * a.H;
  const int P = a.segments;
  const dim3 block(4 * D);
  if (record_event(a, 0, s) != hipSuccess) return hipErrorLaunchFailure;
  if (P > 1) {
    launch_gla_summary(a, s);
    if (record_event(a, 1, s) != hipSuccess) return hipErrorLaunchFailure;
    launch_gla_scan(a, s);
  } else if (record_event(a, 1, s) != hipSuccess) {
    return hipErrorLaunchFailure;
  }
  if (record_event(a, 2, s) != hipSuccess) return hipErrorLaunchFailure;
  hipError_t e;
  if (D == 128 && sizeof(T) == 2 && !(a.flags & kFlagNormalizeKeys)) {
    e = launch_gla_pipe(a, s);
  } else {
    if (a.chunk_carry != nullptr)
      hipLaunchKernelGGL((gla_main_kernel<D, T, true>), dim3((unsigned)(chains * P)), block, 0, s, a);
    else
      hipLaunchKernelGGL((gla_main_kernel<D, T, false>), dim3((unsigned)(chains * P)), block, 0, s, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  return record_event(a, 3, s);
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.rule == 1) return launch_gdn(a, s);
  if (a.dtype == 1) {
    if (a.d == 128) return launch_gla<128, __bf16>(a, s);
    if (a.d == 64) return launch_gla<64, __bf16>(a, s);
  } else {
    if (a.d == 64) return launch_gla<64, float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
