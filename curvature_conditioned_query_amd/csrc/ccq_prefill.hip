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
// Kernel layout.  One workgroup of D/32 waves per (chain, segment).  Wave w owns the
// 32-channel slice [32w, 32w+32) of d:
//  - both fp32 carries live in its MFMA accumulators: tile (a, jm) of C holds
//    C[16a+4g+r][32w+16jm+l] and tile (a, jm) of S holds S^T[16a+4g+r][32w+16jm+l]
//    (l = lane % 16, g = lane / 16, r = element).  Read as an A operand, a pair of such
//    tiles is S (resp. C, which is symmetric) restricted to the wave's rows, so the carry
//    feeds the read-side MFMAs straight from registers and never leaves them inside a chain;
//  - it loads its channels of the next chunk's q, k, v and log decay from HBM into MFMA
//    fragments while the current chunk is computed, and stages them without scalar LDS
//    traffic: transposes are MFMAs against an identity fragment (exact: x * 1 + 0), and the
//    cumulative decay over tokens is an MFMA against a lower-triangular ones fragment.
#include "ccq_device.hpp"
#include "ccq_internal.hpp"

namespace ccq {

constexpr int kL = 64;  // chunk length

// Workspace slot of one (chain, segment): S [D][D] | C [D][D] | ksum [D] | log decay [D], fp32.
size_t fwd_slot_bytes(int d) { return (size_t)(2 * d * d + 2 * d) * sizeof(float); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D, typename T>
struct Cfg {
  static constexpr int NW = D / 32;        // waves per workgroup
  static constexpr int NTH = 64 * NW;      // threads per workgroup (= 2D)
  static constexpr int NA = D / 16;        // 16-wide tiles along d
  static constexpr int NK = D / 32;        // K-steps of 32 along d
  static constexpr int VE = 16 / sizeof(T);  // elements per 16-byte vector
  static constexpr int NV = (kL * D) / (NTH * VE);  // 16-byte vectors per thread per tile
  static constexpr int PAD = 16 / sizeof(T);
  static constexpr int PQ = D + PAD;   // pitch of [64][D] tiles
  static constexpr int PT = kL + PAD;  // pitch of [D][64] and [64][64] tiles
};

template <int D, typename T>
struct Smem {
  using C_ = Cfg<D, T>;
  static constexpr int LO = (sizeof(T) == 2) ? kL : 1;  // rows of the bf16 lo tiles
  T Qs[kL][C_::PQ];   // q rows
  T Qa[kL][C_::PQ];   // q_clean * e^B (hi part for bf16)
  T Qalo[LO][C_::PQ]; // bf16 only: lo part of q_clean * e^B
  T Ks[kL][C_::PQ];   // k rows; later k * e^-B (hi part), in place
  T Klo[LO][C_::PQ];  // bf16 only: lo part of k * e^-B
  T Kt[D][C_::PT];    // k^T
  T Kpt[D][C_::PT];   // (k * e^-B)^T
  T Vt[D][C_::PT];    // v^T
  T Pm[kL][C_::PT];   // tril(Q K^T - c 1^T), then the masked intra-chunk attention matrix
  T Wt[16][C_::PQ];   // rows: w_lambda hi, lo; key sum hi, lo; zeros (B operand of q . [w, m0])
  float m0[D], m1[D], eBL[D], ldec[D];
  f32x4 tok[kL];      // per token: lambda, 1/n, sq/n^2, gate logit + b
};

// Lower-triangular 16x16 tiles of a 64x64 token-token matrix, (row tile, col tile).
__constant__ int8_t kTri[10][2] = {{0, 0}, {1, 0}, {1, 1}, {2, 0}, {2, 1}, {2, 2}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};

template <typename T>
__device__ __forceinline__ void st4(T* p, const f32x4& v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}

template <typename T>
__device__ __forceinline__ f32x4 ld4(const T* p) {
  if constexpr (sizeof(T) == 2) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  } else {
    return *reinterpret_cast<const f32x4*>(p);
  }
}

// 16-byte vector of T as floats (VE = 8 for bf16, 4 for fp32).
template <typename T>
__device__ __forceinline__ void unpack(const u32x4& v, float* out) {
  if constexpr (sizeof(T) == 2) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = (float)b[e];
  } else {
    const f32x4 f = __builtin_bit_cast(f32x4, v);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = f[e];
  }
}


// 8 elements of one row from global memory (16 bytes for bf16, 32 for fp32), or zeros.
template <typename T>
__device__ __forceinline__ Frag<T> gload_frag(const T* p, bool ok) {
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    f.v = __builtin_bit_cast(bf16x8, ok ? *reinterpret_cast<const u32x4*>(p) : z);
  } else {
    const f32x4 lo = ok ? *reinterpret_cast<const f32x4*>(p) : zero4();
    const f32x4 hi = ok ? *reinterpret_cast<const f32x4*>(p + 4) : zero4();
#pragma unroll
    for (int e = 0; e < 4; ++e) { f.v[e] = lo[e]; f.v[4 + e] = hi[e]; }
  }
  return f;
}

template <typename T>
__device__ __forceinline__ void st_frag(T* p, const Frag<T>& f) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x8*>(p) = f.v;
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{f.v[0], f.v[1], f.v[2], f.v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{f.v[4], f.v[5], f.v[6], f.v[7]};
  }
}

template <typename T>
__device__ __forceinline__ T cvt(float x) { return (T)x; }

// Identity slice in KORD_CONTIG order: element e of lane (g, l) is 1 where 8g + e == l + 16h.
// As a B operand against row fragments X[t][k] it yields X[t][16h + n] in the accumulator
// (4 consecutive tokens per lane); as an A operand against row fragments used as B it
// yields X[t][16h + 4g + r] (4 consecutive channels per lane).
template <typename T>
__device__ __forceinline__ Frag<T> ident_frag(int h, int lane) {
  Frag<T> f;
  const int l = lane & 15, g = lane >> 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = cvt<T>((8 * g + e == l + 16 * h) ? 1.0f : 0.0f);
  return f;
}

// Lower-triangular ones L[t][t'] = (t' <= t) as the A operand, in KORD_ACC order over
// t' = 32 kk + 16 (e / 4) + 4 g + e % 4, with t = 16 ti + (lane % 16).
template <typename T>
__device__ __forceinline__ Frag<T> ltri_frag(int ti, int kk, int lane) {
  Frag<T> f;
  const int t = 16 * ti + (lane & 15), g = lane >> 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int tp = 32 * kk + 16 * (e >> 2) + 4 * g + (e & 3);
    f.v[e] = cvt<T>(tp <= t ? 1.0f : 0.0f);
  }
  return f;
}

__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4& v) {
  return bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}

// Ones where token j <= token i, as the B fragment of the inclusive prefix over tokens:
// B[k = j][n = i] with i = 16 ti + (lane % 16), j = 32 kk + 8 g + e (KORD_CONTIG).
template <typename T>
__device__ __forceinline__ Frag<T> causal_ones(int ti, int kk, int lane) {
  Frag<T> f;
  const int i = 16 * ti + (lane & 15);
  const int j0 = 32 * kk + 8 * (lane >> 4);
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = (__bf16)((j0 + e <= i) ? 1.0f : 0.0f);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = (j0 + e <= i) ? 1.0f : 0.0f;
  }
  return f;
}

// MODE 0: full read (o for every token) from the segment's carry-in, carry out at the end.
// MODE 1: segment summary from a zero carry (C, S, ksum and total log decay), no outputs.
template <int D, typename T, int MODE>
__global__ __launch_bounds__(2 * D) void gla_prefill_kernel(FwdArgs a) {
  using C_ = Cfg<D, T>;
  constexpr int NW = C_::NW, NA = C_::NA, NK = C_::NK;
  constexpr int PQ = C_::PQ, PT = C_::PT;
  constexpr bool MAIN = (MODE == 0);
  constexpr bool kSplit = MAIN && sizeof(T) == 2;  // hi/lo operands for the intra term
  __shared__ Smem<D, T> sm;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int cw = 32 * w;  // first channel of this wave's slice
  const int P = a.segments, cps = a.chunks_per_segment;
  const int per_chain = MAIN ? P : P - 1;
  const int chain = blockIdx.x / per_chain, seg = blockIdx.x % per_chain;
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
  f32x4 Cacc[NA][2], Sacc[NA][2];
  const float* Sin = nullptr;
  const float* Cin = nullptr;
  const float* min_ = nullptr;
  if constexpr (MAIN) {
    if (P > 1) {
      const float* slot = slots + ((size_t)chain * P + seg) * slot_f;
      Sin = slot;
      Cin = slot + (size_t)D * D;
      min_ = slot + 2 * (size_t)D * D;
    } else if (a.S0 != nullptr) {
      Sin = a.S0 + (size_t)chain * D * D;
      Cin = a.C0 + (size_t)chain * D * D;
      min_ = a.ksum0 + (size_t)chain * D;
    }
  }
#pragma unroll
  for (int t = 0; t < NA; ++t) {
#pragma unroll
    for (int jm = 0; jm < 2; ++jm) {
      const int row = cw + 16 * jm + l16;
      const int col = 16 * t + 4 * g;
      Sacc[t][jm] = Sin ? *reinterpret_cast<const f32x4*>(Sin + (size_t)row * D + col) : zero4();
      Cacc[t][jm] = Cin ? *reinterpret_cast<const f32x4*>(Cin + (size_t)row * D + col) : zero4();
    }
  }
  int64_t nb = (int64_t)cbeg * kL;  // tokens before this chunk (count base)
  if constexpr (MAIN) {
    if (a.n0 != nullptr) nb += a.n0[chain];
  }
  float b_lam = 0.f;
  if constexpr (MAIN) b_lam = a.b_lambda[h];

  if (tid < D) {
    const int c = tid;
    const float m = min_ ? min_[c] : 0.f;
    sm.m0[c] = m;
    sm.ldec[c] = 0.f;
    if constexpr (MAIN) {
      const float wv = a.w_lambda[(size_t)h * D + c];
      const T whi = (T)wv, mhi = (T)m;
      sm.Wt[0][c] = whi;
      sm.Wt[1][c] = (T)(wv - (float)whi);
      sm.Wt[2][c] = mhi;
      sm.Wt[3][c] = (T)(m - (float)mhi);
#pragma unroll
      for (int r = 4; r < 16; ++r) sm.Wt[r][c] = (T)0.f;
    }
  }
  if constexpr (MAIN) {
    for (int e = tid; e < kL * PT; e += 2 * D) (&sm.Pm[0][0])[e] = (T)0.f;
  }

  // ---- register prefetch: this wave's 32 channels of one chunk, as MFMA row fragments
  // (lane: token 16 ti + l16, channels cw + 8g .. cw + 8g + 7); rows past the end are zero.
  Frag<T> fq[4], fk[4], fv[4], fg[4];
  auto prefetch = [&](int ch) {
    const int t0 = ch * kL;
    const int Lc = min(kL, a.T - t0);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      const int t = 16 * ti + l16;
      const bool ok = t < Lc;
      const size_t off = ok ? (tok0 + t0 + t) * D + cw + 8 * g : 0;
      if constexpr (MAIN) fq[ti] = gload_frag<T>(qg + off, ok);
      fk[ti] = gload_frag<T>(kg + off, ok);
      fv[ti] = gload_frag<T>(vg + off, ok);
      fg[ti] = gload_frag<T>(gg + off, ok);
    }
  };
  if (cbeg < cend) prefetch(cbeg);

  const Frag<T> I0 = ident_frag<T>(0, lane), I1 = ident_frag<T>(1, lane);

  for (int ch = cbeg; ch < cend; ++ch) {
    const int t0 = ch * kL;
    const int Lc = min(kL, a.T - t0);

    // ---- stage this wave's channels: rows, transposes, cumulative decay, k e^-B transposed
    {
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const int t = 16 * ti + l16;
        if constexpr (MAIN) st_frag<T>(&sm.Qs[t][cw + 8 * g], fq[ti]);
        st_frag<T>(&sm.Ks[t][cw + 8 * g], fk[ti]);
        f32x4 V0 = zero4(), V1 = zero4();
        mma(V0, fv[ti], I0);
        mma(V1, fv[ti], I1);
        st4<T>(&sm.Vt[cw + l16][16 * ti + 4 * g], V0);
        st4<T>(&sm.Vt[cw + 16 + l16][16 * ti + 4 * g], V1);
      }
      // one 16-channel half at a time keeps the transposes' registers down
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const Frag<T>& Ih = hh ? I1 : I0;
        const int c = cw + 16 * hh + l16;
        f32x4 KT[4], GT[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          KT[ti] = GT[ti] = zero4();
          mma(KT[ti], fk[ti], Ih);  // KT[ti][r] = k at token 16 ti + 4 g + r, channel c
          mma(GT[ti], fg[ti], Ih);
          st4<T>(&sm.Kt[c][16 * ti + 4 * g], KT[ti]);
        }
        const Frag<T> G0 = acc_frag<T>(GT[0], GT[1]);
        const Frag<T> G1 = acc_frag<T>(GT[2], GT[3]);
        float ks = 0.f;
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          f32x4 Bc = zero4();
          mma(Bc, ltri_frag<T>(ti, 0, lane), G0);
          if (ti >= 2) mma(Bc, ltri_frag<T>(ti, 1, lane), G1);
          // Bc[r] = cumulative log decay at token 16 ti + 4 g + r, channel c
          f32x4 kp;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            kp[r] = KT[ti][r] * __expf(-Bc[r]);
            ks += KT[ti][r];
          }
          st4<T>(&sm.Kpt[c][16 * ti + 4 * g], kp);
          if (ti == 3 && g == 3) {
            sm.eBL[c] = __expf(Bc[3]);
            sm.ldec[c] += Bc[3];
          }
        }
        ks += __shfl_xor(ks, 16, 64);
        ks += __shfl_xor(ks, 32, 64);
        if (g == 0) sm.m1[c] = sm.m0[c] + ks;
      }
      // the summary pass has registers to spare: its next chunk's loads go out now
      if constexpr (!MAIN) {
        if (ch + 1 < cend) prefetch(ch + 1);
      }
    }
    __syncthreads();

    if constexpr (MAIN) {
      // ---- one 16-token row tile per wave: gate logit and m0 . q, then the row tile of
      // P = Q K^T, its inclusive row sums, and Pm = tril(P - c 1^T) with c_i = sq_i / n_i
      for (int it = w; it < 4; it += NW) {
        {
          f32x4 acc = zero4();  // [q] x [w_hi, w_lo, m0_hi, m0_lo]
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) {
            const Frag<T> A = lds_frag<T, KORD_CONTIG>(&sm.Qs[0][0], PQ, 16 * it, 32 * kk, lane);
            const Frag<T> B = lds_frag<T, KORD_CONTIG>(&sm.Wt[0][0], PQ, 0, 32 * kk, lane);
            mma(acc, A, B);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = acc[r] + __shfl_down(acc[r], 1, 64);  // hi + lo columns
            const int i = 16 * it + 4 * g + r;
            if (l16 == 0) sm.tok[i][3] = x + b_lam;
            if (l16 == 2) sm.tok[i][1] = x;  // m0 . q, parked until the row sums are known
          }
        }
        const int i = 16 * it + l16;  // this lane's token in the P tiles below
        f32x4 Pt[4];
        float rs = 0.f;
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
          Pt[tj] = zero4();
          if (tj > it) continue;
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) {
            const Frag<T> A = lds_frag<T, KORD_CONTIG>(&sm.Ks[0][0], PQ, 16 * tj, 32 * kk, lane);
            const Frag<T> B = lds_frag<T, KORD_CONTIG>(&sm.Qs[0][0], PQ, 16 * it, 32 * kk, lane);
            mma(Pt[tj], A, B);
          }
          // Pt[tj][r] = P[i][16 tj + 4 g + r]
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool keep = 16 * tj + 4 * g + r <= i;
            Pt[tj][r] = keep ? Pt[tj][r] : 0.f;
            rs += Pt[tj][r];
          }
        }
        rs += __shfl_xor(rs, 16, 64);
        rs += __shfl_xor(rs, 32, 64);
        const float gate = sm.tok[i][3];
        const float sq = sm.tok[i][1] + rs;
        const float inv_n = __builtin_amdgcn_rcpf((float)(nb + i + 1));
        const float cbar = sq * inv_n;
#pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
          if (tj > it) continue;
          f32x4 pc;
#pragma unroll
          for (int r = 0; r < 4; ++r) pc[r] = (16 * tj + 4 * g + r <= i) ? Pt[tj][r] - cbar : 0.f;
          st4<T>(&sm.Pm[i][16 * tj + 4 * g], pc);
        }
        if (g == 0) sm.tok[i] = f32x4{sigmoidf(gate), inv_n, cbar * inv_n, gate};
      }
      __syncthreads();

      // ---- cleaned query for the wave's 32 channels, and k * e^-B
      {
        f32x4 R[2][4];
#pragma unroll
        for (int jm = 0; jm < 2; ++jm)
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) R[jm][ti] = zero4();
        // Q C0 (A operand straight from the carry accumulators)
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const Frag<T> A0 = acc_frag<T>(Cacc[2 * kk][0], Cacc[2 * kk + 1][0]);
          const Frag<T> A1 = acc_frag<T>(Cacc[2 * kk][1], Cacc[2 * kk + 1][1]);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            const Frag<T> B = lds_frag<T, KORD_ACC>(&sm.Qs[0][0], PQ, 16 * ti, 32 * kk, lane);
            mma(R[0][ti], A0, B);
            mma(R[1][ti], A1, B);
          }
        }
        // + tril(P - c 1^T) K
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const Frag<T> A0 = lds_frag<T, KORD_CONTIG>(&sm.Kt[0][0], PT, cw, 32 * kk, lane);
          const Frag<T> A1 = lds_frag<T, KORD_CONTIG>(&sm.Kt[0][0], PT, cw + 16, 32 * kk, lane);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            if (kk == 1 && ti < 2) continue;  // tokens 32..63 never precede tokens 0..31
            const Frag<T> Bp = lds_frag<T, KORD_CONTIG>(&sm.Pm[0][0], PT, 16 * ti, 32 * kk, lane);
            mma(R[0][ti], A0, Bp);
            mma(R[1][ti], A1, Bp);
          }
        }
        // R[jm][ti][r]: channel cw + 16 jm + 4 g + r, token 16 ti + l16.  The cumulative decay
        // in the same layout, from the chunk's log-decay rows still in registers:
        // Bc^T = (G^T)(L^T) with G^T read off the transposes of the rows.
#pragma unroll
        for (int jm = 0; jm < 2; ++jm) {
          const Frag<T>& Ih = jm ? I1 : I0;
          f32x4 GT[4];
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            GT[ti] = zero4();
            mma(GT[ti], fg[ti], Ih);
          }
          const Frag<T> Ga = acc_frag<T>(GT[0], GT[1]);
          const Frag<T> Gb = acc_frag<T>(GT[2], GT[3]);
          const int m = cw + 16 * jm + 4 * g;
          const f32x4 m04 = *reinterpret_cast<const f32x4*>(&sm.m0[m]);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            f32x4 BT = zero4();
            mma(BT, Ga, ltri_frag<T>(ti, 0, lane));
            if (ti >= 2) mma(BT, Gb, ltri_frag<T>(ti, 1, lane));
            const int i = 16 * ti + l16;
            const f32x4 ts = sm.tok[i];  // lambda, 1/n, sq/n^2
            const f32x4 q4 = ld4<T>(&sm.Qs[i][m]);
            f32x4 qa;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float u = R[jm][ti][r] * ts[1] - m04[r] * ts[2];
              qa[r] = (q4[r] - ts[0] * u) * __expf(BT[r]);
            }
            // k * e^-B at the same (token, channel) positions: identity A against the k rows
            f32x4 KC = zero4();
            mma(KC, Ih, fk[ti]);
            f32x4 kp;
#pragma unroll
            for (int r = 0; r < 4; ++r) kp[r] = KC[r] * __expf(-BT[r]);
            // bf16: hi + lo (the intra-chunk attention is a sum of few, possibly cancelling
            // products when little of the sequence has been read)
            const bf16x4 qh = to_bf16x4(qa), kh = to_bf16x4(kp);
            if constexpr (kSplit) {
              *reinterpret_cast<bf16x4*>(&sm.Qa[i][m]) = qh;
              *reinterpret_cast<bf16x4*>(&sm.Ks[i][m]) = kh;
              f32x4 ql, kl;
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                ql[r] = qa[r] - (float)qh[r];
                kl[r] = kp[r] - (float)kh[r];
              }
              st4<T>(&sm.Qalo[i][m], ql);
              st4<T>(&sm.Klo[i][m], kl);
            } else {
              st4<T>(&sm.Qa[i][m], qa);
              st4<T>(&sm.Ks[i][m], kp);
            }
          }
        }
      }
      __syncthreads();
      // the chunk's row fragments are consumed: next chunk's loads go out now, behind the
      // intra-chunk read, the output store and the carry update
      if (ch + 1 < cend) prefetch(ch + 1);

      // ---- intra-chunk attention (Qc e^B)(K e^-B)^T on the lower tiles -> Pm (masked)
      for (int idx = w; idx < 10; idx += NW) {
        const int ti = kTri[idx][0], tj = kTri[idx][1];
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const Frag<T> A = lds_frag<T, KORD_CONTIG>(&sm.Ks[0][0], PQ, 16 * tj, 32 * kk, lane);
          const Frag<T> B = lds_frag<T, KORD_CONTIG>(&sm.Qa[0][0], PQ, 16 * ti, 32 * kk, lane);
          mma(acc, A, B);
          if constexpr (kSplit) {
            const Frag<T> Al = lds_frag<T, KORD_CONTIG>(&sm.Klo[0][0], PQ, 16 * tj, 32 * kk, lane);
            const Frag<T> Bl = lds_frag<T, KORD_CONTIG>(&sm.Qalo[0][0], PQ, 16 * ti, 32 * kk, lane);
            mma(acc, A, Bl);
            mma(acc, Al, B);
          }
        }
        const int i = 16 * ti + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = (16 * tj + 4 * g + r <= i) ? acc[r] : 0.f;
        st4<T>(&sm.Pm[i][16 * tj + 4 * g], acc);
      }
      __syncthreads();

      // ---- O^T for the wave's 32 value rows: S0 (Qc e^B)^T + V^T A^T
      f32x4 O[2][4];
#pragma unroll
      for (int jm = 0; jm < 2; ++jm)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) O[jm][ti] = zero4();
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const Frag<T> A0 = acc_frag<T>(Sacc[2 * kk][0], Sacc[2 * kk + 1][0]);
        const Frag<T> A1 = acc_frag<T>(Sacc[2 * kk][1], Sacc[2 * kk + 1][1]);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          const Frag<T> B = lds_frag<T, KORD_ACC>(&sm.Qa[0][0], PQ, 16 * ti, 32 * kk, lane);
          mma(O[0][ti], A0, B);
          mma(O[1][ti], A1, B);
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Frag<T> A0 = lds_frag<T, KORD_CONTIG>(&sm.Vt[0][0], PT, cw, 32 * kk, lane);
        const Frag<T> A1 = lds_frag<T, KORD_CONTIG>(&sm.Vt[0][0], PT, cw + 16, 32 * kk, lane);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          if (kk == 1 && ti < 2) continue;
          const Frag<T> B = lds_frag<T, KORD_CONTIG>(&sm.Pm[0][0], PT, 16 * ti, 32 * kk, lane);
          mma(O[0][ti], A0, B);
          mma(O[1][ti], A1, B);
        }
      }
      T* og = static_cast<T*>(a.o);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const int i = 16 * ti + l16;
        if (i < Lc) {
#pragma unroll
          for (int jm = 0; jm < 2; ++jm) st4<T>(og + (tok0 + t0 + i) * D + cw + 16 * jm + 4 * g, O[jm][ti]);
        }
      }
    }

    // ---- carry update: C += K^T K;  S^T = diag(e^{B_63}) (S^T + (K e^-B)^T V)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const Frag<T> Bk0 = lds_frag<T, KORD_CONTIG>(&sm.Kt[0][0], PT, cw, 32 * kk, lane);
      const Frag<T> Bk1 = lds_frag<T, KORD_CONTIG>(&sm.Kt[0][0], PT, cw + 16, 32 * kk, lane);
      const Frag<T> Bv0 = lds_frag<T, KORD_CONTIG>(&sm.Vt[0][0], PT, cw, 32 * kk, lane);
      const Frag<T> Bv1 = lds_frag<T, KORD_CONTIG>(&sm.Vt[0][0], PT, cw + 16, 32 * kk, lane);
#pragma unroll
      for (int t = 0; t < NA; ++t) {
        const Frag<T> Ak = lds_frag<T, KORD_CONTIG>(&sm.Kt[0][0], PT, 16 * t, 32 * kk, lane);
        const Frag<T> Ap = lds_frag<T, KORD_CONTIG>(&sm.Kpt[0][0], PT, 16 * t, 32 * kk, lane);
        mma(Cacc[t][0], Ak, Bk0);
        mma(Cacc[t][1], Ak, Bk1);
        mma(Sacc[t][0], Ap, Bv0);
        mma(Sacc[t][1], Ap, Bv1);
      }
    }
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      const f32x4 e4 = *reinterpret_cast<const f32x4*>(&sm.eBL[16 * t + 4 * g]);
      Sacc[t][0] *= e4;
      Sacc[t][1] *= e4;
    }
    if (tid < D) {
      const float m = sm.m1[tid];
      sm.m0[tid] = m;
      if constexpr (MAIN) {
        const T mhi = (T)m;
        sm.Wt[2][tid] = mhi;
        sm.Wt[3][tid] = (T)(m - (float)mhi);
      }
    }
    nb += Lc;
    __syncthreads();
  }

  // ---- carry out
  float* Sout = nullptr;
  float* Cout = nullptr;
  float* mout = nullptr;
  float* ldout = nullptr;
  if constexpr (MAIN) {
    if (seg == P - 1 && a.S_out != nullptr) {
      Sout = a.S_out + (size_t)chain * D * D;
      Cout = a.C_out + (size_t)chain * D * D;
      mout = a.ksum_out + (size_t)chain * D;
      if (tid == 0) a.n_out[chain] = nb;
    }
  } else {
    float* slot = slots + ((size_t)chain * P + seg) * slot_f;
    Sout = slot;
    Cout = slot + (size_t)D * D;
    mout = slot + 2 * (size_t)D * D;
    ldout = mout + D;
  }
  if (Sout != nullptr) {
#pragma unroll
    for (int t = 0; t < NA; ++t) {
#pragma unroll
      for (int jm = 0; jm < 2; ++jm) {
        const int row = cw + 16 * jm + l16;
        const int col = 16 * t + 4 * g;
        *reinterpret_cast<f32x4*>(Sout + (size_t)row * D + col) = Sacc[t][jm];
        *reinterpret_cast<f32x4*>(Cout + (size_t)row * D + col) = Cacc[t][jm];
      }
    }
    if (tid < D) {
      mout[tid] = sm.m0[tid];
      if (ldout != nullptr) ldout[tid] = sm.ldec[tid];
    }
  }
}

// Exclusive scan of segment summaries into carry-ins, in place.  Slot p holds the summary
// of segment p (p < P-1) and receives the carry-in of segment p (p <= P-1):
//   carry_in[0] = carry0;  carry_in[p+1] = (S_in[p] diag(e^{ldec[p]}) + dS[p], C + dC, m + dm).
// One thread per 4 consecutive floats of the S | C | ksum part of a slot.
template <int D>
__global__ __launch_bounds__(256) void gla_scan_kernel(FwdArgs a) {
  const int chain = blockIdx.y;
  const int P = a.segments;
  const size_t slot_f = 2 * (size_t)D * D + 2 * D;
  const int nf4 = (2 * D * D + D) / 4;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= nf4) return;
  const size_t f = (size_t)idx * 4;
  float* base = static_cast<float*>(a.workspace) + (size_t)chain * P * slot_f;
  const bool isS = f < (size_t)D * D;
  const int col = (int)(f % D);
  f32x4 run = zero4();
  if (a.S0 != nullptr) {
    const float* src;
    if (isS)
      src = a.S0 + (size_t)chain * D * D + f;
    else if (f < 2 * (size_t)D * D)
      src = a.C0 + (size_t)chain * D * D + (f - (size_t)D * D);
    else
      src = a.ksum0 + (size_t)chain * D + (f - 2 * (size_t)D * D);
    run = *reinterpret_cast<const f32x4*>(src);
  }
  for (int p = 0; p < P; ++p) {
    float* slot = base + (size_t)p * slot_f;
    const f32x4 sum = (p < P - 1) ? *reinterpret_cast<const f32x4*>(slot + f) : zero4();
    *reinterpret_cast<f32x4*>(slot + f) = run;
    if (p < P - 1) {
      if (isS) {
        const f32x4 ld = *reinterpret_cast<const f32x4*>(slot + 2 * (size_t)D * D + D + col);
        run = run * f32x4{__expf(ld[0]), __expf(ld[1]), __expf(ld[2]), __expf(ld[3])};
      }
      run += sum;
    }
  }
}

template <int D, typename T>
static hipError_t launch_gla(const FwdArgs& a, hipStream_t s) {
  const int chains = a.B * a.H;
  const int P = a.segments;
  if (P > 1) {
    hipLaunchKernelGGL((gla_prefill_kernel<D, T, 1>), dim3((unsigned)(chains * (P - 1))), dim3(2 * D), 0, s, a);
    const int nf4 = (2 * D * D + D) / 4;
    hipLaunchKernelGGL((gla_scan_kernel<D>), dim3((unsigned)((nf4 + 255) / 256), (unsigned)chains), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL((gla_prefill_kernel<D, T, 0>), dim3((unsigned)(chains * P)), dim3(2 * D), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.rule != 0) return hipErrorNotSupported;
  if (a.dtype == 1) {
    if (a.d == 128) return launch_gla<128, __bf16>(a, s);
    if (a.d == 64) return launch_gla<64, __bf16>(a, s);
  } else {
    if (a.d == 64) return launch_gla<64, float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
