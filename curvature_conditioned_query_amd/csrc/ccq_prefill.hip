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
//   s_i  = m0 + sum_{j<=i} k_j,  n_i = n0 + i + 1
//   R    = Q C0 + tril_incl(Q K^T) K                     (row i = C_i q_i)
//   u_i  = R_i / n_i - s_i (s_i . q_i) / n_i^2           (row i = Sigma_i q_i)
//   qc_i = q_i - lambda_i u_i
//   B_i  = sum_{j<=i} g_j  (per channel, chunk-local)
//   O    = (Qc * e^B) S0^T + tril_incl((Qc * e^B)(K * e^-B)^T) V
//   S_L  = (S0 + V^T (K * e^-B)) diag(e^{B_63})
//   C0 += K^T K;  m0 += sum_j k_j;  n0 += L
// The intra-chunk decay is factored with the chunk start as reference, so e^{-B} stays
// finite while B > -80 inside a chunk (the documented precondition).
//
// Kernel layout.  One workgroup of D/32 waves per (chain, segment).  Wave w keeps the
// 32-wide slice [32w, 32w+32) of both fp32 carries as MFMA accumulators: tile (a, jm) of
// C holds C[16a+4g+r][32w+16jm+l] and tile (a, jm) of S holds S^T[16a+4g+r][32w+16jm+l]
// (lane l = lane % 16, g = lane / 16, r = element).  Read as an A operand, a pair of such
// tiles is S (resp. C, which is symmetric) restricted to the wave's rows, so the carry
// feeds the read-side MFMAs straight from registers and never touches LDS or HBM inside
// the chain.  Chunk tiles are staged in LDS; the next chunk's global loads are issued into
// registers before the current chunk is computed.
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
  static constexpr int PB = D + 4;     // pitch of the fp32 [64][D] decay tile
};

template <int D, typename T>
struct Smem {
  using C_ = Cfg<D, T>;
  T Qs[kL][C_::PQ];   // q rows
  T Qa[kL][C_::PQ];   // q_clean * e^B
  T Ks[kL][C_::PQ];   // k rows, then k * e^-B in place
  T Kt[D][C_::PT];    // k^T
  T Kpt[D][C_::PT];   // (k * e^-B)^T
  T Vt[D][C_::PT];    // v^T
  T Pm[kL][C_::PT];   // masked Q K^T, then the masked intra-chunk attention matrix
  float Bs[kL][C_::PB];  // chunk-local cumulative log decay (inclusive)
  float w[D], m0[D], m1[D], eBL[D], ldec[D];
  float lam[kL], mq[kL], psum[4][kL];
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
  constexpr int NW = C_::NW, NTH = C_::NTH, NA = C_::NA, NK = C_::NK, VE = C_::VE, NV = C_::NV;
  constexpr int PQ = C_::PQ, PT = C_::PT, PB = C_::PB;
  constexpr bool MAIN = (MODE == 0);
  constexpr bool kSplit = MAIN && sizeof(T) == 2;  // hi/lo operands for the intra term
  static_assert(kL * PQ * sizeof(T) <= kL * PB * sizeof(float), "lo tile must fit the decay tile");
  __shared__ Smem<D, T> sm;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
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
      const int row = 32 * w + 16 * jm + l16;
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

  for (int c = tid; c < D; c += NTH) {
    sm.m0[c] = min_ ? min_[c] : 0.f;
    sm.ldec[c] = 0.f;
    if constexpr (MAIN) sm.w[c] = a.w_lambda[(size_t)h * D + c];
  }
  if constexpr (MAIN) {
    for (int e = tid; e < kL * PT; e += NTH) (&sm.Pm[0][0])[e] = (T)0.f;
    for (int e = tid; e < 4 * kL; e += NTH) (&sm.psum[0][0])[e] = 0.f;
  }

  // ---- register prefetch of one chunk (rows >= Lc are zero)
  u32x4 rq[NV], rk[NV], rv[NV], rg[NV];
  auto prefetch = [&](int ch) {
    const int t0 = ch * kL;
    const int Lc = min(kL, a.T - t0);
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int vi = tid + j * NTH;
      const int t = (vi * VE) / D, c = (vi * VE) % D;
      const size_t off = (tok0 + t0 + t) * D + c;
      const bool ok = t < Lc;
      const u32x4 z = {0u, 0u, 0u, 0u};
      if constexpr (MAIN) rq[j] = ok ? *reinterpret_cast<const u32x4*>(qg + off) : z;
      rk[j] = ok ? *reinterpret_cast<const u32x4*>(kg + off) : z;
      rv[j] = ok ? *reinterpret_cast<const u32x4*>(vg + off) : z;
      rg[j] = ok ? *reinterpret_cast<const u32x4*>(gg + off) : z;
    }
  };
  if (cbeg < cend) prefetch(cbeg);

  f32x4 qlo[4][2];
  float klo[NV][VE];
  for (int ch = cbeg; ch < cend; ++ch) {
    const int t0 = ch * kL;
    const int Lc = min(kL, a.T - t0);

    // ---- stage the chunk: q, k rows; k^T, v^T; raw log decay (fp32)
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int vi = tid + j * NTH;
      const int t = (vi * VE) / D, c = (vi * VE) % D;
      if constexpr (MAIN) *reinterpret_cast<u32x4*>(&sm.Qs[t][c]) = rq[j];
      *reinterpret_cast<u32x4*>(&sm.Ks[t][c]) = rk[j];
      float kf[VE], vf[VE], gf[VE];
      unpack<T>(rk[j], kf);
      unpack<T>(rv[j], vf);
      unpack<T>(rg[j], gf);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        sm.Kt[c + e][t] = (T)kf[e];
        sm.Vt[c + e][t] = (T)vf[e];
        sm.Bs[t][c + e] = gf[e];
      }
    }
    __syncthreads();
    if (ch + 1 < cend) prefetch(ch + 1);

    // ---- per-token gate and m0 . q  (NW lanes per token, 32 channels each)
    if constexpr (MAIN) {
      const int i = w * (kL / NW) + lane / NW;
      const int p = lane % NW;
      float wq = 0.f, mq = 0.f;
#pragma unroll 8
      for (int e = 0; e < 32; ++e) {
        const int c = 32 * p + e;
        const float qv = (float)sm.Qs[i][c];
        wq += sm.w[c] * qv;
        mq += sm.m0[c] * qv;
      }
      wq = group_sum<NW>(wq);
      mq = group_sum<NW>(mq);
      if (p == 0) {
        sm.lam[i] = sigmoidf(wq + b_lam);
        sm.mq[i] = mq;
      }
    }
    // ---- cumulative log decay per channel, key sum, chunk decay e^{B_63}
    if (tid < D) {
      const int c = tid;
      float run = 0.f, ks = 0.f;
#pragma unroll 16
      for (int t = 0; t < kL; ++t) {
        run += sm.Bs[t][c];
        sm.Bs[t][c] = run;
        ks += (float)sm.Kt[c][t];
      }
      sm.m1[c] = sm.m0[c] + ks;
      sm.eBL[c] = __expf(run);
      sm.ldec[c] += run;
    }
    // ---- P^T = K Q^T on the lower tiles -> Pm[i][j] (masked, j <= i) and row sums
    if constexpr (MAIN) {
      for (int idx = w; idx < 10; idx += NW) {
        const int ti = kTri[idx][0], tj = kTri[idx][1];
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const Frag<T> A = lds_frag<T, KORD_CONTIG>(&sm.Ks[0][0], PQ, 16 * tj, 32 * kk, lane);
          const Frag<T> B = lds_frag<T, KORD_CONTIG>(&sm.Qs[0][0], PQ, 16 * ti, 32 * kk, lane);
          mma(acc, A, B);
        }
        const int i = 16 * ti + l16;
        float ps = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * tj + 4 * g + r;
          acc[r] = (j <= i) ? acc[r] : 0.f;
          ps += acc[r];
        }
        ps += __shfl_xor(ps, 16, 64);
        ps += __shfl_xor(ps, 32, 64);
        if (g == 0) sm.psum[tj][i] = ps;
        st4<T>(&sm.Pm[i][16 * tj + 4 * g], acc);
      }
    }
    __syncthreads();

    // ---- cleaned query for the wave's 32 channels (MAIN), k * e^-B in both layouts
    if constexpr (MAIN) {
      f32x4 R[2][4], Sp[2][4];
#pragma unroll
      for (int jm = 0; jm < 2; ++jm)
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) R[jm][ti] = Sp[jm][ti] = zero4();
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
      // tril(Q K^T) K and the inclusive key prefix sum_{j<=i} k_j
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Frag<T> A0 = lds_frag<T, KORD_CONTIG>(&sm.Kt[0][0], PT, 32 * w, 32 * kk, lane);
        const Frag<T> A1 = lds_frag<T, KORD_CONTIG>(&sm.Kt[0][0], PT, 32 * w + 16, 32 * kk, lane);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          if (kk == 1 && ti < 2) continue;  // tokens 32..63 never precede tokens 0..31
          const Frag<T> Bp = lds_frag<T, KORD_CONTIG>(&sm.Pm[0][0], PT, 16 * ti, 32 * kk, lane);
          const Frag<T> Bo = causal_ones<T>(ti, kk, lane);
          mma(R[0][ti], A0, Bp);
          mma(R[1][ti], A1, Bp);
          mma(Sp[0][ti], A0, Bo);
          mma(Sp[1][ti], A1, Bo);
        }
      }
      // u = R / n - s (s . q) / n^2;  qc = q - lambda u;  Qa = qc * e^B.  For bf16 operands
      // Qa is kept as hi + lo (lo = bf16(x - hi)): the intra-chunk attention matrix is a sum
      // of few, possibly cancelling products when little of the sequence has been read.
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) {
        const int i = 16 * ti + l16;
        const float inv_n = 1.0f / (float)(nb + i + 1);
        const float sq = sm.mq[i] + sm.psum[0][i] + sm.psum[1][i] + sm.psum[2][i] + sm.psum[3][i];
        const float coef = sq * inv_n * inv_n;
        const float lam = sm.lam[i];
#pragma unroll
        for (int jm = 0; jm < 2; ++jm) {
          const int m = 32 * w + 16 * jm + 4 * g;
          const f32x4 q4 = ld4<T>(&sm.Qs[i][m]);
          const f32x4 b4 = *reinterpret_cast<const f32x4*>(&sm.Bs[i][m]);
          f32x4 qa;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float s = Sp[jm][ti][r] + sm.m0[m + r];
            const float u = R[jm][ti][r] * inv_n - s * coef;
            qa[r] = (q4[r] - lam * u) * __expf(b4[r]);
          }
          st4<T>(&sm.Qa[i][m], qa);
          if constexpr (kSplit) qlo[ti][jm] = qa - ld4<T>(&sm.Qa[i][m]);
        }
      }
      // k * e^-B, row-major, hi in place (nothing reads Ks in this phase); lo kept in registers
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int vi = tid + j * NTH;
        const int t = (vi * VE) / D, c = (vi * VE) % D;
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const float kp = (float)sm.Ks[t][c + e] * __expf(-sm.Bs[t][c + e]);
          const T hi = (T)kp;
          sm.Ks[t][c + e] = hi;
          if constexpr (kSplit) klo[j][e] = kp - (float)hi;
        }
      }
    }
    // (k * e^-B)^T
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int vi = tid + j * NTH;
      const int c = (vi * VE) / kL, t = (vi * VE) % kL;
#pragma unroll
      for (int e = 0; e < VE; ++e) sm.Kpt[c][t + e] = (T)((float)sm.Kt[c][t + e] * __expf(-sm.Bs[t + e][c]));
    }
    __syncthreads();

    if constexpr (MAIN) {
      if constexpr (kSplit) {
        // lo parts into tiles nobody reads any more: Qa lo over q rows, (k e^-B) lo over the decay tile
        T* Klo = reinterpret_cast<T*>(&sm.Bs[0][0]);
#pragma unroll
        for (int ti = 0; ti < 4; ++ti)
#pragma unroll
          for (int jm = 0; jm < 2; ++jm) st4<T>(&sm.Qs[16 * ti + l16][32 * w + 16 * jm + 4 * g], qlo[ti][jm]);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int vi = tid + j * NTH;
          const int t = (vi * VE) / D, c = (vi * VE) % D;
#pragma unroll
          for (int e = 0; e < VE; ++e) Klo[t * PQ + c + e] = (T)klo[j][e];
        }
        __syncthreads();
      }
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
            const Frag<T> Al = lds_frag<T, KORD_CONTIG>(reinterpret_cast<const T*>(&sm.Bs[0][0]), PQ, 16 * tj, 32 * kk, lane);
            const Frag<T> Bl = lds_frag<T, KORD_CONTIG>(&sm.Qs[0][0], PQ, 16 * ti, 32 * kk, lane);
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
        const Frag<T> A0 = lds_frag<T, KORD_CONTIG>(&sm.Vt[0][0], PT, 32 * w, 32 * kk, lane);
        const Frag<T> A1 = lds_frag<T, KORD_CONTIG>(&sm.Vt[0][0], PT, 32 * w + 16, 32 * kk, lane);
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
          for (int jm = 0; jm < 2; ++jm) st4<T>(og + (tok0 + t0 + i) * D + 32 * w + 16 * jm + 4 * g, O[jm][ti]);
        }
      }
    }

    // ---- carry update: C += K^T K;  S^T = diag(e^{B_63}) (S^T + (K e^-B)^T V)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const Frag<T> Bk0 = lds_frag<T, KORD_CONTIG>(&sm.Kt[0][0], PT, 32 * w, 32 * kk, lane);
      const Frag<T> Bk1 = lds_frag<T, KORD_CONTIG>(&sm.Kt[0][0], PT, 32 * w + 16, 32 * kk, lane);
      const Frag<T> Bv0 = lds_frag<T, KORD_CONTIG>(&sm.Vt[0][0], PT, 32 * w, 32 * kk, lane);
      const Frag<T> Bv1 = lds_frag<T, KORD_CONTIG>(&sm.Vt[0][0], PT, 32 * w + 16, 32 * kk, lane);
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
    if (tid < D) sm.m0[tid] = sm.m1[tid];
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
        const int row = 32 * w + 16 * jm + l16;
        const int col = 16 * t + 4 * g;
        *reinterpret_cast<f32x4*>(Sout + (size_t)row * D + col) = Sacc[t][jm];
        *reinterpret_cast<f32x4*>(Cout + (size_t)row * D + col) = Cacc[t][jm];
      }
    }
    for (int c = tid; c < D; c += NTH) {
      mout[c] = sm.m0[c];
      if (ldout != nullptr) ldout[c] = sm.ldec[c];
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
