// Backward of one step of the CCQ recurrence (the adjoint of the decode step), gfx950.
//
// The pages train CCQ models from scratch (10100.com write-up, "方法解析" point 3), so the read
// step needs gradients.  Forward step per (sequence, head), carry (S, C, m, n) before it
// (cleaning, gate and read of the gist.science summary §2 "机制" / "集成", statistics of §2
// "理论推导"):
//   C1 = C + k k^T;  m1 = m + k;  n1 = n + 1;  r = C1 q;  sq = m1 . q
//   u = r / n1 - m1 sq / n1^2;  lam = sigmoid(w . q + b);  qc = q - lam u
//   GLA: S1 = S diag(alpha) + v k^T        GDN: S1 = a (S - beta (S k) k^T) + beta v k^T
//   o = S1 qc
// Given do and the adjoint of the carry after the step (dS, dC, dm), with Sh = dS + do qc^T:
//   dqc = S1^T do;  du = -lam dqc;  dlogit = -(u . dqc) lam (1 - lam);  dw = dlogit q;  db = dlogit
//   dR = du / n1;  dsq = -(m1 . du) / n1^2;  dm_in = dm + dsq q - sq du / n1^2
//   dq = dqc + dlogit w + C1^T dR + dsq m1;  dC_in = dC + dR q^T;  dk_stat = (dC_in + dC_in^T) k + dm_in
//   GLA: dv = Sh k;  dk = Sh^T v + dk_stat;  dg_c = alpha_c sum_i S_ic Sh_ic;  dS_in = Sh diag(alpha)
//   GDN: dv = beta Sh k;  dk = sum_i [Sh_i (beta v_i - a beta (S k)_i) - a beta S_i (Sh k)_i] + dk_stat
//        dg = a <Sh, S - beta (S k) k^T>;  dbeta = (Sh k) . (v - a S k);  dS_in = a (Sh - beta (Sh k) k^T)
// Memory-bound like the decode step: S, dS, C, dC (fp32 d x d each) are read once and dS, dC
// written once, in place.  One workgroup of NT = 8 d threads per (sequence, head); thread t owns
// float4 column group t mod d/4 of rows t / (d/4) + i NT / (d/4).  Row reductions stay inside a
// wave (xor shuffles over the d/4 lanes of a row); column reductions add the wave's two row
// groups with one shuffle and the waves' partials through LDS.
#include "ccq_device.hpp"
#include "ccq_internal.hpp"

namespace ccq {

template <int D, typename T, int RULE, int NT>
__global__ __launch_bounds__(NT) void step_backward_kernel(StepBackArgs a) {
  constexpr int C4 = D / 4;        // float4 per row
  constexpr int RPI = NT / C4;     // rows covered per iteration
  constexpr int IT = D / RPI;      // rows per thread
  constexpr int NWV = NT / 64;     // waves
  constexpr int NVW = (D + 63) / 64;  // waves holding the d-long vectors
  static_assert(C4 == 32 && NT % 64 == 0, "two row groups per wave");
  static_assert(IT * RPI == D, "rows must tile the workgroup");

  const int head = blockIdx.x;
  const int h = head % a.H;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int col4 = tid % C4, row0 = tid / C4;

  __shared__ float q_s[D], k_s[D], v_s[D], al_s[D], w_s[D], m1_s[D], do_s[D];
  __shared__ float r_s[D], sk_s[D], qc_s[D], u_s[D], dqc_s[D], dR_s[D], dm_s[D];
  __shared__ float colp[3][NWV][D];   // column-reduction partials (three vectors at a time)
  __shared__ float red[4][NWV];       // block-reduction partials
  __shared__ float sc[8];             // scalars: lam, dlogit, dsq, sq, da, dbeta, 1/n1

  // ---- token vectors, gate parameters, key sum, count
  const size_t vo = (size_t)head * D;
  if (tid < D) {
    const float kv = to_f32(static_cast<const T*>(a.k)[vo + tid]);
    q_s[tid] = to_f32(static_cast<const T*>(a.q)[vo + tid]);
    k_s[tid] = kv;
    v_s[tid] = to_f32(static_cast<const T*>(a.v)[vo + tid]);
    if constexpr (RULE == 0) al_s[tid] = __expf(to_f32(static_cast<const T*>(a.log_alpha)[vo + tid]));
    w_s[tid] = a.w_lambda[(size_t)h * D + tid];
    m1_s[tid] = a.ksum[vo + tid] + kv;
    do_s[tid] = a.d_o[vo + tid];
    dm_s[tid] = a.dksum[vo + tid];
  }
  float alpha_s = 1.f, beta_s = 0.f;
  if constexpr (RULE == 1) {
    alpha_s = __expf(to_f32(static_cast<const T*>(a.log_alpha)[head]));
    beta_s = to_f32(static_cast<const T*>(a.beta)[head]);
  }
  const float inv_n = 1.0f / (float)(a.n[head] + 1);
  const float b_lam = a.b_lambda[h];

  // ---- the state and its adjoint, the statistic and its adjoint
  const float* Sg = a.S + (size_t)head * D * D;
  const float* Cg = a.C + (size_t)head * D * D;
  float* dSg = a.dS + (size_t)head * D * D;
  float* dCg = a.dC + (size_t)head * D * D;
  f32x4 S[IT], Sh[IT], C1[IT], Ch[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const size_t off = (size_t)(row0 + i * RPI) * D + 4 * col4;
    S[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sg + off));
    Sh[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dSg + off));
    C1[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Cg + off));
    Ch[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dCg + off));
  }
  lds_barrier();
  const f32x4 k4 = *reinterpret_cast<const f32x4*>(&k_s[4 * col4]);
  const f32x4 q4 = *reinterpret_cast<const f32x4*>(&q_s[4 * col4]);

  // ---- forward recompute: C1 = C + k k^T, r = C1 q, (GDN) sk = S k; w . q and m1 . q
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int row = row0 + i * RPI;
    C1[i] += k_s[row] * k4;
    float pr = C1[i][0] * q4[0] + C1[i][1] * q4[1] + C1[i][2] * q4[2] + C1[i][3] * q4[3];
    pr = group_sum<C4>(pr);
    if (col4 == 0) r_s[row] = pr;
    if constexpr (RULE == 1) {
      float ps = S[i][0] * k4[0] + S[i][1] * k4[1] + S[i][2] * k4[2] + S[i][3] * k4[3];
      ps = group_sum<C4>(ps);
      if (col4 == 0) sk_s[row] = ps;
    }
  }
  if (tid < D) {
    const float pw = group_sum<64>(w_s[tid] * q_s[tid]);
    const float pm = group_sum<64>(m1_s[tid] * q_s[tid]);
    if (lane == 0) {
      red[0][wv] = pw;
      red[1][wv] = pm;
    }
  }
  lds_barrier();
  if (tid < D) {
    float wq = 0.f, sq = 0.f;
#pragma unroll
    for (int v = 0; v < NVW; ++v) {
      wq += red[0][v];
      sq += red[1][v];
    }
    const float lam = sigmoidf(wq + b_lam);
    const float u = r_s[tid] * inv_n - m1_s[tid] * (sq * inv_n * inv_n);
    u_s[tid] = u;
    qc_s[tid] = q_s[tid] - lam * u;
    if (tid == 0) {
      sc[0] = lam;
      sc[3] = sq;
    }
  }
  lds_barrier();

  // ---- state adjoint: Sh = dS + do qc^T; row reductions Sh k; column reductions of S1^T do
  // and the rule's dk / dg terms; dS_in written back
  const f32x4 qc4 = *reinterpret_cast<const f32x4*>(&qc_s[4 * col4]);
  f32x4 cA = zero4(), cB = zero4(), cC = zero4();  // per-thread column partials
  float pa = 0.f, pb = 0.f;                         // GDN: <Sh, S - beta sk k^T>, dbeta terms
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int row = row0 + i * RPI;
    const float dor = do_s[row], vr = v_s[row];
    Sh[i] += dor * qc4;
    float shk = Sh[i][0] * k4[0] + Sh[i][1] * k4[1] + Sh[i][2] * k4[2] + Sh[i][3] * k4[3];
    shk = group_sum<C4>(shk);
    f32x4 din;
    if constexpr (RULE == 0) {
      const f32x4 al4 = *reinterpret_cast<const f32x4*>(&al_s[4 * col4]);
      const f32x4 S1 = S[i] * al4 + vr * k4;
      cA += dor * S1;          // S1^T do
      cB += vr * Sh[i];        // Sh^T v
      cC += S[i] * Sh[i];      // colsum(S o Sh)
      din = Sh[i] * al4;
      if (col4 == 0) a.dv[vo + row] = shk;
    } else {
      const float skr = sk_s[row];
      const f32x4 S1 = alpha_s * (S[i] - (beta_s * skr) * k4) + (beta_s * vr) * k4;
      cA += dor * S1;
      cB += (beta_s * vr - alpha_s * beta_s * skr) * Sh[i] - (alpha_s * beta_s * shk) * S[i];
      const f32x4 Sm = S[i] - (beta_s * skr) * k4;
      pa += Sh[i][0] * Sm[0] + Sh[i][1] * Sm[1] + Sh[i][2] * Sm[2] + Sh[i][3] * Sm[3];
      if (col4 == 0) pb += shk * (vr - alpha_s * skr);
      din = alpha_s * (Sh[i] - (beta_s * shk) * k4);
      if (col4 == 0) a.dv[vo + row] = beta_s * shk;
    }
    __builtin_nontemporal_store(din, reinterpret_cast<f32x4*>(dSg + (size_t)row * D + 4 * col4));
  }
  // column partials: the wave's two row groups, then the waves through LDS
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    cA[e] += __shfl_xor(cA[e], 32, 64);
    cB[e] += __shfl_xor(cB[e], 32, 64);
    cC[e] += __shfl_xor(cC[e], 32, 64);
  }
  if (lane < 32) {
    *reinterpret_cast<f32x4*>(&colp[0][wv][4 * col4]) = cA;
    *reinterpret_cast<f32x4*>(&colp[1][wv][4 * col4]) = cB;
    *reinterpret_cast<f32x4*>(&colp[2][wv][4 * col4]) = cC;
  }
  if constexpr (RULE == 1) {
    pa = group_sum<64>(pa);
    pb = group_sum<64>(pb);
    if (lane == 0) {
      red[2][wv] = pa;
      red[3][wv] = pb;
    }
  }
  lds_barrier();

  // ---- per channel: dqc, the write-side dk and dg; the CCQ adjoint's dot products
  float dkw = 0.f;
  if (tid < D) {
    float dqc = 0.f, c2 = 0.f;
#pragma unroll 4
    for (int v = 0; v < NWV; ++v) {
      dqc += colp[0][v][tid];
      dkw += colp[1][v][tid];
      c2 += colp[2][v][tid];
    }
    dqc_s[tid] = dqc;
    if constexpr (RULE == 0) a.dlog_alpha[vo + tid] = al_s[tid] * c2;
    const float lam = sc[0];
    const float du = -lam * dqc;
    const float pud = group_sum<64>(u_s[tid] * dqc);
    const float pmd = group_sum<64>(m1_s[tid] * du);
    if (lane == 0) {
      red[0][wv] = pud;
      red[1][wv] = pmd;
    }
  }
  if constexpr (RULE == 1) {
    if (tid == 0) {
      float da = 0.f, db_ = 0.f;
#pragma unroll
      for (int v = 0; v < NWV; ++v) {
        da += red[2][v];
        db_ += red[3][v];
      }
      a.dlog_alpha[head] = alpha_s * da;
      a.dbeta[head] = db_;
    }
  }
  lds_barrier();
  if (tid < D) {
    float ud = 0.f, md = 0.f;
#pragma unroll
    for (int v = 0; v < NVW; ++v) {
      ud += red[0][v];
      md += red[1][v];
    }
    const float lam = sc[0], sq = sc[3];
    const float dlogit = -ud * lam * (1.f - lam);
    const float dsq = -md * inv_n * inv_n;
    const float du = -lam * dqc_s[tid];
    dR_s[tid] = du * inv_n;
    const float dmi = dm_s[tid] + dsq * q_s[tid] - sq * inv_n * inv_n * du;
    dm_s[tid] = dmi;
    a.dksum[vo + tid] = dmi;
    a.dw[vo + tid] = dlogit * q_s[tid];
    if (tid == 0) {
      a.db[head] = dlogit;
      sc[1] = dlogit;
      sc[2] = dsq;
    }
  }
  lds_barrier();

  // ---- statistic adjoint: dC_in = dC + dR q^T (written back); C1^T dR and dC_in^T k by
  // columns, dC_in k by rows
  f32x4 cD = zero4(), cE = zero4();
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int row = row0 + i * RPI;
    const float dRr = dR_s[row], kr = k_s[row];
    Ch[i] += dRr * q4;
    __builtin_nontemporal_store(Ch[i], reinterpret_cast<f32x4*>(dCg + (size_t)row * D + 4 * col4));
    cD += dRr * C1[i];   // C1^T dR
    cE += kr * Ch[i];    // dC_in^T k
    float ck = Ch[i][0] * k4[0] + Ch[i][1] * k4[1] + Ch[i][2] * k4[2] + Ch[i][3] * k4[3];
    ck = group_sum<C4>(ck);
    if (col4 == 0) r_s[row] = ck;  // dC_in k (r_s is free again)
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    cD[e] += __shfl_xor(cD[e], 32, 64);
    cE[e] += __shfl_xor(cE[e], 32, 64);
  }
  if (lane < 32) {
    *reinterpret_cast<f32x4*>(&colp[0][wv][4 * col4]) = cD;
    *reinterpret_cast<f32x4*>(&colp[1][wv][4 * col4]) = cE;
  }
  lds_barrier();
  if (tid < D) {
    float cdr = 0.f, cek = 0.f;
#pragma unroll 4
    for (int v = 0; v < NWV; ++v) {
      cdr += colp[0][v][tid];
      cek += colp[1][v][tid];
    }
    const float dlogit = sc[1], dsq = sc[2];
    a.dq[vo + tid] = dqc_s[tid] + dlogit * w_s[tid] + cdr + dsq * m1_s[tid];
    a.dk[vo + tid] = dkw + r_s[tid] + cek + dm_s[tid];
  }
}

template <int D, typename T>
static hipError_t launch_step_backward_t(const StepBackArgs& a, hipStream_t s) {
  constexpr int NT = 8 * D;
  const dim3 grid((unsigned)(a.N * a.H)), block(NT);
  if (a.rule == 0)
    hipLaunchKernelGGL((step_backward_kernel<D, T, 0, NT>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((step_backward_kernel<D, T, 1, NT>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_step_backward(const StepBackArgs& a, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.d == 128) return launch_step_backward_t<128, __bf16>(a, s);
  } else {
    if (a.d == 128) return launch_step_backward_t<128, float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
