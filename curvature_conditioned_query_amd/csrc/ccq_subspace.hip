// Key-covariance subspace diagnostic (gfx950).
//
// The 10100.com write-up of the CCQ paper (section "记忆体检") checks the geometry the cleaned
// query relies on: Δμ, how much less the needle keys than the distractor keys align with the
// top-16 eigen-subspace of the key covariance.  Per (b, h):
//   Sigma = C / n - mu mu^T, mu = ksum / n        (the statistics, gist.science summary §2 "理论推导")
//   Sigma = U diag(lambda) U^T, lambda descending  (symmetric eigen-decomposition)
//   a_t   = |U_r^T k_t|^2 / |k_t|^2               (0 for a zero key)
//   Δμ    = mean of a over needle tokens - mean over the others.
//
// subspace_eigen_kernel: one workgroup per (b, h), the dense symmetric eigenproblem by the
// textbook route (Golub and Van Loan, "Matrix Computations": Householder tridiagonalisation,
// Sturm-sequence bisection, inverse iteration):
//  1. Sigma / max|Sigma_ij| in LDS is reduced to tridiagonal form T = Q^T A Q by d - 2
//     Householder reflectors H_k = I - tau_k v_k v_k^T.  Step k takes the symmetric rank-2 update
//     A <- A - v w^T - w v^T (w = p - (tau/2)(p.v) v, p = tau A v) in one pass that also forms the
//     next reflector's product p' = tau' A' v', so a step costs one workgroup barrier.  Lane l of
//     every wave holds entries l and l + 64 of v, w and p in registers, and every wave rebuilds
//     the column that becomes final (and the next reflector from it) by itself; wave w updates
//     the trailing block's column groups 4 (w + 8 g) .. 4 (w + 8 g) + 3 for every row (spread
//     over the matrix, so that the shrinking block keeps every wave busy), takes those columns'
//     v and w entries from the lanes that hold them, and leaves its share of A' v' in LDS.
//     Reflector k's vector is kept in row k of A (columns k+1 ..).
//  2. Each eigenvalue of T (scaled into [-1, 1] by its Gershgorin bound) is found by
//     multisection: the lanes of a group count, by the Sturm sequence of T - x I, the eigenvalues
//     below G interior points of the group's interval and keep the sub-interval that holds their
//     eigenvalue, until it is a few ulps wide.  The count runs the recurrence in IEEE arithmetic
//     (a zero pivot gives an infinite one, whose reciprocal is zero: Demmel and Li's exception-
//     handling form), with e_i^2 floored at 1e-30 so that no product 0 x inf arises.
//  3. The top-r eigenvectors of T: one lane per vector runs two steps of inverse iteration from
//     a hashed start vector, solving with T - lambda I = L diag(q) L^T (no pivoting: q_i is the
//     Sturm recurrence at lambda, pivots below 2^-23 of ||T|| raised to that size, which is what
//     makes the solve amplify the wanted eigenvector; Peters and Wilkinson's analysis of inverse
//     iteration); two passes of modified Gram-Schmidt then make them orthonormal
//     (vectors of tight clusters converge to mixtures of the cluster's eigenvectors: any
//     orthonormal basis of the cluster is a valid answer there).
//  4. The back-transformation u = H_0 H_1 ... H_{d-3} z, one wave per vector, no barriers; each
//     vector is normalised and signed so that its largest-magnitude entry (lowest index among
//     equals) is positive.
// A zero Sigma (n = 0, or identical keys) has eigenvalues 0 and the basis e_0 .. e_{r-1}.
// subspace_align_kernel: 64 tokens per workgroup, 4 lanes per token, basis rows in LDS.
// subspace_delta_kernel: one workgroup per (b, h) reduces a_t under the needle mask.
#include "ccq_device.hpp"
#include "ccq_internal.hpp"

namespace ccq {

constexpr int kEigThreads = 512;
constexpr int kEigWaves = kEigThreads / 64;
constexpr int kIvStride = kMaxSubspaceRank + 1;  // inverse-iteration arrays: entry i of vector t at [i][t]
constexpr int kInvIters = 2;                     // inverse-iteration steps per vector
constexpr int kMaxRounds = 40;                   // multisection rounds per eigenvalue (cap)

template <int D>
struct EigSmem {
  alignas(16) float A[D][D + 4];  // the scaled Sigma; row k then holds reflector k's vector
  float dg[D], od[D], tau[D];     // T's diagonal, off-diagonal (od[i] couples i and i + 1), tau_k
  alignas(16) float2 de2[D];      // scaled (d_i, max(e_{i-1}^2, 1e-30)): the Sturm coefficients
  float eh[D];                    // scaled e_i
  float lasc[D], ldesc[D];        // eigenvalues of the scaled T, ascending and descending
  float mu[D];                    // ksum / n
  float red[kEigWaves];
  int ired[kEigWaves];
  float gs[4];                    // Sigma's scale, T's Gershgorin bound, interval low, high
  union {
    alignas(16) float raw[D][D + 4];            // C as stored (packed: its upper triangle)
    alignas(16) float ps[2][D][kEigWaves];      // per-wave shares of A v (double-buffered)
    struct {
      float rq[D][kIvStride], l[D][kIvStride], y[D][kIvStride];  // 1 / q_i, l_i, the iterate
    } iv;
    alignas(16) float q[kMaxSubspaceRank][D];  // Gram-Schmidt: the vectors published so far
  } u;
};

template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_f(float x) {  // rows outside ROWS read 0
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}

__device__ __forceinline__ float lane_read(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Sum over the wave, the same value in every lane: DPP sums inside rows of 16, then row 3
// collects the other rows through the row broadcasts, and lane 63 is read.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<0xB1>(x);          // lane ^ 1
  x += dpp_f<0x4E>(x);          // lane ^ 2
  x += dpp_f<0x141>(x);         // half-row mirror: sums of 8
  x += dpp_f<0x140>(x);         // row mirror: sums of 16
  x += dpp_f<0x142, 0xA>(x);    // rows 1, 3 add lane 15 of the row before
  x += dpp_f<0x143, 0xC>(x);    // rows 2, 3 add lane 31
  return lane_read(x, 63);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// Entry idx of a wave vector held as c[e] = entry (lane + 64 e); idx is wave-uniform.
template <int EPL>
__device__ __forceinline__ float wave_entry(const float (&c)[EPL], int idx) {
  float x = c[0];
  if constexpr (EPL > 1) x = idx >= 64 ? c[1] : c[0];
  return lane_read(x, idx & 63);
}

// Number of eigenvalues of the scaled tridiagonal below x: the negative terms of the Sturm
// recurrence q_i = (d_i - x) - e_{i-1}^2 / q_{i-1}.  The coefficients are read 8 terms at a time,
// one block ahead of the recurrence.
template <int D>
__device__ __forceinline__ int sturm_count(const float2* de2, float x) {
  const f32x4* src = reinterpret_cast<const f32x4*>(de2);
  int cnt = 0;
  float q = 1.f;
  f32x4 cur[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) cur[h] = src[h];
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    f32x4 nxt[4];
    if (c + 1 < D / 8) {
#pragma unroll
      for (int h = 0; h < 4; ++h) nxt[h] = src[4 * (c + 1) + h];
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      q = (cur[h][0] - x) - cur[h][1] * __builtin_amdgcn_rcpf(q);
      cnt += q < 0.f ? 1 : 0;
      q = (cur[h][2] - x) - cur[h][3] * __builtin_amdgcn_rcpf(q);
      cnt += q < 0.f ? 1 : 0;
    }
    if (c + 1 < D / 8) {
#pragma unroll
      for (int h = 0; h < 4; ++h) cur[h] = nxt[h];
    }
  }
  return cnt;
}

// Start vector of inverse iteration: a hash of (entry, vector) mapped into [-1, 1).
__device__ __forceinline__ float start_entry(int i, int t) {
  uint32_t h = (uint32_t)i * 0x9E3779B1u ^ ((uint32_t)t * 0x85EBCA77u + 0x165667B1u);
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  h *= 0x297A2D39u;
  h ^= h >> 15;
  return (float)(h >> 8) * 1.1920928955078125e-7f - 1.0f;
}

// Row of packed (upper-triangle, row-major) index e of a d x d matrix: the largest i with
// i d - i (i - 1) / 2 <= e.
__device__ __forceinline__ int packed_row(int e, int d) {
  const float b = (float)(2 * d + 1);
  int i = (int)((b - sqrtf(b * b - 8.0f * (float)e)) * 0.5f);
  i = max(0, min(d - 1, i));
  if (i + 1 < d && (i + 1) * d - (i + 1) * i / 2 <= e) ++i;
  if (i * d - i * (i - 1) / 2 > e) --i;
  return i;
}

template <int D>
__global__ __launch_bounds__(kEigThreads) void subspace_eigen_kernel(SubspaceArgs a) {
  constexpr int EPL = D / 64;         // entries of a wave vector per lane: i = lane + 64 e
  constexpr int GPW = D / 32;         // float4 column groups per wave in the trailing-block update
  constexpr int G = kEigThreads / D;  // lanes per eigenvalue in the multisection
  __shared__ EigSmem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, and known to be so
  const int head = blockIdx.x;
  const int r = a.r;
  const bool packed = (a.flags & kFlagPackedCov) != 0;
  const float* C = a.C + (size_t)head * (packed ? D * (D + 1) / 2 : D * D);
  const int64_t n = a.n[head];
  const float inv_n = n > 0 ? 1.0f / (float)n : 0.0f;
  float* ev = a.eigvals + (size_t)head * D;
  float* basis = a.basis + (size_t)head * r * D;

  // C as stored into LDS, coalesced (packed: the upper triangle), mu = ksum / n
  if (packed) {
    constexpr int NPK = D * (D + 1) / 2, NL = (NPK + kEigThreads - 1) / kEigThreads;
    float v[NL];
#pragma unroll
    for (int s = 0; s < NL; ++s) {
      const int e = tid + kEigThreads * s;
      v[s] = e < NPK ? C[e] : 0.f;
    }
#pragma unroll
    for (int s = 0; s < NL; ++s) {
      const int e = tid + kEigThreads * s;
      if (e < NPK) {
        const int i = packed_row(e, D);
        sm.u.raw[i][i + e - (i * D - i * (i - 1) / 2)] = v[s];
      }
    }
  } else {
    constexpr int NL = D * D / kEigThreads;
    float v[NL];
#pragma unroll
    for (int s = 0; s < NL; ++s) v[s] = C[tid + kEigThreads * s];
#pragma unroll
    for (int s = 0; s < NL; ++s) {
      const int e = tid + kEigThreads * s;
      sm.u.raw[e / D][e % D] = v[s];
    }
  }
  if (tid < D) sm.mu[tid] = a.ksum[(size_t)head * D + tid] * inv_n;
  __syncthreads();
  // Sigma = (C + C^T) / 2n - mu mu^T (C is symmetric by definition; the mean of the two stored
  // triangles makes the working matrix exactly symmetric), and its largest |entry|
  float amax = 0.f;
#pragma unroll 4
  for (int e = tid; e < D * D; e += kEigThreads) {
    const int i = e / D, j = e % D;
    const float cij = packed ? sm.u.raw[min(i, j)][max(i, j)] : 0.5f * (sm.u.raw[i][j] + sm.u.raw[j][i]);
    const float sij = n > 0 ? cij * inv_n - sm.mu[i] * sm.mu[j] : 0.f;
    sm.A[i][j] = sij;
    amax = fmaxf(amax, fabsf(sij));
  }
  amax = wave_max(amax);
  if (lane == 0) sm.red[wv] = amax;
  for (int i = tid; i < D; i += kEigThreads) {
    sm.od[i] = 0.f;
    sm.tau[i] = 0.f;
  }
  __syncthreads();
  float sig = 0.f;
#pragma unroll
  for (int x = 0; x < kEigWaves; ++x) sig = fmaxf(sig, sm.red[x]);
  if (!(sig > 0.f)) {  // Sigma = 0: every eigenvalue 0, the basis e_0 .. e_{r-1}
    for (int i = tid; i < D; i += kEigThreads) ev[i] = 0.f;
    for (int e = tid; e < r * D; e += kEigThreads) basis[e] = (e / D == e % D) ? 1.f : 0.f;
    if (tid == 0 && a.iters != nullptr) a.iters[head] = 0;
    return;
  }
  {
    const float isig = 1.0f / sig;
#pragma unroll 4
    for (int e = tid; e < D * D; e += kEigThreads) sm.A[e / D][e % D] *= isig;  // own entries only
    for (int e = tid; e < D * kEigWaves; e += kEigThreads) sm.u.ps[1][e / kEigWaves][e % kEigWaves] = 0.f;
  }
  __syncthreads();

  // ---- 1. Householder tridiagonalisation.  Iteration k (k = -1 .. d-3) applies reflector k
  // (v_k, tau_k, and the waves' shares of A v_k from the previous iteration) to the trailing
  // block, makes column k+1 final (diagonal d_{k+1}) and builds reflector k+1 from it.
  float tau_k = 0.f;
  float vk[EPL], wk[EPL], vn[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) vk[e] = 0.f;
  for (int k = -1; k <= D - 3; ++k) {
    const int cur = k & 1, nxt = cur ^ 1, c1 = k + 1, s0 = c1 + 1;
    float colv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) colv[e] = sm.A[lane + 64 * e][c1];
    // p_k = tau_k A v_k, K = tau_k / 2 (p_k . v_k), w_k = p_k - K v_k
    float pk[EPL], pv = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int i = lane + 64 * e;
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(&sm.u.ps[cur][i][0]);
      const f32x4 s2 = *reinterpret_cast<const f32x4*>(&sm.u.ps[cur][i][4]);
      pk[e] = tau_k * (((s1[0] + s1[1]) + (s1[2] + s1[3])) + ((s2[0] + s2[1]) + (s2[2] + s2[3])));
      pv += pk[e] * vk[e];  // v_k is zero above row k + 1
    }
    const float K = 0.5f * tau_k * wave_sum(pv);
#pragma unroll
    for (int e = 0; e < EPL; ++e) wk[e] = lane + 64 * e >= c1 ? pk[e] - K * vk[e] : 0.f;
    const float vc1 = wave_entry<EPL>(vk, c1), wc1 = wave_entry<EPL>(wk, c1);
    float c[EPL];
    float ssq = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int i = lane + 64 * e;
      c[e] = colv[e] - vk[e] * wc1 - wk[e] * vc1;  // column c1 after reflector k (rows >= c1)
      if (i >= c1 + 2) ssq += c[e] * c[e];
    }
    ssq = wave_sum(ssq);
    const float dk = wave_entry<EPL>(c, c1), alpha = wave_entry<EPL>(c, c1 + 1);
    // reflector c1: H x = beta e_0 for x = column c1 below the diagonal (H = I when x is
    // already a multiple of e_0)
    float beta = alpha, tau_n = 0.f, sc = 0.f;
    if (ssq > 0.f) {
      const float nrm = __builtin_amdgcn_sqrtf(alpha * alpha + ssq);
      beta = alpha >= 0.f ? -nrm : nrm;
      tau_n = (beta - alpha) * __builtin_amdgcn_rcpf(beta);
      sc = __builtin_amdgcn_rcpf(alpha - beta);
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int i = lane + 64 * e;
      vn[e] = i == c1 + 1 ? 1.f : (i >= c1 + 2 ? c[e] * sc : 0.f);
      if (wv == 0 && i > c1) sm.A[c1][i] = vn[e];  // row c1 is not part of the block any more
    }
    if (wv == 0 && lane == 0) {
      sm.dg[c1] = dk;
      sm.od[c1] = beta;
      sm.tau[c1] = tau_n;
    }
    // trailing block (rows and columns >= s0), this wave's column groups: A <- A - v_k w_k^T -
    // w_k v_k^T, and this wave's share of A v_{c1} over the updated entries.  Group g spans
    // columns 4 (wv + 8 g) ..; a group left of s0 is skipped (wave-uniform).
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    {
      bool act[GPW];
      float vj[GPW][4], wj[GPW][4], nj[GPW][4];
#pragma unroll
      for (int g = 0; g < GPW; ++g) {
        const int jg = 4 * (wv + kEigWaves * g), ge = (32 * g) / 64, jl = jg & 63;  // entry jg: lane jl, slot ge
        act[g] = jg + 3 >= s0;
        if (act[g]) {
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            vj[g][x] = lane_read(vk[ge], jl + x);
            wj[g][x] = lane_read(wk[ge], jl + x);
            nj[g][x] = lane_read(vn[ge], jl + x);
          }
        }
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int i = lane + 64 * e;
        if (i < s0) continue;
        f32x4 a4[GPW];
#pragma unroll
        for (int g = 0; g < GPW; ++g)
          if (act[g]) a4[g] = *reinterpret_cast<const f32x4*>(&sm.A[i][4 * (wv + kEigWaves * g)]);
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
          if (!act[g]) continue;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const float t = a4[g][x] - vk[e] * wj[g][x] - wk[e] * vj[g][x];
            a4[g][x] = t;
            acc[e] += t * nj[g][x];  // n_j = 0 left of s0
          }
        }
#pragma unroll
        for (int g = 0; g < GPW; ++g) {
          const int jg = 4 * (wv + kEigWaves * g);
          if (!act[g]) continue;
          if (jg >= s0) {
            *reinterpret_cast<f32x4*>(&sm.A[i][jg]) = a4[g];
          } else {  // the group holding column c1, which stays as it was
#pragma unroll
            for (int x = 0; x < 4; ++x)
              if (jg + x >= s0) sm.A[i][jg + x] = a4[g][x];
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e) sm.u.ps[nxt][lane + 64 * e][wv] = acc[e];
#pragma unroll
    for (int e = 0; e < EPL; ++e) vk[e] = vn[e];
    tau_k = tau_n;
    lds_barrier();
  }
  if (tid == 0) sm.dg[D - 1] = sm.A[D - 1][D - 1];
  __syncthreads();

  // ---- 2. eigenvalues of T by multisection on the Sturm counts
  if (wv == 0) {
    float gb = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int i = lane + 64 * e;
      gb = fmaxf(gb, fabsf(sm.dg[i]) + fabsf(sm.od[i]) + (i > 0 ? fabsf(sm.od[i - 1]) : 0.f));
    }
    gb = wave_max(gb);  // Gershgorin bound of T (> 0: T is similar to a non-zero matrix)
    const float ig = 1.0f / gb;
    float lo = 2.f, hi = -2.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int i = lane + 64 * e;
      const float di = sm.dg[i] * ig, ei = sm.od[i] * ig, em = i > 0 ? sm.od[i - 1] * ig : 0.f;
      sm.de2[i] = make_float2(di, fmaxf(em * em, 1e-30f));
      sm.eh[i] = ei;
      lo = fminf(lo, di - fabsf(em) - fabsf(ei));
      hi = fmaxf(hi, di + fabsf(em) + fabsf(ei));
    }
    lo = -wave_max(-lo);
    hi = wave_max(hi);
    if (lane == 0) {
      sm.gs[0] = sig;
      sm.gs[1] = gb;
      sm.gs[2] = lo - 0x1p-20f;
      sm.gs[3] = hi + 0x1p-20f;
    }
  }
  __syncthreads();
  int rounds = 0;
  {
    const int j = tid / G, s = tid % G;  // eigenvalue j (ascending), point s of its group
    float lo = sm.gs[2], hi = sm.gs[3];
    const float step = 1.0f / (float)(G + 1);
    while (rounds < kMaxRounds && hi - lo > 0x1p-23f * (1.0f + fmaxf(fabsf(lo), fabsf(hi)))) {
      const float x = lo + (hi - lo) * ((float)(s + 1) * step);
      int zero = 0;  // an offset the compiler cannot see through: the coefficients are read in
      asm volatile("" : "+s"(zero));  // every round, not hoisted into (too many) registers
      const bool above = sturm_count<D>(sm.de2 + zero, x) > j;  // lambda_j < x
      const uint64_t ball = __ballot(above);
      const uint32_t bits = (uint32_t)(ball >> (lane - s)) & ((1u << G) - 1u);
      const int f = __builtin_ctz(bits | (1u << G));  // the first point above lambda_j (G: none)
      const float nlo = f == 0 ? lo : lo + (hi - lo) * ((float)f * step);
      const float nhi = f == G ? hi : lo + (hi - lo) * ((float)(f + 1) * step);
      ++rounds;
      if (nlo == lo && nhi == hi) break;
      lo = nlo;
      hi = nhi;
    }
    if (s == 0) sm.lasc[j] = 0.5f * (lo + hi);
  }
  {
    int rs = (tid % G == 0) ? rounds : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) rs += __shfl_xor(rs, off, 64);
    if (lane == 0) sm.ired[wv] = rs;
  }
  __syncthreads();
  // descending order (an exact rank: ties keep the higher ascending index first)
  const float escale = sm.gs[0] * sm.gs[1];
  for (int j = tid; j < D; j += kEigThreads) {
    const float lj = sm.lasc[j];
    int rk = 0;
#pragma unroll 8
    for (int i = 0; i < D; ++i) {
      const float li = sm.lasc[i];
      rk += (li > lj || (li == lj && i > j)) ? 1 : 0;
    }
    sm.ldesc[rk] = lj;
    ev[rk] = lj * escale;
  }
  if (tid == 0 && a.iters != nullptr) {
    int tot = 0;
#pragma unroll
    for (int x = 0; x < kEigWaves; ++x) tot += sm.ired[x];
    a.iters[head] = tot;
  }
  __syncthreads();

  // ---- 3. inverse iteration on the scaled T, one lane per wanted vector.  Operands are read
  // 8 entries at a time ahead of the recurrences.  Each solve starts from a right-hand side of
  // largest entry 2^-64, which leaves 2^190 of headroom for the growth through tiny pivots
  // (2^23 at most per pivot), so no entry overflows.
  if (tid < r) {
    constexpr int NB = 8;
    const int t = tid;
    const float lam = sm.ldesc[t];
    constexpr float kPivFloor = 0x1p-23f;
    auto& RQ = sm.u.iv.rq;
    auto& L = sm.u.iv.l;
    auto& Y = sm.u.iv.y;
    // T - lambda I = L diag(q) L^T: q_i = (d_i - lambda) - e_{i-1} l_i, l_i = e_{i-1} / q_{i-1}
    float rq = 0.f, ymax = 0.f;
#pragma unroll 1
    for (int i0 = 0; i0 < D; i0 += NB) {
      float dd[NB], em[NB];
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        dd[x] = sm.de2[i0 + x].x;
        em[x] = i0 + x > 0 ? sm.eh[i0 + x - 1] : 0.f;
      }
#pragma unroll
      for (int x = 0; x < NB; ++x) {
        const float li = em[x] * rq;
        float q = (dd[x] - lam) - em[x] * li;
        q = fabsf(q) < kPivFloor ? (q < 0.f ? -kPivFloor : kPivFloor) : q;
        rq = __builtin_amdgcn_rcpf(q);
        RQ[i0 + x][t] = rq;
        L[i0 + x][t] = li;
        const float y0 = start_entry(i0 + x, t);
        Y[i0 + x][t] = y0;
        ymax = fmaxf(ymax, fabsf(y0));
      }
    }
#pragma unroll 1
    for (int it = 0; it < kInvIters; ++it) {
      // L diag(q) L^T z = y 2^-64 / max|y|: forward through L, then back through diag(q) L^T;
      // z overwrites y
      const float ys = 0x1p-64f * __builtin_amdgcn_rcpf(ymax);
      float yp = 0.f;
#pragma unroll 1
      for (int i0 = 0; i0 < D; i0 += NB) {
        float yv[NB], lv[NB];
#pragma unroll
        for (int x = 0; x < NB; ++x) {
          yv[x] = Y[i0 + x][t];
          lv[x] = L[i0 + x][t];
        }
#pragma unroll
        for (int x = 0; x < NB; ++x) {
          yp = yv[x] * ys - lv[x] * yp;
          Y[i0 + x][t] = yp;
        }
      }
      float zn = 0.f;
      ymax = 0.f;
#pragma unroll 1
      for (int i0 = D - NB; i0 >= 0; i0 -= NB) {
        float yv[NB], rv[NB], lv[NB];
#pragma unroll
        for (int x = 0; x < NB; ++x) {
          yv[x] = Y[i0 + x][t];
          rv[x] = RQ[i0 + x][t];
          lv[x] = i0 + x + 1 < D ? L[i0 + x + 1][t] : 0.f;
        }
#pragma unroll
        for (int x = NB - 1; x >= 0; --x) {
          zn = yv[x] * rv[x] - lv[x] * zn;
          Y[i0 + x][t] = zn;
          ymax = fmaxf(ymax, fabsf(zn));
        }
      }
    }
  }
  __syncthreads();

  // ---- 4. orthonormalise (modified Gram-Schmidt, twice), back-transform, sign, store.
  // Wave wv owns vectors t = wv + 8 s.
  constexpr int S = kMaxSubspaceRank / kEigWaves;
  float z[S][EPL];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int t = wv + kEigWaves * s;
#pragma unroll
    for (int e = 0; e < EPL; ++e) z[s][e] = t < r ? sm.u.iv.y[lane + 64 * e][t] : 0.f;
  }
  __syncthreads();  // y is read before q (which overlaps it) is written
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int sj = 0; sj < S; ++sj) {
      for (int jw = 0; jw < kEigWaves; ++jw) {
        const int j = jw + kEigWaves * sj;
        if (j >= r) break;
        if (wv == jw) {
          float nn = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) nn += z[sj][e] * z[sj][e];
          nn = wave_sum(nn);
          const float in = nn > 0.f ? 1.0f / sqrtf(nn) : 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            z[sj][e] *= in;
            sm.u.q[j][lane + 64 * e] = z[sj][e];
          }
        }
        lds_barrier();
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int t = wv + kEigWaves * s;
          if (t <= j || t >= r) continue;
          float qj[EPL];
          float dot = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            qj[e] = sm.u.q[j][lane + 64 * e];
            dot += qj[e] * z[s][e];
          }
          dot = wave_sum(dot);
#pragma unroll
          for (int e = 0; e < EPL; ++e) z[s][e] -= dot * qj[e];
        }
      }
    }
  }
  // u = H_0 H_1 ... H_{d-3} z; reflector k - 1 is read while k is applied
  {
    float hv[EPL], ht = sm.tau[D - 3];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int i = lane + 64 * e;
      hv[e] = i > D - 3 ? sm.A[D - 3][i] : 0.f;
    }
    for (int k = D - 3; k >= 0; --k) {
      float vkk[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) vkk[e] = hv[e];
      const float tk = ht;
      if (k > 0) {
        ht = sm.tau[k - 1];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const int i = lane + 64 * e;
          hv[e] = i > k - 1 ? sm.A[k - 1][i] : 0.f;
        }
      }
      if (tk == 0.f) continue;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        if (wv + kEigWaves * s >= r) continue;
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dot += vkk[e] * z[s][e];
        const float f = tk * wave_sum(dot);
#pragma unroll
        for (int e = 0; e < EPL; ++e) z[s][e] -= f * vkk[e];
      }
    }
  }
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int t = wv + kEigWaves * s;
    if (t >= r) continue;
    float nn = 0.f, best = -1.f, bv = 0.f;
    int bi = D;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      nn += z[s][e] * z[s][e];
      if (fabsf(z[s][e]) > best) {
        best = fabsf(z[s][e]);
        bv = z[s][e];
        bi = lane + 64 * e;
      }
    }
    nn = wave_sum(nn);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ob = __shfl_xor(best, off, 64), ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ob > best || (ob == best && oi < bi)) {
        best = ob;
        bv = ov;
        bi = oi;
      }
    }
    const float f = (bv < 0.f ? -1.f : 1.f) / sqrtf(nn);
#pragma unroll
    for (int e = 0; e < EPL; ++e) basis[(size_t)t * D + lane + 64 * e] = f * z[s][e];
  }
}

// a_t = |U_r k_t|^2 / |k_t|^2: 64 tokens per workgroup, lanes 4t .. 4t+3 split the d channels.
template <int D, typename T>
__global__ __launch_bounds__(256) void subspace_align_kernel(SubspaceArgs a) {
  constexpr int CPL = D / 4;  // channels per lane
  __shared__ float U[kMaxSubspaceRank][D];
  const int head = blockIdx.y, tid = threadIdx.x;
  const int r = a.r;
  for (int e = tid; e < r * D; e += 256) U[e / D][e % D] = a.basis[(size_t)head * r * D + e];
  __syncthreads();
  const int tok = blockIdx.x * 64 + (tid >> 2), part = tid & 3;
  if (tok >= a.T) return;  // whole groups of 4 lanes leave together
  const T* kp = static_cast<const T*>(a.k) + ((size_t)head * a.T + tok) * D + part * CPL;
  float kv[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) kv[c] = to_f32(kp[c]);
  float kk = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) kk += kv[c] * kv[c];
  float num = 0.f;
  for (int j = 0; j < r; ++j) {
    float y = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) y += U[j][part * CPL + c] * kv[c];
    y += __shfl_xor(y, 1, 64);
    y += __shfl_xor(y, 2, 64);
    num += y * y;
  }
  kk += __shfl_xor(kk, 1, 64);
  kk += __shfl_xor(kk, 2, 64);
  if (part == 0) a.align[(size_t)head * a.T + tok] = kk > 0.f ? num / kk : 0.f;
}

// Δμ = mean a over needle tokens - mean a over the others (NaN if either set is empty).
__global__ __launch_bounds__(256) void subspace_delta_kernel(SubspaceArgs a) {
  __shared__ float red[3][4];
  const int head = blockIdx.x, tid = threadIdx.x;
  const float* al = a.align + (size_t)head * a.T;
  const uint8_t* nd = a.needle + (size_t)head * a.T;
  float sn = 0.f, sd = 0.f, cn = 0.f;
  for (int t = tid; t < a.T; t += 256) {
    const float v = al[t];
    if (nd[t]) {
      sn += v;
      cn += 1.f;
    } else {
      sd += v;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    sn += __shfl_xor(sn, off, 64);
    sd += __shfl_xor(sd, off, 64);
    cn += __shfl_xor(cn, off, 64);
  }
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = sn;
    red[1][tid >> 6] = sd;
    red[2][tid >> 6] = cn;
  }
  __syncthreads();
  if (tid == 0) {
    float SN = 0.f, SD = 0.f, CN = 0.f;
    for (int v = 0; v < 4; ++v) {
      SN += red[0][v];
      SD += red[1][v];
      CN += red[2][v];
    }
    const float CD = (float)a.T - CN;
    a.delta_mu[head] = (CN > 0.f && CD > 0.f) ? SN / CN - SD / CD : __builtin_nanf("");
  }
}

template <int D, typename T>
static hipError_t launch_subspace_t(const SubspaceArgs& a, hipStream_t s) {
  const int heads = a.B * a.H;
  hipLaunchKernelGGL((subspace_eigen_kernel<D>), dim3((unsigned)heads), dim3(kEigThreads), 0, s, a);
  hipLaunchKernelGGL((subspace_align_kernel<D, T>), dim3((unsigned)((a.T + 63) / 64), (unsigned)heads), dim3(256),
                     0, s, a);
  if (a.needle != nullptr) hipLaunchKernelGGL(subspace_delta_kernel, dim3((unsigned)heads), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_subspace(const SubspaceArgs& a, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.d == 128) return launch_subspace_t<128, __bf16>(a, s);
    if (a.d == 64) return launch_subspace_t<64, __bf16>(a, s);
  } else {
    if (a.d == 128) return launch_subspace_t<128, float>(a, s);
    if (a.d == 64) return launch_subspace_t<64, float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
