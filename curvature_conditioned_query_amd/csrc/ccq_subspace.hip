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
// subspace_eigen_kernel: one workgroup per (b, h) runs the parallel cyclic Jacobi method on
// Sigma held in LDS.  Each of the d - 1 steps of a sweep pairs all d indices into d/2 disjoint
// (p, q) pairs (round-robin ordering); the rotation of every pair is computed from the 2 x 2
// block (a_pp, a_pq, a_qq) as in the classical symmetric Jacobi method, and because the pairs
// are disjoint the whole step is A <- J^T A J with J block-diagonal: every 2 x 2 block (pair k
// rows, pair l columns) becomes J_k^T B J_l, computed once for k <= l on the upper triangle
// (the only part of A kept current), and the eigenvector matrix (kept transposed, one
// eigenvector per LDS row) gets its rows p, q rotated.  A rotation is skipped when |a_pq| is negligible against sqrt(|a_pp a_qq|) or below
// 2^-22 of the trace; sweeps stop when a sweep rotates nothing (at most kMaxSweeps).
// subspace_align_kernel: 64 tokens per workgroup, 4 lanes per token, basis rows in LDS.
// subspace_delta_kernel: one workgroup per (b, h) reduces a_t under the needle mask.
#include "ccq_device.hpp"
#include "ccq_internal.hpp"

namespace ccq {

constexpr int kMaxSweeps = 24;
constexpr int kEigThreads = 512;

template <int D>
struct EigSmem {
  float A[D][D + 1];
  alignas(16) float Vt[D][D + 4];  // row i: eigenvector i (columns of the accumulated rotation); float4 rows
  float c[D / 2], s[D / 2], t[D / 2];
  int p[D / 2], q[D / 2];
  float red[kEigThreads / 64];
  int rot;  // rotations applied in the current sweep
};

// Pair k of round-robin step `step` over d indices (d even): index d-1 stays, the others turn.
template <int D>
__device__ __forceinline__ void rr_pair(int step, int k, int& p, int& q) {
  int a, b;
  if (k == 0) {
    a = D - 1;
    b = step;
  } else {
    a = (step + k) % (D - 1);
    b = (step - k + (D - 1)) % (D - 1);
  }
  p = a < b ? a : b;
  q = a < b ? b : a;
}

template <int D>
__global__ __launch_bounds__(kEigThreads) void subspace_eigen_kernel(SubspaceArgs a) {
  constexpr int NP = D / 2;                 // pairs per step
  constexpr int NB = NP * (NP + 1) / 2;     // 2 x 2 blocks with k <= l
  __shared__ EigSmem<D> sm;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int head = blockIdx.x;
  const bool packed = (a.flags & kFlagPackedCov) != 0;
  const float* C = a.C + (size_t)head * (packed ? D * (D + 1) / 2 : D * D);
  const float* m = a.ksum + (size_t)head * D;
  const int64_t n = a.n[head];
  const float inv_n = n > 0 ? 1.0f / (float)n : 0.0f;

  // Sigma = (C + C^T) / 2n - mu mu^T  (C is symmetric by definition; the mean of the two
  // stored triangles keeps the Jacobi iteration on an exactly symmetric matrix); V = I
#pragma unroll 2
  for (int e = tid; e < D * D; e += kEigThreads) {
    const int i = e / D, j = e % D;
    float cij;
    if (packed) {
      cij = C[packed_index(i, j, D)];
    } else {
      cij = 0.5f * (C[(size_t)i * D + j] + C[(size_t)j * D + i]);
    }
    const float sij = cij * inv_n - (m[i] * inv_n) * (m[j] * inv_n);
    sm.A[i][j] = n > 0 ? sij : 0.0f;
    sm.Vt[i][j] = (i == j) ? 1.0f : 0.0f;
  }
  __syncthreads();
  // matrix scale for the skip test: sum of |diagonal| (the trace of the positive semidefinite
  // Sigma, which bounds its largest eigenvalue)
  {
    float tr = 0.f;
    for (int i = tid; i < D; i += kEigThreads) tr += fabsf(sm.A[i][i]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) tr += __shfl_xor(tr, off, 64);
    if (lane == 0) sm.red[wv] = tr;
  }
  __syncthreads();
  float scale = 0.f;
#pragma unroll
  for (int v = 0; v < kEigThreads / 64; ++v) scale += sm.red[v];
  // Off-diagonal entries below 2^-22 of the scale are left alone: an entry of size e moves an
  // eigenvalue by at most e and an eigenvector by about e over its gap.
  const float abs_floor = 2.384185791015625e-7f * scale;

  int sweep = 0;
  for (; sweep < kMaxSweeps; ++sweep) {
    if (tid == 0) sm.rot = 0;
    __syncthreads();
    for (int step = 0; step < D - 1; ++step) {
      // rotation of every pair from its 2 x 2 block
      if (tid < NP) {
        int p, q;
        rr_pair<D>(step, tid, p, q);
        const float app = sm.A[p][p], aqq = sm.A[q][q], apq = sm.A[p][q];
        float c = 1.f, s = 0.f, t = 0.f;
        if (fabsf(apq) > abs_floor && fabsf(apq) > 1e-7f * sqrtf(fabsf(app * aqq))) {
          const float tau = (aqq - app) / (2.0f * apq);
          // tan of the rotation angle, the root of t^2 + 2 tau t - 1 = 0 of smaller magnitude
          t = fabsf(tau) < 1e15f ? (tau >= 0.f ? 1.0f : -1.0f) / (fabsf(tau) + sqrtf(1.0f + tau * tau))
                                 : 0.5f / tau;
          c = 1.0f / sqrtf(1.0f + t * t);
          s = t * c;
          sm.rot = 1;  // any writer sets the same value
        }
        sm.p[tid] = p;
        sm.q[tid] = q;
        sm.c[tid] = c;
        sm.s[tid] = s;
        sm.t[tid] = t;
      }
      __syncthreads();
      // A <- J^T A J, block by block: the 2 x 2 block of pair k's rows and pair l's columns,
      // for k <= l only.  A is kept as its upper triangle (entry (i, j) read and written at
      // (min, max)), so each block is read and written once and needs no mirror.  Thread
      // groups take column pairs l and NP-1-l together, which balances the triangle.
      {
        constexpr int TPL = kEigThreads / (NP / 2);  // threads per couple of column pairs
        const int lc = tid / TPL, j0 = tid % TPL;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int l = h2 == 0 ? lc : NP - 1 - lc;
          const int pl = sm.p[l], ql = sm.q[l];
          const float cl = sm.c[l], sl = sm.s[l];
#pragma unroll 1
          for (int k = j0; k <= l; k += TPL) {
            if (k == l) {
              const float t = sm.t[k];
              if (t != 0.f) {
                const float apq = sm.A[pl][ql];
                sm.A[pl][pl] -= t * apq;
                sm.A[ql][ql] += t * apq;
                sm.A[pl][ql] = 0.f;
              }
            } else {
              const float ck = sm.c[k], sk = sm.s[k];
              if (sk == 0.f && sl == 0.f) continue;
              const int pk = sm.p[k], qk = sm.q[k];
              float* e00 = &sm.A[min(pk, pl)][max(pk, pl)];
              float* e01 = &sm.A[min(pk, ql)][max(pk, ql)];
              float* e10 = &sm.A[min(qk, pl)][max(qk, pl)];
              float* e11 = &sm.A[min(qk, ql)][max(qk, ql)];
              const float b00 = *e00, b01 = *e01, b10 = *e10, b11 = *e11;
              // rows: J_k^T B
              const float r00 = ck * b00 - sk * b10, r01 = ck * b01 - sk * b11;
              const float r10 = sk * b00 + ck * b10, r11 = sk * b01 + ck * b11;
              // columns: (J_k^T B) J_l
              *e00 = cl * r00 - sl * r01;
              *e01 = sl * r00 + cl * r01;
              *e10 = cl * r10 - sl * r11;
              *e11 = sl * r10 + cl * r11;
            }
          }
        }
      }
      // V <- V J: rows p, q of V^T, float4 at a time; each thread keeps one pair
      {
        constexpr int TPP = kEigThreads / NP;  // threads per pair
        const int k = tid / TPP, j0 = tid % TPP;
        const float s = sm.s[k];
        if (s != 0.f) {
          const float c = sm.c[k];
          const int p = sm.p[k], q = sm.q[k];
#pragma unroll
          for (int j = j0; j < D / 4; j += TPP) {
            const f32x4 vp = *reinterpret_cast<const f32x4*>(&sm.Vt[p][4 * j]);
            const f32x4 vq = *reinterpret_cast<const f32x4*>(&sm.Vt[q][4 * j]);
            *reinterpret_cast<f32x4*>(&sm.Vt[p][4 * j]) = c * vp - s * vq;
            *reinterpret_cast<f32x4*>(&sm.Vt[q][4 * j]) = s * vp + c * vq;
          }
        }
      }
      __syncthreads();
    }
    if (sm.rot == 0) break;  // uniform: read after the step's barrier
    __syncthreads();         // everyone has read rot before it is cleared
  }
  if (tid == 0 && a.sweeps != nullptr) a.sweeps[head] = sweep < kMaxSweeps ? sweep + 1 : kMaxSweeps;

  // eigenvalues in descending order (ties: lower index first); top-r eigenvectors with their
  // largest-magnitude entry made positive (lowest index among equal magnitudes)
  float* ev = a.eigvals + (size_t)head * D;
  float* basis = a.basis + (size_t)head * a.r * D;
  for (int i = tid; i < D; i += kEigThreads) {
    const float li = sm.A[i][i];
    int rank = 0;
#pragma unroll 4
    for (int j = 0; j < D; ++j) {
      const float lj = sm.A[j][j];
      rank += (lj > li || (lj == li && j < i)) ? 1 : 0;
    }
    ev[rank] = li;
    if (rank < a.r) {
      // the accumulated fp32 rotations leave each eigenvector's norm off 1 by about d^2 ulps:
      // it is rescaled to unit length on the way out
      int arg = 0;
      float best = -1.f, nrm = 0.f;
#pragma unroll 4
      for (int j = 0; j < D; ++j) {
        const float v = sm.Vt[i][j];
        nrm += v * v;
        if (fabsf(v) > best) {
          best = fabsf(v);
          arg = j;
        }
      }
      const float sg = (sm.Vt[i][arg] < 0.f ? -1.f : 1.f) / sqrtf(nrm);
#pragma unroll 4
      for (int j = 0; j < D; ++j) basis[(size_t)rank * D + j] = sg * sm.Vt[i][j];
    }
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
