// Decode step of the CCQ read (one new token per sequence and head), state in place.
//
// Per (sequence, head), following the cleaning, gate and read of the gist.science summary
// of arXiv 2606.01294 (§2 "机制", §2 "集成") with the statistics kept as sums:
//   n += 1;  C += k k^T;  ksum += k
//   Sigma q = C q / n - ksum (ksum . q) / n^2      (Cbar - mu mu^T applied to q, §2 "理论推导")
//   lambda = sigmoid(w . q + b);  q_clean = q - lambda Sigma q
//   GLA: S <- S diag(alpha) + v k^T;   GDN: S <- alpha S (I - beta k k^T) + beta v k^T
//   o = S q_clean  (S after the write)
//
// Memory-bound: every head moves its fp32 C and S (2 x d^2 x 4 bytes) in and out once.
// One 256-thread workgroup per head.  Thread t owns float4 column group (t mod d/4) of
// rows t/(d/4) + i*(256/(d/4)); every load of C and S is issued before the first
// barrier, so a workgroup has its whole 2 x d^2 x 4 bytes in flight at once.  Rows are
// reduced across the d/4 lanes that share them with xor shuffles inside a wave.
#include "ccq_device.hpp"
#include "ccq_internal.hpp"

namespace ccq {

constexpr int kDecodeThreads = 256;

template <int D, typename T, int RULE>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeArgs a) {
  constexpr int C4 = D / 4;                 // float4 per row
  constexpr int RPI = kDecodeThreads / C4;  // rows covered per iteration
  constexpr int IT = D / RPI;               // iterations per thread
  static_assert(C4 <= 64 && (64 % C4) == 0, "a row must sit inside one wave");

  const int head = blockIdx.x;  // (sequence, head) pair, 0 .. N*H-1
  const int h = head % a.H;
  const int tid = threadIdx.x;
  const int col4 = tid % C4;
  const int row0 = tid / C4;

  __shared__ float q_s[D], k_s[D], v_s[D], al_s[D], kn_s[D], r_s[D], qt_s[D];
  __shared__ float scal[4];  // lambda, msq, n (as float), k.q (unused by GLA)

  const T* qg = static_cast<const T*>(a.q) + (size_t)head * D;
  const T* kg = static_cast<const T*>(a.k) + (size_t)head * D;
  const T* vg = static_cast<const T*>(a.v) + (size_t)head * D;
  float* Cg = a.C + (size_t)head * D * D;
  float* Sg = a.S + (size_t)head * D * D;

  // Issue the state loads first: they are the bandwidth.
  f32x4 cr[IT], sr[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int row = row0 + i * RPI;
    cr[i] = *reinterpret_cast<const f32x4*>(Cg + (size_t)row * D + 4 * col4);
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int row = row0 + i * RPI;
    sr[i] = *reinterpret_cast<const f32x4*>(Sg + (size_t)row * D + 4 * col4);
  }

  float alpha_s = 1.f, beta_s = 0.f;
  if constexpr (RULE == 1) {
    alpha_s = __expf(ldf(static_cast<const T*>(a.log_alpha), head));
    beta_s = ldf(static_cast<const T*>(a.beta), head);
  }
  if (tid < D) {
    q_s[tid] = ldf(qg, tid);
    k_s[tid] = ldf(kg, tid);
    v_s[tid] = ldf(vg, tid);
    if constexpr (RULE == 0) al_s[tid] = __expf(ldf(static_cast<const T*>(a.log_alpha), (size_t)head * D + tid));
  }
  lds_barrier();

  // Wave 0: updated key sum, the gate, and ksum_new . q.
  if (tid < 64) {
    float wq = 0.f, msq = 0.f;
    for (int c = tid; c < D; c += 64) {
      const float kn = a.ksum[(size_t)head * D + c] + k_s[c];
      a.ksum[(size_t)head * D + c] = kn;
      kn_s[c] = kn;
      wq += a.w_lambda[(size_t)h * D + c] * q_s[c];
      msq += kn * q_s[c];
    }
    wq = group_sum<64>(wq);
    msq = group_sum<64>(msq);
    if (tid == 0) {
      const int64_t n1 = a.n[head] + 1;
      a.n[head] = n1;
      scal[0] = sigmoidf(wq + a.b_lambda[h]);
      scal[1] = msq;
      scal[2] = (float)n1;
    }
  }

  const f32x4 k4 = *reinterpret_cast<const f32x4*>(k_s + 4 * col4);
  const f32x4 q4 = *reinterpret_cast<const f32x4*>(q_s + 4 * col4);

  // C pass: C_new = C + k k^T, r = C_new q (row-local), write back.
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int row = row0 + i * RPI;
    const float kr = k_s[row];
    f32x4 cn = cr[i] + kr * k4;
    *reinterpret_cast<f32x4*>(Cg + (size_t)row * D + 4 * col4) = cn;
    float pr = cn[0] * q4[0] + cn[1] * q4[1] + cn[2] * q4[2] + cn[3] * q4[3];
    pr = group_sum<C4>(pr);
    if (col4 == 0) r_s[row] = pr;
  }

  // S pass: the write rule, row-local; the new state stays in registers for the read.
  if constexpr (RULE == 0) {
    const f32x4 a4 = *reinterpret_cast<const f32x4*>(al_s + 4 * col4);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int row = row0 + i * RPI;
      sr[i] = sr[i] * a4 + v_s[row] * k4;
      *reinterpret_cast<f32x4*>(Sg + (size_t)row * D + 4 * col4) = sr[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int row = row0 + i * RPI;
      float sk = sr[i][0] * k4[0] + sr[i][1] * k4[1] + sr[i][2] * k4[2] + sr[i][3] * k4[3];
      sk = group_sum<C4>(sk);
      sr[i] = alpha_s * (sr[i] - (beta_s * sk) * k4) + (beta_s * v_s[row]) * k4;
      *reinterpret_cast<f32x4*>(Sg + (size_t)row * D + 4 * col4) = sr[i];
    }
  }
  lds_barrier();  // r_s, kn_s and scal complete

  if (tid < D) {
    const float lam = scal[0], msq = scal[1], nf = scal[2];
    const float inv_n = 1.0f / nf;
    const float u = r_s[tid] * inv_n - kn_s[tid] * (msq * inv_n * inv_n);
    qt_s[tid] = q_s[tid] - lam * u;
  }
  lds_barrier();

  const f32x4 qt4 = *reinterpret_cast<const f32x4*>(qt_s + 4 * col4);
  T* og = static_cast<T*>(a.o) + (size_t)head * D;
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int row = row0 + i * RPI;
    float po = sr[i][0] * qt4[0] + sr[i][1] * qt4[1] + sr[i][2] * qt4[2] + sr[i][3] * qt4[3];
    po = group_sum<C4>(po);
    if (col4 == 0) og[row] = from_f32<T>(po);
  }
}

template <int D, typename T>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)(a.N * a.H)), block(kDecodeThreads);
  if (a.rule == 0)
    hipLaunchKernelGGL((decode_kernel<D, T, 0>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, T, 1>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.d == 128) return launch_decode_t<128, __bf16>(a, s);
    if (a.d == 64) return launch_decode_t<64, __bf16>(a, s);
  } else {
    if (a.d == 128) return launch_decode_t<128, float>(a, s);
    if (a.d == 64) return launch_decode_t<64, float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
