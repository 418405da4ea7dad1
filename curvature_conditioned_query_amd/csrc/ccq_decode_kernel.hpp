// Decode step of the CCQ read (one new token per sequence and head), state in place.  Included
// by the two translation units that instantiate it: ccq_decode.hip (full C) and
// ccq_decode_packed.hip (packed C), which the build compiles with different scheduler settings.
//
// Per (sequence, head), following the cleaning, gate and read of the gist.science summary
// of arXiv 2606.01294 (§2 "机制", §2 "集成") with the statistics kept as sums:
//   n += 1;  C += k k^T;  ksum += k
//   Sigma q = C q / n - ksum (ksum . q) / n^2      (Cbar - mu mu^T applied to q, §2 "理论推导")
//   lambda = sigmoid(w . q + b);  q_clean = q - lambda Sigma q
//   GLA: S <- S diag(alpha) + v k^T;   GDN: S <- alpha S (I - beta k k^T) + beta v k^T
//   o = S q_clean  (S after the write)
//
// Memory-bound: every head moves its fp32 C and S (2 x d^2 x 4 bytes) in and out once, with
// non-temporal loads and stores (the state is touched once per step and is far larger than
// the caches).  One workgroup of NT threads per head (1024 at d = 128).  The per-token operands (q, k, v,
// gates, ksum, n, w_lambda) are loaded first and the state after them, so the waits for the
// small operands never wait for the state (the vector-memory counter drains in order);
// then thread t owns float4 column group (t mod d/4) of rows t/(d/4) + i*(NT/(d/4)), with
// every load of C and S in flight before the first use.  Rows are reduced across the d/4
// lanes that share them with xor shuffles inside a wave; d-long dot products are reduced
// per wave and summed from LDS.
//
// Packed statistics (PACKED): C arrives as its upper triangle, row by row, d (d + 1) / 2
// floats per head.  Threads stream it as consecutive float4 (coalesced, as for the full
// matrix), find the (row, column) of each entry from its index, add k_i k_j, store it back
// and copy it into an LDS upper triangle (row-major, so the copy is contiguous across lanes).
// C q is then read from LDS in two conflict-free sweeps: the part on and right of the
// diagonal along rows (float4 per lane, masked below the diagonal) and the part left of it
// down columns (lanes on consecutive columns, so each read instruction is row-contiguous).
#pragma once

#include "ccq_device.hpp"
#include "ccq_internal.hpp"

namespace ccq {

// First row of the packed upper triangle whose entries start at or after index e: the row r
// with start(r) <= e < start(r + 1), start(r) = r d - r (r - 1) / 2.
template <int D>
__device__ __forceinline__ int packed_row_of(int e) {
  constexpr float b = 2.0f * D + 1.0f;
  int r = (int)((b - __builtin_sqrtf(b * b - 8.0f * (float)e)) * 0.5f);
  r = r < 0 ? 0 : (r > D - 1 ? D - 1 : r);
  if (packed_index(r, r, D) > e) --r;
  else if (r + 1 < D && packed_index(r + 1, r + 1, D) <= e) ++r;
  return r;
}

template <int D, typename T, int RULE, int NT, bool NORM, bool PACKED>
__global__ __launch_bounds__(NT) void decode_kernel(DecodeArgs a) {
  constexpr int C4 = D / 4;       // float4 per row
  constexpr int RPI = NT / C4;    // rows covered per iteration
  constexpr int IT = D / RPI;     // iterations per thread
  constexpr int NWV = (D + 63) / 64;  // waves holding the d-long vectors
  constexpr int TRI = D * (D + 1) / 2;  // packed entries per head
  constexpr int TQ = TRI / 4;           // ... as float4
  constexpr int PI = (TQ + NT - 1) / NT;  // packed float4 per thread (the last partly)
  constexpr int JB = NT / D, RJ = D / JB;  // column sweep: row blocks of RJ rows
  constexpr int PC = D + 4;               // pitch of the LDS triangle (float4 rows)
  static_assert(C4 <= 64 && (64 % C4) == 0, "a row must sit inside one wave");
  static_assert(IT * RPI == D, "rows must tile the workgroup");
  static_assert(TRI % 4 == 0 && JB * RJ == D, "packed layout tiles the workgroup");

  const int head = blockIdx.x;  // (sequence, head) pair, 0 .. N*H-1
  const int h = head % a.H;
  const int tid = threadIdx.x;
  const int col4 = tid % C4;
  const int row0 = tid / C4;

  __shared__ float q_s[D], k_s[D], v_s[D], al_s[D], kn_s[D], r_s[D], qt_s[D];
  __shared__ float part[3][NWV];  // per-wave partial w . q, ksum_new . q and (NORM) k . k
  __shared__ float nf_s;
  // PACKED: the updated triangle (entries left of the diagonal unused) and the column-sweep
  // partial sums
  __shared__ float tri_s[PACKED ? D : 1][PACKED ? PC : 1];
  __shared__ float colp_s[PACKED ? JB : 1][PACKED ? D : 1];

  // ---- per-token operands first (every thread loads; threads past d repeat an index)
  const int c = tid % D;
  const T qraw = static_cast<const T*>(a.q)[(size_t)head * D + c];
  const T kraw = static_cast<const T*>(a.k)[(size_t)head * D + c];
  const T vraw = static_cast<const T*>(a.v)[(size_t)head * D + c];
  const T graw = (RULE == 0) ? static_cast<const T*>(a.log_alpha)[(size_t)head * D + c]
                             : static_cast<const T*>(a.log_alpha)[head];
  const T braw = (RULE == 1) ? static_cast<const T*>(a.beta)[head] : T(0.f);
  const float mv = a.ksum[(size_t)head * D + c];
  const float wv = a.w_lambda[(size_t)h * D + c];
  const int64_t n0 = a.n[head];
  const float b_lam = a.b_lambda[h];

  // ---- then the state
  float* Cg = a.C + (size_t)head * (PACKED ? TRI : D * D);
  float* Sg = a.S + (size_t)head * D * D;
  f32x4 cr[PACKED ? PI : IT], sr[IT];
  if constexpr (PACKED) {
#pragma unroll
    for (int i = 0; i < PI; ++i) {
      const int u = tid + i * NT;
      cr[i] = (u < TQ) ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Cg) + u) : zero4();
    }
  } else {
#pragma unroll
    for (int i = 0; i < IT; ++i) cr[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Cg + (size_t)(row0 + i * RPI) * D + 4 * col4));
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) sr[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sg + (size_t)(row0 + i * RPI) * D + 4 * col4));
  // nothing that uses the operands above may be scheduled before the state loads are issued
  __builtin_amdgcn_sched_barrier(0);
  const float qv = to_f32(qraw), vv = to_f32(vraw);
  float kv = to_f32(kraw);
  if constexpr (NORM) {  // k / max(|k|, 1e-12), the d-long sum reduced per wave and from LDS
    if (tid < D) {
      const float pk = group_sum<64>(kv * kv);
      if ((tid & 63) == 0) part[2][tid >> 6] = pk;
    }
    lds_barrier();
    float ss = 0.f;
#pragma unroll
    for (int v = 0; v < NWV; ++v) ss += part[2][v];
    kv *= __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
  }
  float alpha_s = 1.f, beta_s = 0.f;
  if constexpr (RULE == 1) {
    alpha_s = __expf(to_f32(graw));
    beta_s = to_f32(braw);
  }

  // ---- token vectors to LDS, updated key sum and count, partial dot products
  if (tid < D) {
    const float kn = mv + kv;
    q_s[tid] = qv;
    k_s[tid] = kv;
    v_s[tid] = vv;
    if constexpr (RULE == 0) al_s[tid] = __expf(to_f32(graw));
    kn_s[tid] = kn;
    a.ksum[(size_t)head * D + tid] = kn;
    const float pw = group_sum<64>(wv * qv);
    const float pm = group_sum<64>(kn * qv);
    if ((tid & 63) == 0) {
      part[0][tid >> 6] = pw;
      part[1][tid >> 6] = pm;
    }
  }
  if (tid == 0) {
    const int64_t n1 = n0 + 1;
    a.n[head] = n1;
    nf_s = (float)n1;
  }
  lds_barrier();

  const f32x4 k4 = *reinterpret_cast<const f32x4*>(k_s + 4 * col4);
  const f32x4 q4 = *reinterpret_cast<const f32x4*>(q_s + 4 * col4);

  if constexpr (PACKED) {
    // C pass, packed: C_new = C + k k^T entry by entry, written back and copied to LDS.
#pragma unroll
    for (int i = 0; i < PI; ++i) {
      const int u = tid + i * NT;
      if (u < TQ) {
        const int e0 = 4 * u;
        int r = packed_row_of<D>(e0);
        int rs = packed_index(r, r, D);          // start of row r
        int re = rs + (D - r);                   // start of row r + 1
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          while (e0 + x >= re) {  // a float4 spans at most 4 rows
            ++r;
            rs = re;
            re = rs + (D - r);
          }
          const int j = r + (e0 + x - rs);
          const float cn = cr[i][x] + k_s[r] * k_s[j];
          cr[i][x] = cn;
          tri_s[r][j] = cn;
        }
        __builtin_nontemporal_store(cr[i], reinterpret_cast<f32x4*>(Cg) + u);
      }
    }
  } else {
    // C pass: C_new = C + k k^T, r = C_new q (row-local), write back.
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int row = row0 + i * RPI;
      const float kr = k_s[row];
      f32x4 cn = cr[i] + kr * k4;
      __builtin_nontemporal_store(cn, reinterpret_cast<f32x4*>(Cg + (size_t)row * D + 4 * col4));
      float pr = cn[0] * q4[0] + cn[1] * q4[1] + cn[2] * q4[2] + cn[3] * q4[3];
      pr = group_sum<C4>(pr);
      if (col4 == 0) r_s[row] = pr;
    }
  }

  // S pass: the write rule, row-local; the new state stays in registers for the read.
  if constexpr (RULE == 0) {
    const f32x4 a4 = *reinterpret_cast<const f32x4*>(al_s + 4 * col4);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int row = row0 + i * RPI;
      sr[i] = sr[i] * a4 + v_s[row] * k4;
      __builtin_nontemporal_store(sr[i], reinterpret_cast<f32x4*>(Sg + (size_t)row * D + 4 * col4));
    }
  } else {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int row = row0 + i * RPI;
      float sk = sr[i][0] * k4[0] + sr[i][1] * k4[1] + sr[i][2] * k4[2] + sr[i][3] * k4[3];
      sk = group_sum<C4>(sk);
      sr[i] = alpha_s * (sr[i] - (beta_s * sk) * k4) + (beta_s * v_s[row]) * k4;
      __builtin_nontemporal_store(sr[i], reinterpret_cast<f32x4*>(Sg + (size_t)row * D + 4 * col4));
    }
  }
  if constexpr (PACKED) {
    lds_barrier();  // triangle complete
    // on and right of the diagonal: sum_{j >= i} C_ij q_j along row i
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int row = row0 + i * RPI;
      const f32x4 cn = *reinterpret_cast<const f32x4*>(&tri_s[row][4 * col4]);
      float pr = 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const float cv = (4 * col4 + x >= row) ? cn[x] : 0.f;  // left of the diagonal: unwritten
        pr += cv * q4[x];
      }
      pr = group_sum<C4>(pr);
      if (col4 == 0) r_s[row] = pr;
    }
    // left of the diagonal: sum_{j < i} C_ji q_j down column i, in JB blocks of rows
    {
      const int col = tid % D, jb = tid / D;
      float pc = 0.f;
#pragma unroll
      for (int jj = 0; jj < RJ; ++jj) {
        const int j = jb * RJ + jj;
        const float cv = tri_s[j < col ? j : col][col];  // always a written entry
        pc += (j < col) ? cv * q_s[j] : 0.f;
      }
      colp_s[jb][col] = pc;
    }
  }
  lds_barrier();  // r_s complete

  if (tid < D) {
    float wq = 0.f, msq = 0.f;
#pragma unroll
    for (int v = 0; v < NWV; ++v) {
      wq += part[0][v];
      msq += part[1][v];
    }
    const float lam = sigmoidf(wq + b_lam);
    const float inv_n = 1.0f / nf_s;
    float rq = r_s[tid];
    if constexpr (PACKED) {
#pragma unroll
      for (int b = 0; b < JB; ++b) rq += colp_s[b][tid];
    }
    const float u = rq * inv_n - kn_s[tid] * (msq * inv_n * inv_n);
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

// Launch of the PACKED variants of decode_kernel<D, T> for the rule and flags in a.
template <int D, typename T, bool PACKED>
hipError_t launch_decode_variant(const DecodeArgs& a, hipStream_t s) {
  constexpr int NT = 8 * D;  // 1024 threads at d = 128: 4 float4 of C and of S per thread
  const dim3 grid((unsigned)(a.N * a.H)), block(NT);
  const bool norm = (a.flags & kFlagNormalizeKeys) != 0;
  if (a.rule == 0) {
    if (norm)
      hipLaunchKernelGGL((decode_kernel<D, T, 0, NT, true, PACKED>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_kernel<D, T, 0, NT, false, PACKED>), grid, block, 0, s, a);
  } else {
    if (norm)
      hipLaunchKernelGGL((decode_kernel<D, T, 1, NT, true, PACKED>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((decode_kernel<D, T, 1, NT, false, PACKED>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <bool PACKED>
hipError_t launch_decode_dtype(const DecodeArgs& a, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.d == 128) return launch_decode_variant<128, __bf16, PACKED>(a, s);
    if (a.d == 64) return launch_decode_variant<64, __bf16, PACKED>(a, s);
  } else {
    if (a.d == 128) return launch_decode_variant<128, float, PACKED>(a, s);
    if (a.d == 64) return launch_decode_variant<64, float, PACKED>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
