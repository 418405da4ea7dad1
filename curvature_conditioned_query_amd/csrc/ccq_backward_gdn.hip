// Chunked backward of the CCQ read step on a Gated DeltaNet backbone (gfx950): the gradients of a
// loss L(o, final carry) with respect to q, k, v, log alpha, beta, the gate parameters and the carry
// in, with the forward carry recomputed per chunk.
//
// The pages train CCQ models on both backbones from scratch (10100.com write-up, section "方法解析"
// point 3; gist.science summary of arXiv 2606.01294, §4), which needs this pass; the forward it
// differentiates is the chunked prefill (summary §2 "理论推导", "机制", "集成") with the Gated
// DeltaNet write rule S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
//
// Chunk algebra of the forward (rows i of a 64-token chunk, carry S_c at its start; lg_i the
// chunk-local cumulative log decay, gamma_i = e^{lg_i}, Gam_ij = gamma_i / gamma_j, D_i = gamma_L /
// gamma_i with L the chunk's last token):
//   A = strict_tril(beta_i Gam_ij k_i . k_j),  T = (I + A)^{-1},  X = diag(beta) (V - diag(gamma) K S_c^T),
//   Delta = T X,  M = tril_incl(Qc K^T) * Gam,  O = diag(gamma) Qc S_c^T + M Delta,
//   S_{c+1} = gamma_L S_c + Delta^T diag(D) K.
// Its adjoint, with dO and dS_L (the adjoint of S_{c+1}, carried back from later chunks):
//   dDelta = M^T dO + diag(D) K dS_L^T,  dX = T^T dDelta,  dM = tril_incl(dO Delta^T),
//   dQc = diag(gamma) dO S_c + (dM * Gam) K                                   (-> the read's adjoint)
//   dA = -strict_tril(dX Delta^T),  W_A = dA * beta_i Gam_ij,
//   dk (write rule) = (dM * Gam)^T Qc - diag(beta gamma) dX S_c + (W_A + W_A^T) K + diag(D) Delta dS_L,
//   dv = diag(beta) dX,  dbeta_i = dX_i . (V - diag(gamma) K S_c^T)_i + sum_j dA_ij Gam_ij k_i . k_j,
//   dlg_i = rowsum_i - colsum_i of (dM * M) and of (dA * A) + gamma_i dO_i . (Qc S_c^T)_i
//           - beta_i gamma_i dX_i . (K S_c^T)_i - D_i k_i . (Delta dS_L)_i,
//   and the chunk's last token adds gamma_L <dS_L, S_c> + sum_i D_i k_i . (Delta dS_L)_i;
//   dlog alpha_j = sum_{i >= j in the chunk} dlg_i;
//   dS_c = dS_L (gamma_L I - K^T diag(D) W) + R_c with W = T diag(beta gamma) K and
//   R_c = dO^T diag(gamma) Qc - (T^T M^T dO)^T diag(beta gamma) K.
// The last line is the reverse recurrence over chunks: the adjoint of the state is carried back by
// the transpose of the chunk's transition, a d x d matrix, not the diagonal of the GLA rule.
//
// Passes (one stream, in order):
//   1. chunk carries: the Gated DeltaNet prefill's segment summary and scans (about one segment per
//      compute unit), then a walk over each segment's chunks that writes S_c, C_c (input dtype) and
//      m_c for every chunk;
//   2. pass A, one workgroup per (chain, chunk): the read recomputed, (I + A)^{-1} formed in fp32 by
//      16-token blocks (written to the workspace), Delta, dQc, R_c, the read's adjoint (dq final,
//      the statistics part of dk, dG_c = dR^T Q, chunk sums);
//   3. reverse scans over chunks: dS_end(c) per 32-row block of the state (the matrix transition
//      above), and the additive statistics adjoints G, dm_after, dw, db;
//   4. pass B, one workgroup per (chain, chunk): dv, dk, dbeta, dlog alpha.
// Contractions are MFMAs with fp32 accumulation and operands of the input dtype, as in the GLA
// backward (ccq_backward.hip), whose strip helpers and read adjoint this file shares.
#include "ccq_backward_common.hpp"
#include "ccq_internal.hpp"
#include "ccq_prefill_gdn_kernels.hpp"

namespace ccq {

using namespace bk;

namespace {

// Segments of the carry pass: about one (chain, segment) workgroup per compute unit, as the prefill
// chooses (a function of B, H, T only, so the workspace size is too).
__host__ __device__ inline int gdn_bwd_segments(size_t chains, int NC, int* cps_out) {
  int P = (int)((256 + chains - 1) / chains);
  if (P > NC) P = NC;
  if (P < 1) P = 1;
  const int cps = (NC + P - 1) / P;
  if (cps_out) *cps_out = cps;
  return (NC + cps - 1) / cps;
}

constexpr int kTT = kL * kL;  // elements of a chunk's (I + A)^{-1}

// Workspace of one Gated DeltaNet backward call, in this order (E = the input dtype):
//   segment slots   fp32 chains x P x (3 D^2 + D) + 8 chains  (the prefill's Gated DeltaNet layout)
//   chunk carries   E    chains x NC x 2 D^2   S_c | C_c
//   chunk key sums  fp32 chains x NC x D       m_c
//   inverses        E    chains x NC x 64^2    (I + A)^{-1}
//   adjoint mats    E    chains x NC x 2 D^2   R_c | dG_c, then dS_end | G
//   adjoint tails   fp32 chains x NC x 4 D     dm | dw | db (D, [0] used) | -
//   qc, dk part     fp32 2 x chains x NC x 64 x D (strip-major)
struct GdnBwdBytes {
  size_t seg, car, carm, tinv, mat, tail, qc, dkp, total;
};

__host__ __device__ inline GdnBwdBytes gdn_bwd_bytes(size_t chains, int NC, size_t d, size_t E) {
  GdnBwdBytes b;
  const int P = gdn_bwd_segments(chains, NC, nullptr);
  size_t off = 0;
  b.seg = off;
  off += fwd_count_offset(chains, P, gdn_slot_floats((int)d) * sizeof(float)) + chains * 8;
  off = (off + 255) & ~(size_t)255;
  b.car = off;
  off += chains * NC * 2 * d * d * E;
  b.carm = off;
  off += chains * NC * d * 4;
  b.tinv = off;
  off += chains * NC * kTT * E;
  b.mat = off;
  off += chains * NC * 2 * d * d * E;
  b.tail = off;
  off += chains * NC * 4 * d * 4;
  b.qc = off;
  off += chains * NC * kL * d * 4;
  b.dkp = off;
  off += chains * NC * kL * d * 4;
  b.total = off;
  return b;
}

template <typename T>
struct GdnBwdLayout {
  float* seg;
  T* car;
  float* carm;
  T* tinv;
  T* mat;
  float* tail;
  float *qc, *dkp;
};

template <typename T>
__device__ __forceinline__ GdnBwdLayout<T> gdn_layout(const BwdArgs& a) {
  const GdnBwdBytes b = gdn_bwd_bytes((size_t)a.B * a.H, a.nchunks, (size_t)a.d, sizeof(T));
  char* w = static_cast<char*>(a.workspace);
  GdnBwdLayout<T> L{reinterpret_cast<float*>(w + b.seg), reinterpret_cast<T*>(w + b.car),
                    reinterpret_cast<float*>(w + b.carm), reinterpret_cast<T*>(w + b.tinv),
                    reinterpret_cast<T*>(w + b.mat), reinterpret_cast<float*>(w + b.tail),
                    reinterpret_cast<float*>(w + b.qc), reinterpret_cast<float*>(w + b.dkp)};
  if (a.chunk_carry != nullptr) {  // the chunk carries the forward wrote (same layout, own buffer)
    char* cc = static_cast<char*>(const_cast<void*>(a.chunk_carry));
    L.car = reinterpret_cast<T*>(cc);
    L.carm = reinterpret_cast<float*>(cc + chunk_carry_mat_bytes((size_t)a.B * a.H, (size_t)a.nchunks, (size_t)a.d, sizeof(T)));
  }
  return L;
}

// The chunk's gates into LDS (one wave, lane = token): beta, the chunk-local cumulative log decay lg
// (inclusive), gamma = e^lg, beta gamma and D = e^{lg_L - lg}; tokens at or past Lc count as
// log alpha = 0, beta = 0.  Returns gamma_L (every lane).
// chunk_gates from the token's log alpha x and beta b, already loaded (0 past the end).
__device__ __forceinline__ float chunk_gates_from(float x, float b, int lane, float* lg_, float* gam, float* beta,
                                                  float* bgam, float* dd) {
  float lg = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(lg, off, 64);
    if (lane >= off) lg += y;
  }
  const float lgL = __shfl(lg, 63, 64);
  const float ga = __expf(lg);
  if (lg_) lg_[lane] = lg;
  if (gam) gam[lane] = ga;
  if (beta) beta[lane] = b;
  if (bgam) bgam[lane] = b * ga;
  if (dd) dd[lane] = __expf(lgL - lg);
  return __expf(lgL);
}

template <typename T>
__device__ __forceinline__ float chunk_gates(const T* gg, const T* bg, size_t row0, int Lc, int lane, float* lg_,
                                             float* gam, float* beta, float* bgam, float* dd) {
  const bool ok = lane < Lc;
  const float x = ok ? ldf(gg, row0 + lane) : 0.f;
  const float b = ok ? ldf(bg, row0 + lane) : 0.f;
  return chunk_gates_from(x, b, lane, lg_, gam, beta, bgam, dd);
}

// acc = X Y for 16 x 16 fp32 blocks in LDS (fp32 MFMA, K in slices of 4: lane (g, l) supplies
// X[l][4 g + r] and Y[4 g + r][l] for slice r); acc[r] at lane (g, l) is (X Y)[4 g + r][l].
__device__ __forceinline__ f32x4 mm16(const float* X, int px, const float* Y, int py, int lane, f32x4 acc) {
  const int g = lane >> 4, l = lane & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[l * px + 4 * g + r], Y[(4 * g + r) * py + l], acc, 0, 0, 0);
  return acc;
}

// acc = -X Z for a 16 x 16 fp32 block X in LDS and Z held in accumulator layout (Z[4 g + r][l] in
// element r of lane (g, l), which is exactly the B operand of slice r).
__device__ __forceinline__ f32x4 neg_mm16_acc(const float* X, int px, const f32x4& z, int lane) {
  const int g = lane >> 4, l = lane & 15;
  f32x4 acc = zero4();
#pragma unroll
  for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-X[l * px + 4 * g + r], z[r], acc, 0, 0, 0);
  return acc;
}

// Index of the off-diagonal 16 x 16 block (i, j), i > j, of a 64 x 64 lower-triangular matrix:
// (1,0) (2,1) (3,2) by the first diagonal, then (2,0) (3,1), then (3,0).
__device__ __forceinline__ int offd(int i, int j) { return (i - j == 1) ? j : (i - j == 2) ? 3 + j : 5; }

// (I + A)^{-1} of a chunk in fp32 by 16-token blocks, A strictly lower triangular in the LDS tile As
// (pitch PT; its lower blocks are read, its upper blocks serve as scratch).  Diagonal blocks on the
// last four waves, one each, by the product form of the prefill (diag_block_inverse_mfma);
// off-diagonal ones from T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj, one block per wave and diagonal,
// the nearest diagonal first, on waves 0..2.  Results: Tb (diagonal blocks), To (off-diagonal,
// indexed by offd), both [.][16][20] fp32.  Every thread of the workgroup calls it; it ends with a
// barrier.  `between` runs on every wave after the diagonal blocks are out, before the off-diagonal
// rounds (work for the last waves, which take no part in those).
template <int NW, typename Between>
__device__ __forceinline__ void chunk_inverse(float (*As)[PT], float (*Tb)[16][20], float (*To)[16][20], int w, int lane,
                                              Between&& between) {
  static_assert(NW >= 4, "the diagonal blocks take four waves, the first off-diagonal round three");
  if (w >= NW - 4) diag_block_inverse_mfma(As, Tb, w - (NW - 4), lane);
  __syncthreads();
  between();
  const int g = lane >> 4, l = lane & 15;
  for (int dgl = 1; dgl <= 3; ++dgl) {
    if (w < 4 - dgl) {
      const int i = w + dgl, j = w;
      // Z = A_ij T_jj + sum_{k=j+1}^{i-1} A_ik T_kj
      f32x4 z = mm16(&As[16 * i][16 * j], PT, &Tb[j][0][0], 20, lane, zero4());
      for (int k = j + 1; k < i; ++k) z = mm16(&As[16 * i][16 * k], PT, &To[offd(k, j)][0][0], 20, lane, z);
      const f32x4 t = neg_mm16_acc(&Tb[i][0][0], 20, z, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) To[offd(i, j)][4 * g + r][l] = t[r];
    }
    __syncthreads();
  }
}

// Element (i, j) of (I + A)^{-1} from its blocks (zero above the diagonal).
__device__ __forceinline__ float inv_at(const float (*Tb)[16][20], const float (*To)[16][20], int i, int j) {
  const int bi = i >> 4, bj = j >> 4;
  if (bj > bi) return 0.f;
  return bi == bj ? Tb[bi][i & 15][j & 15] : To[offd(bi, bj)][i & 15][j & 15];
}

// out[ti] += X rows (64 x D LDS tile, pitch px) times the D x 16 block M[cw .. cw + 15][:]^T of a
// global row-major matrix M (read as rows: out = X M^T restricted to M's rows cw ..).
template <int D, typename O, typename TX, typename TM>
__device__ __forceinline__ void strip_times_rowsT(const TX* X, int px, const TM* M, int cw, int lane, f32x4 (&out)[4]) {
  strip_times_sym<D, O>(X, px, M, cw, lane, out);
}

}  // namespace

// ---------------------------------------------------------------- 1. chunk carries

// Carry at every chunk start of a segment, from the segment's carry-in (the prefill's Gated
// DeltaNet summary and scans; for segment 0, the caller's carry or zeros): before chunk c it writes
// S_c, C_c (input dtype) and m_c, then applies the chunk's update with the prefill's own steps
// (A, the diagonal-block inverses, X, the blocked solve, the state and statistic updates).  Only a
// chain's last chunk can be ragged, and the carry after it is never needed, so every chunk applied
// here is a whole one.
template <int D, typename T>
__global__ __launch_bounds__(4 * D) void gdn_bwd_walk_kernel(BwdArgs a, int P, int cps) {
  using C_ = Cfg<D, T>;
  constexpr int NW = C_::NW, NA = C_::NA, PQ = C_::PQ, NT = 64 * NW;
  constexpr int EPU = 16 / (int)sizeof(T), NU = kL / EPU;  // 16-byte units of a 64-token gate row
  __shared__ GdnSmem<D, T> sm;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), cw = 16 * w;
  const int NC = a.nchunks;
  const int chain = blockIdx.x / P, seg = blockIdx.x % P;
  const int c0 = seg * cps, c1 = min(NC, c0 + cps);
  const size_t DD = (size_t)D * D;
  const GdnBwdLayout<T> L = gdn_layout<T>(a);
  const float *S_in = nullptr, *C_in = nullptr, *m_in = nullptr;
  if (P > 1 && seg > 0) {  // the scans left the carry-in of segments 1.. in their slots
    const float* slot = L.seg + ((size_t)chain * P + seg) * gdn_slot_floats(D);
    S_in = slot;
    C_in = slot + DD;
    m_in = slot + 2 * DD;
  } else if (a.S0 != nullptr) {
    S_in = a.S0 + (size_t)chain * DD;
    C_in = a.C0 + (size_t)chain * DD;
    m_in = a.ksum0 + (size_t)chain * D;
  }
  const T* kg = static_cast<const T*>(a.k);
  const T* vg = static_cast<const T*>(a.v);
  const T* gg = static_cast<const T*>(a.log_alpha);
  const T* bg = static_cast<const T*>(a.beta);
  T* gr = &sm.Qa[0][0];  // raw log alpha | beta of chunk c at gr + 2 kL (c & 1) (the walk reads no query)
  auto row0_of = [&](int c) { return (size_t)chain * a.T + (size_t)c * kL; };
  // Only the chunks before the segment's last are applied, and those are whole: the chain's last
  // chunk, the only one that can be ragged, is never applied (the carry after it is not needed).
  auto issue_kg = [&](int c) {  // chunk c's keys and raw gates
    dma_tile<D, T, PQ>(sm.Ks[c & 1], kg + row0_of(c) * D, kL, w, NW, lane);
    if (w == 0 && lane < 2 * NU) {
      const T* src = lane < NU ? gg + row0_of(c) + EPU * lane : bg + row0_of(c) + EPU * (lane - NU);
      dma_lane(gr + 2 * kL * (c & 1), src);
    }
  };
  auto issue_v = [&](int c) { dma_tile<D, T, PQ>(sm.Vs, vg + row0_of(c) * D, kL, w, NW, lane); };

  // Sacc[t] = S^T[16 t + 4 g + r][cw + l16], Cacc[t] = C[16 t + 4 g + r][cw + l16] (C symmetric)
  f32x4 Sacc[NA], Cacc[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    const size_t o = (size_t)(cw + l16) * D + 16 * t + 4 * g;
    Sacc[t] = S_in ? *reinterpret_cast<const f32x4*>(S_in + o) : zero4();
    Cacc[t] = C_in ? *reinterpret_cast<const f32x4*>(C_in + o) : zero4();
  }
  if (tid < D) sm.m0[tid] = m_in ? m_in[tid] : 0.f;
  if (c0 < c1 - 1) {
    issue_kg(c0);
    issue_v(c0);
  }
  vm_wait_all();
  __syncthreads();
  auto store_carry = [&](int c) {  // the carry at chunk c's start: S_c, C_c (input dtype), m_c
    const size_t cs = (size_t)chain * NC + c;
    T* Sd = L.car + cs * 2 * DD;
    T* Cd = Sd + DD;
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      const size_t o = (size_t)(cw + l16) * D + 16 * t + 4 * g;
      st4<T>(Sd + o, Sacc[t]);
      st4<T>(Cd + o, Cacc[t]);
    }
    if (tid < D) L.carm[cs * D + tid] = sm.m0[tid];
  };
  for (int c = c0; c < c1; ++c) {
    if (c == c1 - 1) {
      store_carry(c);
      break;
    }
    const bool more = c + 1 < c1 - 1;  // chunk c + 1 is applied too: its tiles stream in meanwhile
    if (more) issue_kg(c + 1);  // buffers (c + 1) & 1 were last read in the chunk before
    T (*Ks)[PQ] = sm.Ks[c & 1];
    if (w == 1) {
      const T* gc = gr + 2 * kL * (c & 1);
      gdn_gates<D, T>(sm, to_f32(gc[lane]), to_f32(gc[kL + lane]), lane);
    }
    lds_barrier();
    gdn_build_A<D, T>(sm, Ks, w, NW, lane);
    if (tid >= 2 * D) gdn_key_sums<D, T>(sm, Ks, tid - 2 * D);
    lds_barrier();
    if (w >= NW - 4) gdn_diag_inverse_mfma<D, T>(sm, w - (NW - 4), lane);
    f32x4 X[4];
    gdn_rhs<D, T, true>(sm, Ks, [&](int t) -> const f32x4& { return Sacc[t]; }, cw, lane, X);
    lds_barrier();  // the value tile is read
    if (more) issue_v(c + 1);
    // the carry at chunk c's start, issued after every load of the step so that the step's closing
    // wait need not wait for these stores
    store_carry(c);
    f32x4 Dl[4];
    gdn_solve<D, T>(sm, X, lane, Dl);
    gdn_state_update<D, T>(sm, Ks, [&](int t) -> f32x4& { return Sacc[t]; }, Dl, lane);
    gdn_cov_update<D, T>(Ks, Cacc, cw, lane);
    lds_barrier();  // every wave is done with the chunk's tiles and m1
    if (tid < D) sm.m0[tid] = sm.m1[tid];
    // chunk c + 1 has landed once at most this step's 2 NA (+ 1) carry stores are outstanding
    if constexpr (NA == 8) {
      asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    } else {
      static_assert(NA == 4, "store count per chunk");
      asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    }
    lds_barrier();
  }
}

// ---------------------------------------------------------------- 2. pass A

namespace {
template <int D, typename T>
struct SmemGA {
  static constexpr int PQ = Cfg<D, T>::PQ, PF = pf<D>(), NW = D / 16, PE = kL + 16 / (int)sizeof(T);
  union {
    T Q[kL][PQ];       // q (read only by the recomputed read)
    float As[kL][PT];  // then A (fp32)
    T Dt[kL][PQ];      // then Delta (operand dtype)
  } u0;
  T K[kL][PQ];
  union {
    struct {
      union {
        T V[kL][PQ];   // v (read by X only)
        T Qc[kL][PQ];  // then the cleaned query
      } vq;
      T dO[kL][PQ];
    } in;
    float dR[kL][PF];  // the read's adjoint, once Qc and dO are no longer read
  } u1;
  float P[kL][PT];     // tril(Q K^T)
  T Tm[kL][PE];        // (I + A)^{-1}
  union {
    T Mt[kL][PE];      // tril(Qc K^T) * Gam, then tril(dO Delta^T) * Gam
    struct {
      float Tb[4][16][20];
      float To[6][16][20];
    } inv;
  } u2;
  union {
    T Zt[kL][PQ];      // T^T M^T dO
    float M2[kL][PT];  // then tril(dR K^T)
  } u3;
  float red[NW][kL][2];
  f32x4 tok[kL];
  float tok2[kL][2];
  float lg[kL], gam[kL], beta[kL], bgam[kL];
};
}  // namespace

template <int D, typename T>
__global__ __launch_bounds__(4 * D) void gdn_bwd_a_kernel(BwdArgs a) {
  using SM = SmemGA<D, T>;
  using O = T;
  constexpr int NW = D / 16, NT = 64 * NW, PQ = SM::PQ, PF = SM::PF, PE = SM::PE, NA = D / 16;
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), cw = 16 * w;
  const int NC = a.nchunks;
  const int chain = blockIdx.x / NC, c = blockIdx.x % NC, h = chain % a.H;
  const int t0 = c * kL, Lc = min(kL, a.T - t0);
  const size_t row0 = (size_t)chain * a.T + t0;
  const GdnBwdLayout<T> L = gdn_layout<T>(a);
  const size_t slot = (size_t)chain * NC + c;
  const T* Sc = L.car + slot * 2 * D * D;
  const T* Cc = Sc + (size_t)D * D;
  const float* mc = L.carm + slot * D;
  T* bmat = L.mat + slot * 2 * D * D;
  float* tail = L.tail + slot * 4 * D;
  const size_t sv = (slot * NW + w) * kL * 16;  // this wave's strip in the strip-major buffers
  const int64_t nc = (a.n0 != nullptr ? a.n0[chain] : 0) + t0;

  // the chunk's reads, issued together: token tiles straight from HBM into LDS, the wave's fragments of
  // C_c (both products with it take them from registers), the gates and scalars
  dma_tile<D, T, PQ>(sm.u0.Q, static_cast<const T*>(a.q) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.K, static_cast<const T*>(a.k) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.u1.in.vq.V, static_cast<const T*>(a.v) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.u1.in.dO, static_cast<const T*>(a.d_o) + row0 * D, Lc, w, NW, lane);
  Frag<O> cf[D / 32];
  sym_frags<D, O>(Cc, cw, lane, cf);
  const float wv = a.w_lambda[(size_t)h * D + cw + l16];
  const float mv = mc[cw + l16];
  const float b_lam = a.b_lambda[h];
  if (w == 0)
    chunk_gates<T>(static_cast<const T*>(a.log_alpha), static_cast<const T*>(a.beta), row0, Lc, lane, sm.lg, sm.gam,
                   sm.beta, sm.bgam, nullptr);
  vm_wait_all();
  __syncthreads();
  if (Lc < kL) {  // a ragged last chunk: rows past the end of the sequence read as zeros
    zero_tail<D, T, PQ>(sm.u0.Q, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.K, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.u1.in.vq.V, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.u1.in.dO, Lc, tid, NT);
    __syncthreads();
  }

  f32x4 qs[4], ks[4];
  read_strip(&sm.u0.Q[0][0], PQ, cw, lane, qs);
  read_strip(&sm.K[0][0], PQ, cw, lane, ks);
  // the read recomputed: token scalars, P = tril(Q K^T), u and the cleaned query
  f32x4 us[4], qc[4];
  read_forward<D, O, NW>(&sm.u0.Q[0][0], &sm.K[0][0], PQ, sm.P, sm.red, sm.tok, cf, wv, mv, b_lam, nc, qs, ks, tid, us,
                         qc);
  store_strip_vec(L.qc + sv, lane, qc);
  __syncthreads();  // the q tile is no longer read

  // A = strict_tril(beta_i Gam_ij k_i . k_j) on the lower 16 x 16 tiles (fp32, over the q tile)
  for (int idx = w; idx < 10; idx += NW) {
    const int ti = tri_row(idx), tj = tri_col(idx);
    f32x4 acc = zero4();  // k_j . k_i at j = 16 tj + 4 g + r, i = 16 ti + l16
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      mma(acc, lds_frag<O, KORD_CONTIG>(&sm.K[0][0], PQ, 16 * tj, 32 * kk, lane),
          lds_frag<O, KORD_CONTIG>(&sm.K[0][0], PQ, 16 * ti, 32 * kk, lane));
    const int i = 16 * ti + l16, j0 = 16 * tj + 4 * g;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      sm.u0.As[i][j0 + r] = (j0 + r < i) ? sm.beta[i] * __expf(sm.lg[i] - sm.lg[j0 + r]) * acc[r] : 0.f;
  }
  __syncthreads();
  // X = beta (V - gamma K S_c^T) on the wave's value channels: on the waves that do not form the
  // diagonal blocks' inverses while that runs, on the waves that do while waves 0..2 form the
  // off-diagonal blocks
  f32x4 x[4];
  auto form_x = [&]() {
    f32x4 vs[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) x[ti] = zero4();
    strip_times_rowsT<D, O>(&sm.K[0][0], PQ, Sc, cw, lane, x);  // (K S_c^T)[i][cw + l]
    read_strip(&sm.u1.in.vq.V[0][0], PQ, cw, lane, vs);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + 4 * g + r;
        x[ti][r] = sm.beta[i] * (vs[ti][r] - sm.gam[i] * x[ti][r]);
      }
    // the wave's v columns are read: the cleaned query takes their place (same columns)
    write_strip(&sm.u1.in.vq.Qc[0][0], PQ, cw, lane, qc);
  };
  if (w < NW - 4) form_x();
  chunk_inverse<NW>(sm.u0.As, sm.u2.inv.Tb, sm.u2.inv.To, w, lane, [&]() {
    if (w >= NW - 4) form_x();
  });
  // (I + A)^{-1} in the operand dtype: to LDS for the products here and to the workspace for the
  // reverse scan and pass B
  {
    T* tw = L.tinv + slot * kTT;
    for (int e = tid; e < kTT; e += NT) {
      const T x = (T)inv_at(sm.u2.inv.Tb, sm.u2.inv.To, e >> 6, e & 63);
      sm.Tm[e >> 6][e & 63] = x;
      tw[e] = x;
    }
  }
  // Delta = T X
  f32x4 dl[4];
  {
    __syncthreads();  // Tm complete
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) dl[ti] = zero4();
    tril_times_strip<O>(&sm.Tm[0][0], PE, x, lane, dl);
  }
  write_strip(&sm.u0.Dt[0][0], PQ, cw, lane, dl);  // A and the fp32 blocks of T are no longer read
  __syncthreads();
  // M = tril(Qc K^T) * Gam
  for (int idx = w; idx < 16; idx += NW) {
    const int ti = idx >> 2, tj = idx & 3;
    const f32x4 acc = tril_tile<D, O>(&sm.u1.in.vq.Qc[0][0], PQ, &sm.K[0][0], PQ, ti, tj, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * g + r, j = 16 * tj + l16;
      sm.u2.Mt[i][j] = (T)(j <= i ? acc[r] * __expf(sm.lg[i] - sm.lg[j]) : 0.f);
    }
  }
  __syncthreads();
  f32x4 dos[4];
  read_strip(&sm.u1.in.dO[0][0], PQ, cw, lane, dos);
  // Z' = T^T M^T dO (the part of dX that does not depend on dS_L), to LDS for R_c
  {
    f32x4 z[4], zp[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) z[ti] = zp[ti] = zero4();
    trilT_times_strip<O>(&sm.u2.Mt[0][0], PE, dos, lane, z);
    trilT_times_strip<O>(&sm.Tm[0][0], PE, z, lane, zp);
    write_strip(&sm.u3.Zt[0][0], PQ, cw, lane, zp);
  }
  __syncthreads();  // M is no longer read; Z' is visible
  // dM * Gam = tril(dO Delta^T) * Gam (over M)
  for (int idx = w; idx < 16; idx += NW) {
    const int ti = idx >> 2, tj = idx & 3;
    const f32x4 acc = tril_tile<D, O>(&sm.u1.in.dO[0][0], PQ, &sm.u0.Dt[0][0], PQ, ti, tj, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * g + r, j = 16 * tj + l16;
      sm.u2.Mt[i][j] = (T)(j <= i ? acc[r] * __expf(sm.lg[i] - sm.lg[j]) : 0.f);
    }
  }
  // R_c = dO^T diag(gamma) Qc - Z'^T diag(beta gamma) K: the chunk's part of the adjoint of S_c that
  // does not go through dS_L
  {
    f32x4 gq[4], bk_[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + 4 * g + r;
        gq[ti][r] = sm.gam[i] * qc[ti][r];
        bk_[ti][r] = -sm.bgam[i] * ks[ti][r];
      }
#pragma unroll 2
    for (int ta = 0; ta < NA; ++ta) {
      f32x4 acc = tileT_times_strip<O>(&sm.u1.in.dO[0][0], PQ, ta, gq, lane);
      acc += tileT_times_strip<O>(&sm.u3.Zt[0][0], PQ, ta, bk_, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) bmat[(size_t)(16 * ta + 4 * g + r) * D + cw + l16] = (T)acc[r];
    }
  }
  __syncthreads();  // dM * Gam is visible
  // dQc = diag(gamma) dO S_c + (dM * Gam) K
  f32x4 dqc[4];
  {
    f32x4 os[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) os[ti] = dqc[ti] = zero4();
    strip_times_mat<D, O>(&sm.u1.in.dO[0][0], PQ, Sc, cw, lane, os);
    tril_times_strip<O>(&sm.u2.Mt[0][0], PE, ks, lane, dqc);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) dqc[ti][r] += sm.gam[16 * ti + 4 * g + r] * os[ti][r];
  }
  // the read's adjoint: dq, the chunk's statistics part of dk, dG_c and the chunk sums (dR is
  // written over the Qc and dO tiles, tril(dR K^T) over Z': none is read after this)
  read_adjoint<D, O, NW, PF>(&sm.K[0][0], PQ, sm.P, sm.u1.dR, sm.u3.M2, sm.red, sm.tok, sm.tok2, cf, wv, mv, qs, ks,
                             us, dqc, tid, Lc, a.dq + row0 * D, L.dkp + sv, bmat + (size_t)D * D, tail);
}

// ---------------------------------------------------------------- 3. reverse scans

// dS_end(c) for every chunk, walking the chunks of a chain backwards: dS_end(NC-1) = dS_T (or 0),
//   dS_end(c-1) = gamma_L dS_end(c) - (((dS_end(c) K^T) * D) T * (beta gamma)) K + R_c,
// and what is left after chunk 0 is the adjoint of the carry in.  Workgroup (32-row block of dS,
// chain), two waves of 16 rows each; a wave keeps its rows transposed in MFMA accumulators
// (dSt[a][r] at lane (g, l) = dS[v0 + l][16 a + 4 g + r]), so the running adjoint never leaves the
// registers.  dS_end(c) replaces R_c in the workspace (input dtype).
// The same walk carries the additive adjoints: G(c) = dC_T + sum over later chunks of dG (the second
// half of each chunk's adjoint matrices, replaced in place) on the workgroup's 32 rows, and, on the
// first row block of a chain, dm_after(c) (replacing the chunk's dm) with dw and db summed; their
// loads go out at the top of a chunk's step and the sums at its end, in the shadow of the dS chain.
// The walk is software-pipelined one chunk ahead, and every read goes straight from HBM into LDS
// (direct loads the compiler does not wait for): while chunk c is applied, chunk c-1's key tile,
// inverse, R block and raw gates stream into the other half of two LDS buffers.  Each wave forms the
// chunk's gates itself (a 64-lane scan into its own LDS slots), so one wait and one barrier per
// chunk suffice, and the wait leaves the chunk's dS_end stores in flight.
template <int D, typename T>
__global__ __launch_bounds__(128) void gdn_bwd_scan_s_kernel(BwdArgs a) {
  using O = T;
  constexpr int PQ = Cfg<D, T>::PQ, PE = kL + 16 / (int)sizeof(T), NA = D / 16;
  constexpr int EPU = 16 / (int)sizeof(T), NU = kL / EPU;  // 16-byte units of a 64-token gate row
  __shared__ T Ks[2][kL][PQ];
  __shared__ T Tm[2][kL][PE];
  __shared__ T Rs[2][32][PQ];   // the workgroup's 32 rows of R_c
  __shared__ T Gr[2][2][kL];    // raw log alpha, beta
  __shared__ __align__(16) float dd[2][kL];    // per wave: D, beta gamma (its own copies)
  __shared__ __align__(16) float bgam[2][kL];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chain = blockIdx.y, r0 = 32 * blockIdx.x, v0 = r0 + 16 * w;
  const int NC = a.nchunks;
  const size_t DD = (size_t)D * D;
  const GdnBwdLayout<T> L = gdn_layout<T>(a);
  const T* kg = static_cast<const T*>(a.k);
  const T* gg = static_cast<const T*>(a.log_alpha);
  const T* bg = static_cast<const T*>(a.beta);
  auto chunk_len = [&](int c) { return min(kL, a.T - c * kL); };
  auto row0_of = [&](int c) { return (size_t)chain * a.T + (size_t)c * kL; };
  auto rmat = [&](int c) { return L.mat + ((size_t)chain * NC + c) * 2 * DD; };
  // chunk c's key tile, inverse and R block into buffer c & 1 (both waves), its raw gates (wave 0;
  // a whole chunk only: the ragged last chunk's gates are written in the prologue)
  auto issue = [&](int c, int ln) {
    dma_tile<D, T, PQ>(Ks[c & 1], kg + row0_of(c) * D, chunk_len(c), w, 2, ln);
    dma_tile<kL, T, PE>(Tm[c & 1], L.tinv + ((size_t)chain * NC + c) * kTT, kL, w, 2, ln);
    dma_block<D, T, PQ, 32>(Rs[c & 1], rmat(c) + (size_t)r0 * D, w, 2, ln);
    if (w == 0 && ln < 2 * NU) {
      const T* src = ln < NU ? gg + row0_of(c) + EPU * ln : bg + row0_of(c) + EPU * (ln - NU);
      dma_lane(&Gr[c & 1][0][0], src);
    }
  };

  f32x4 dSt[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t)
    dSt[t] = a.dS_T ? *reinterpret_cast<const f32x4*>(a.dS_T + (size_t)chain * DD + (size_t)(v0 + l16) * D + 16 * t + 4 * g)
                    : zero4();
  // G on rows r0 .. r0 + 31: thread tid owns 16-byte vectors tid + 128 j
  constexpr int EPV = 16 / (int)sizeof(T), GV = 32 * D / EPV / 128;
  static_assert(GV * 128 * EPV == 32 * D, "whole vectors per thread");
  T* gmat = L.mat + (size_t)chain * NC * 2 * DD + DD + (size_t)r0 * D;  // chunk 0's G block
  float grun[GV][EPV];
#pragma unroll
  for (int j = 0; j < GV; ++j) {
    const float* src = a.dC_T ? a.dC_T + (size_t)chain * DD + (size_t)r0 * D + (size_t)(tid + 128 * j) * EPV : nullptr;
#pragma unroll
    for (int e = 0; e < EPV; ++e) grun[j][e] = src ? src[e] : 0.f;
  }
  // tails dm | dw | db (first row block): thread tid < 3D/4 owns 4 floats of part (4 tid) / D
  const bool tails = blockIdx.x == 0 && tid < 3 * D / 4;
  const int tpart = (4 * tid) / D;  // 0 dm (scanned), 1 dw, 2 db (summed)
  // (every thread reads a whole-block address, so the loads below need no branch: 4 (tid mod D) < 4 D)
  float* tbase = L.tail + (size_t)chain * NC * 4 * D + 4 * (tid & (D - 1));
  f32x4 trun = (tails && tpart == 0 && a.dksum_T) ? *reinterpret_cast<const f32x4*>(a.dksum_T + (size_t)chain * D + 4 * tid)
                                                   : zero4();
  // chunk c's dG on the workgroup's rows and its tails, loaded one step ahead of their use so that
  // the wait for them never waits for the direct loads issued after them
  auto load_sums = [&](int c, u32x4 (&gx)[GV], f32x4& tx) {
#pragma unroll
    for (int j = 0; j < GV; ++j) gx[j] = *reinterpret_cast<const u32x4*>(gmat + (size_t)c * 2 * DD + (size_t)(tid + 128 * j) * EPV);
    const f32x4 t = *reinterpret_cast<const f32x4*>(tbase + (size_t)c * 4 * D);
    tx = tails ? t : zero4();
  };
  u32x4 gx[GV];
  f32x4 tx = zero4();
  if (NC > 0) load_sums(NC - 1, gx, tx);
  if (NC > 0) {
    const int c = NC - 1, Lc = chunk_len(c);
    if (Lc == kL) {
      issue(c, lane);
    } else {  // the ragged last chunk: gates written here (zero past the end), key rows zeroed below
      dma_tile<D, T, PQ>(Ks[c & 1], kg + row0_of(c) * D, Lc, w, 2, lane);
      dma_tile<kL, T, PE>(Tm[c & 1], L.tinv + ((size_t)chain * NC + c) * kTT, kL, w, 2, lane);
      dma_block<D, T, PQ, 32>(Rs[c & 1], rmat(c) + (size_t)r0 * D, w, 2, lane);
      if (w == 0) {
        const bool ok = lane < Lc;
        const size_t i = row0_of(c) + (ok ? lane : 0);
        const T x = gg[i], b = bg[i];
        Gr[c & 1][0][lane] = ok ? x : T(0.f);
        Gr[c & 1][1][lane] = ok ? b : T(0.f);
      }
    }
    vm_wait_all();
    __syncthreads();
    if (Lc < kL) {
      zero_tail<D, T, PQ>(Ks[c & 1], Lc, tid, 128);
      __syncthreads();
    }
  }
  vm_wait_all();  // also on the path that skipped the prologue's loads: none is pending in the walk
  for (int c = NC - 1; c >= 0; --c) {
    // lane index recomputed per chunk (opaque), so lane-derived addresses are not held across the loop
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const int gq = ln >> 4, lq = ln & 15;
    u32x4 gxn[GV];  // chunk c - 1's (chunk 0's again on the last step: not used)
    f32x4 txn;
    load_sums(c > 0 ? c - 1 : 0, gxn, txn);
    if (c > 0) issue(c - 1, ln);  // buffers (c - 1) & 1 were last read in the chunk before
    {
      T* R = rmat(c) + (size_t)(v0 + lq) * D + 4 * gq;
#pragma unroll
      for (int t = 0; t < NA; ++t) st4<T>(R + 16 * t, dSt[t]);  // dS_end(c), over R_c (read from LDS)
    }
    const int b = c & 1;
    // this wave's copy of the chunk's gates: lg = inclusive scan of log alpha, D = e^{lg_L - lg},
    // beta gamma = beta e^{lg}, gamma_L
    float gL;
    {
      float lg = to_f32(Gr[b][0][ln]);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(lg, off, 64);
        if (ln >= off) lg += y;
      }
      const float lgL = __shfl(lg, 63, 64);
      dd[w][ln] = __expf(lgL - lg);
      bgam[w][ln] = to_f32(Gr[b][1][ln]) * __expf(lg);
      gL = __expf(lgL);
    }
    const T (*Kc)[PQ] = Ks[b];
    const T (*Tc)[PE] = Tm[b];
    // Y^T = K dS^T (token rows), scaled by D
    f32x4 y[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) y[ti] = zero4();
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const Frag<O> bf = acc_frag<O>(dSt[2 * kk], dSt[2 * kk + 1]);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) mma(y[ti], lds_frag<O, KORD_ACC>(&Kc[0][0], PQ, 16 * ti, 32 * kk, ln), bf);
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) y[ti] *= *reinterpret_cast<const f32x4*>(&dd[w][16 * ti + 4 * gq]);
    // Y'^T = T^T (D Y^T), scaled by beta gamma
    f32x4 yp[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) yp[ti] = zero4();
    trilT_times_strip<O>(&Tc[0][0], PE, y, ln, yp);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) yp[ti] *= *reinterpret_cast<const f32x4*>(&bgam[w][16 * ti + 4 * gq]);
    // dS^T = gamma_L dS^T - K^T Y'^T + R_c^T
#pragma unroll
    for (int t = 0; t < NA; ++t) dSt[t] = gL * dSt[t] + ld4<T>(&Rs[b][16 * w + lq][16 * t + 4 * gq]);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const Frag<O> bf = acc_frag<O>(yp[2 * kk], yp[2 * kk + 1]);
#pragma unroll
      for (int t = 0; t < NA; ++t) {
        f32x4 acc = zero4();
        mma(acc, tile_cols<O, KORD_ACC>(&Kc[0][0], PQ, 32 * kk, 16 * t, ln), bf);
        dSt[t] -= acc;
      }
    }
    // G(c) and dm_after(c) in place, then the chunk's own terms join the running sums (the loaded
    // terms pass through an empty asm here, so nothing reads them, and no wait for them falls,
    // before this point)
#pragma unroll
    for (int j = 0; j < GV; ++j) asm volatile("" : "+v"(gx[j]));
    asm volatile("" : "+v"(tx));
#pragma unroll
    for (int j = 0; j < GV; ++j) {
      *reinterpret_cast<uint4*>(gmat + (size_t)c * 2 * DD + (size_t)(tid + 128 * j) * EPV) = pack16<T>(grun[j]);
      float x[EPV];
      unpack16<T>(__builtin_bit_cast(uint4, gx[j]), x);
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        grun[j][e] += x[e];
        asm volatile("" : "+v"(grun[j][e]));  // the sums stay in this step, ahead of the wait below
      }
    }
    if (tails) {
      if (tpart == 0) *reinterpret_cast<f32x4*>(tbase + (size_t)c * 4 * D) = trun;
      trun += tx;
    }
#pragma unroll
    for (int j = 0; j < GV; ++j) gx[j] = gxn[j];
    tx = txn;
    if (c > 0) {
      // chunk c - 1 has landed once only the stores issued after its loads (NA of dS_end, GV of G,
      // and on some waves one tail) may be outstanding; the barrier also frees chunk c's buffers
      // for chunk c - 2
      constexpr int after = NA + GV;
      if constexpr (after == 12) {
        asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      } else if constexpr (after == 8) {
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      } else {
        static_assert(after == 6, "store count per chunk");
        asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      }
      lds_barrier();
    }
  }
  if (a.dS0 != nullptr) {
#pragma unroll
    for (int t = 0; t < NA; ++t)
      *reinterpret_cast<f32x4*>(a.dS0 + (size_t)chain * DD + (size_t)(v0 + l16) * D + 16 * t + 4 * g) = dSt[t];
  }
  if (a.dC0 != nullptr) {
#pragma unroll
    for (int j = 0; j < GV; ++j)
#pragma unroll
      for (int e = 0; e < EPV; ++e) a.dC0[(size_t)chain * DD + (size_t)r0 * D + (size_t)(tid + 128 * j) * EPV + e] = grun[j][e];
  }
  if (tails) {
    if (tpart == 0 && a.dksum0) *reinterpret_cast<f32x4*>(a.dksum0 + (size_t)chain * D + 4 * tid) = trun;
    if (tpart == 1) *reinterpret_cast<f32x4*>(a.dw + (size_t)chain * D + (4 * tid - D)) = trun;
    if (tpart == 2 && 4 * tid == 2 * D) a.db[chain] = trun[0];
  }
}

// ---------------------------------------------------------------- 4. pass B

namespace {
template <int D, typename T>
struct SmemGB {
  static constexpr int PQ = Cfg<D, T>::PQ, NW = D / 16, PE = kL + 16 / (int)sizeof(T);
  T K[kL][PQ];
  T dO[kL][PQ];
  union {
    T V[kL][PQ];   // v (read by X only)
    T Qc[kL][PQ];  // then the cleaned query
  } vq;
  T Dt[kL][PQ];    // Delta
  T dXt[kL][PQ];   // dX
  union {
    T Tm[kL][PE];  // (I + A)^{-1}
    T dA[kL][PE];  // then -strict_tril(dX Delta^T), then W_A = dA * beta Gam
  } u0;
  union {
    T Mt[kL][PE];  // tril(Qc K^T) * Gam
    T AK[kL][PE];  // then strict_tril(Gam K K^T)
  } u1;
  T dM[kL][PE];    // tril(dO Delta^T), then * Gam
  T Scs[D][PQ];    // S_c
  float red[NW][kL][4];
  float lg[kL], gam[kL], beta[kL], bgam[kL], dd[kL];
  float dlg[kL], db2[kL];
  float dot[NW];
};
}  // namespace

template <int D, typename T>
__global__ __launch_bounds__(4 * D) void gdn_bwd_b_kernel(BwdArgs a) {
  using SM = SmemGB<D, T>;
  using O = T;
  constexpr int NW = D / 16, NT = 64 * NW, PQ = SM::PQ, PE = SM::PE;
  __shared__ SM sm;
  constexpr int EPU = 16 / (int)sizeof(T), NP = D * D / (EPU * NT);  // dS_end blocks per thread (the dot below)
  static_assert(NP * EPU * NT == D * D, "dS_end splits evenly over the workgroup");
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), cw = 16 * w;
  const int NC = a.nchunks;
  const int chain = blockIdx.x / NC, c = blockIdx.x % NC;
  const int t0 = c * kL, Lc = min(kL, a.T - t0);
  const size_t row0 = (size_t)chain * a.T + t0;
  const GdnBwdLayout<T> L = gdn_layout<T>(a);
  const size_t slot = (size_t)chain * NC + c;
  const size_t DD = (size_t)D * D;
  const T* Sc = L.car + slot * 2 * DD;
  const T* dSe = L.mat + slot * 2 * DD;  // dS_end(c)
  const T* Ga = dSe + DD;                // G(c)
  const float dma = L.tail[slot * 4 * D + cw + l16];
  const size_t sv = (slot * NW + w) * kL * 16;
  const int rtok = 16 * (l16 >> 2) + 4 * g + (l16 & 3);  // the token chan_reduce16 leaves here

  // the chunk's reads, issued together: token tiles, the inverse and S_c straight from HBM into LDS,
  // the cleaned-query strip and this thread's 16-byte blocks of dS_end (for <dS_L, S_c>) into registers
  dma_tile<D, T, PQ>(sm.K, static_cast<const T*>(a.k) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.dO, static_cast<const T*>(a.d_o) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.vq.V, static_cast<const T*>(a.v) + row0 * D, Lc, w, NW, lane);
  dma_tile<kL, T, PE>(sm.u0.Tm, L.tinv + slot * kTT, kL, w, NW, lane);
#pragma unroll
  for (int hh = 0; hh < D / kL; ++hh) dma_tile<D, T, PQ>(&sm.Scs[kL * hh], Sc + (size_t)kL * hh * D, kL, w, NW, lane);
  uint4 dsb[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) dsb[p] = *reinterpret_cast<const uint4*>(dSe + (size_t)(tid + NT * p) * EPU);
  f32x4 qcs[4];
  load_strip_vec(L.qc + sv, lane, qcs);
  float gL = 0.f;
  if (w == 0)
    gL = chunk_gates<T>(static_cast<const T*>(a.log_alpha), static_cast<const T*>(a.beta), row0, Lc, lane, sm.lg, sm.gam,
                        sm.beta, sm.bgam, sm.dd);
  vm_wait_all();
  __syncthreads();
  if (Lc < kL) {  // a ragged last chunk: rows past the end of the sequence read as zeros
    zero_tail<D, T, PQ>(sm.K, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.dO, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.vq.V, Lc, tid, NT);
    __syncthreads();
  }
  // <dS_L, S_c>: this thread's blocks, summed over the wave (the waves' sums are added at the end)
  {
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int f = (tid + NT * p) * EPU;
      float x[EPU], y[EPU];
      unpack16<T>(dsb[p], x);
      unpack16<T>(*reinterpret_cast<const uint4*>(&sm.Scs[f / D][f % D]), y);
#pragma unroll
      for (int e = 0; e < EPU; ++e) s += x[e] * y[e];
    }
    {  // wave sum, lane index taken opaque here so that its shuffle addresses are not kept to the end
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
#pragma unroll
      for (int off = 32; off > 0; off >>= 1)
        s += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((ln ^ off) << 2, __builtin_bit_cast(int, s)));
    }
    if (lane == 0) sm.dot[w] = s;
  }

  f32x4 ks[4], dos[4];
  read_strip(&sm.K[0][0], PQ, cw, lane, ks);
  read_strip(&sm.dO[0][0], PQ, cw, lane, dos);
  // K (G + G^T): the statistics part of dk from later tokens
  f32x4 kg[4];
  {
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) kg[ti] = zero4();
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const Frag<O> gc = frag_cols<O, KORD_CONTIG>(Ga, D, 32 * kk, cw, lane);  // G[c][kappa]
      const Frag<O> gr = frag_rows<O, KORD_CONTIG>(Ga, D, cw, 32 * kk, lane);  // G[kappa][c]
      Frag<O> b;
#pragma unroll
      for (int e = 0; e < 8; ++e) b.v[e] = cvt<O>(to_f32(gc.v[e]) + to_f32(gr.v[e]));
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) mma(kg[ti], lds_frag<O, KORD_CONTIG>(&sm.K[0][0], PQ, 16 * ti, 32 * kk, lane), b);
    }
  }
  // KS = K S_c^T, xr = V - gamma KS, X = beta xr, Delta = T X (value channels cw + l)
  f32x4 KS[4], xr[4], dl[4];
  {
    f32x4 vs[4], x[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) KS[ti] = dl[ti] = zero4();
    strip_times_tile_rows<D, O>(&sm.K[0][0], PQ, &sm.Scs[0][0], PQ, cw, lane, KS);
    read_strip(&sm.vq.V[0][0], PQ, cw, lane, vs);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + 4 * g + r;
        xr[ti][r] = vs[ti][r] - sm.gam[i] * KS[ti][r];
        x[ti][r] = sm.beta[i] * xr[ti][r];
      }
    tril_times_strip<O>(&sm.u0.Tm[0][0], PE, x, lane, dl);
  }
  write_strip(&sm.Dt[0][0], PQ, cw, lane, dl);
  write_strip(&sm.vq.Qc[0][0], PQ, cw, lane, qcs);  // over the wave's own v columns, already read
  __syncthreads();
  // M = tril(Qc K^T) * Gam and dM = tril(dO Delta^T)
  for (int idx = w; idx < 16; idx += NW) {
    const int ti = idx >> 2, tj = idx & 3;
    const f32x4 m = tril_tile<D, O>(&sm.vq.Qc[0][0], PQ, &sm.K[0][0], PQ, ti, tj, lane);
    const f32x4 dm = tril_tile<D, O>(&sm.dO[0][0], PQ, &sm.Dt[0][0], PQ, ti, tj, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * g + r, j = 16 * tj + l16;
      sm.u1.Mt[i][j] = (T)(j <= i ? m[r] * __expf(sm.lg[i] - sm.lg[j]) : 0.f);
      sm.dM[i][j] = (T)dm[r];  // zero above the diagonal already
    }
  }
  __syncthreads();
  // dlg from Gam in M: rowsum_i - colsum_i of dM * M, token i = lane, each wave over its share of
  // j (partial sums parked in red, which the channel sums at the end are the first to write again)
  constexpr int JW = kL / NW;
  {
    float s = 0.f;
#pragma unroll 1
    for (int j = JW * w; j < JW * (w + 1); ++j)
      s += to_f32(sm.dM[lane][j]) * to_f32(sm.u1.Mt[lane][j]) - to_f32(sm.dM[j][lane]) * to_f32(sm.u1.Mt[j][lane]);
    sm.red[w][lane][0] = s;
  }
  // dDelta = M^T dO + D (K dS_L^T), dX = T^T dDelta, dv = beta dX
  f32x4 dX[4];
  {
    f32x4 ddl[4], kd[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) ddl[ti] = kd[ti] = dX[ti] = zero4();
    trilT_times_strip<O>(&sm.u1.Mt[0][0], PE, dos, lane, ddl);
    strip_times_rowsT<D, O>(&sm.K[0][0], PQ, dSe, cw, lane, kd);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) ddl[ti][r] += sm.dd[16 * ti + 4 * g + r] * kd[ti][r];
    trilT_times_strip<O>(&sm.u0.Tm[0][0], PE, ddl, lane, dX);
    f32x4 dv[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) dv[ti][r] = sm.beta[16 * ti + 4 * g + r] * dX[ti][r];
    store_strip_rows<D>(a.dv + row0 * D, Lc, cw, lane, dv);
  }
  write_strip(&sm.dXt[0][0], PQ, cw, lane, dX);
  __syncthreads();  // T, M and the dlg sums over dM * M are done; dX is visible
  // dA = -strict_tril(dX Delta^T) (over T) and AK = strict_tril(Gam K K^T) (over M)
  for (int idx = w; idx < 16; idx += NW) {
    const int ti = idx >> 2, tj = idx & 3;
    const f32x4 da = tril_tile<D, O>(&sm.dXt[0][0], PQ, &sm.Dt[0][0], PQ, ti, tj, lane);
    const f32x4 kk = tril_tile<D, O>(&sm.K[0][0], PQ, &sm.K[0][0], PQ, ti, tj, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * g + r, j = 16 * tj + l16;
      sm.u0.dA[i][j] = (T)(j < i ? -da[r] : 0.f);
      sm.u1.AK[i][j] = (T)(j < i ? kk[r] * __expf(sm.lg[i] - sm.lg[j]) : 0.f);
    }
  }
  __syncthreads();
  // dlg from Gam in A (A = beta_i AK): rowsum_i - colsum_i of dA * A; dbeta's second term
  // sum_j dA_ij AK_ij (the same split over waves)
  {
    float rs = 0.f, cs = 0.f;
#pragma unroll 1
    for (int j = JW * w; j < JW * (w + 1); ++j) {
      rs += to_f32(sm.u0.dA[lane][j]) * to_f32(sm.u1.AK[lane][j]);
      cs += sm.beta[j] * to_f32(sm.u0.dA[j][lane]) * to_f32(sm.u1.AK[j][lane]);
    }
    sm.red[w][lane][1] = rs;
    sm.red[w][lane][2] = cs;
  }
  __syncthreads();  // dA, AK and dM are read for the sums
  if (tid < kL) {  // the waves' partial sums
    float s1 = 0.f, rs = 0.f, cs = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      s1 += sm.red[v][tid][0];
      rs += sm.red[v][tid][1];
      cs += sm.red[v][tid][2];
    }
    sm.db2[tid] = rs;
    sm.dlg[tid] = s1 + sm.beta[tid] * rs - cs;
  }
  // W_A = dA * beta_i Gam_ij (over dA), dM * Gam (over dM)
  for (int e = tid; e < kL * kL; e += NT) {
    const int i = e >> 6, j = e & 63;
    const float gm = j <= i ? __expf(sm.lg[i] - sm.lg[j]) : 0.f;
    sm.u0.dA[i][j] = (T)(to_f32(sm.u0.dA[i][j]) * sm.beta[i] * gm);
    sm.dM[i][j] = (T)(to_f32(sm.dM[i][j]) * gm);
  }
  __syncthreads();
  // dk (write rule) = (dM * Gam)^T Qc - diag(beta gamma) dX S_c + (W_A + W_A^T) K + diag(D) Delta dS_L
  f32x4 dkr[4], dsl[4], xs[4];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) dkr[ti] = dsl[ti] = xs[ti] = zero4();
  trilT_times_strip<O>(&sm.dM[0][0], PE, qcs, lane, dkr);
  tril_times_strip<O>(&sm.u0.dA[0][0], PE, ks, lane, dkr);
  trilT_times_strip<O>(&sm.u0.dA[0][0], PE, ks, lane, dkr);
  strip_times_tile<D, O>(&sm.dXt[0][0], PQ, &sm.Scs[0][0], PQ, cw, lane, xs);
  strip_times_mat<D, O>(&sm.Dt[0][0], PQ, dSe, cw, lane, dsl);
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * g + r;
      dsl[ti][r] *= sm.dd[i];
      dkr[ti][r] += dsl[ti][r] - sm.bgam[i] * xs[ti][r];
    }
  {
    f32x4 dkp[4], dk[4];
    load_strip_vec(L.dkp + sv, lane, dkp);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) dk[ti] = dkr[ti] + kg[ti] + dkp[ti] + dma;
    store_strip_rows<D>(a.dk + row0 * D, Lc, cw, lane, dk);
  }
  // per-token channel sums: dX . xr (dbeta), dX . KS, dO . (Qc S_c^T), k . (D Delta dS_L) (dlg)
  {
    f32x4 qS[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) qS[ti] = zero4();
    strip_times_tile_rows<D, O>(&sm.vq.Qc[0][0], PQ, &sm.Scs[0][0], PQ, cw, lane, qS);
    float v0[16], v1[16], v2[16], v3[16];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v0[4 * ti + r] = dX[ti][r] * xr[ti][r];
        v1[4 * ti + r] = dX[ti][r] * KS[ti][r];
        v2[4 * ti + r] = dos[ti][r] * qS[ti][r];
        v3[4 * ti + r] = ks[ti][r] * dsl[ti][r];
      }
    sm.red[w][rtok][0] = chan_reduce16(v0, l16);
    sm.red[w][rtok][1] = chan_reduce16(v1, l16);
    sm.red[w][rtok][2] = chan_reduce16(v2, l16);
    sm.red[w][rtok][3] = chan_reduce16(v3, l16);
  }
  __syncthreads();
  if (w == 0) {
    const int i = lane;
    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
    for (int v = 0; v < NW; ++v) {
      r0 += sm.red[v][i][0];
      r1 += sm.red[v][i][1];
      r2 += sm.red[v][i][2];
      r3 += sm.red[v][i][3];
    }
    const float dbeta = r0 + sm.db2[i];
    float dlg = sm.dlg[i] + sm.gam[i] * r2 - sm.bgam[i] * r1 - r3;
    float dot = 0.f;
    for (int v = 0; v < NW; ++v) dot += sm.dot[v];
    const float s3 = group_sum<64>(r3);
    if (i == kL - 1) dlg += gL * dot + s3;
    // dlog alpha_j = sum_{i >= j} dlg_i
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(dlg, off, 64);
      if (i + off < 64) dlg += y;
    }
    if (i < Lc) {
      a.dlog_alpha[row0 + i] = dlg;
      a.dbeta[row0 + i] = dbeta;
    }
  }
}

// ---------------------------------------------------------------- launch

size_t gdn_bwd_workspace_bytes(int B, int H, int T, int d, int dtype) {
  const size_t chains = (size_t)B * H;
  const int NC = (T + kL - 1) / kL;
  return gdn_bwd_bytes(chains, NC, (size_t)d, dtype == 1 ? 2 : 4).total;
}

template <int D, typename T>
static hipError_t launch_gdn_bwd_t(const BwdArgs& a, hipStream_t s) {
  const int chains = a.B * a.H, NC = a.nchunks;
  auto rec = [&](int i) -> hipError_t {
    return a.events ? hipEventRecord(static_cast<hipEvent_t>(a.events[i]), s) : hipSuccess;
  };
  int cps = 0;
  const int P = gdn_bwd_segments((size_t)chains, NC, &cps);
  // 1. carries at every chunk start: the prefill's segment summary and scans, then the walk
  FwdArgs f{};
  f.rule = 1;
  f.dtype = a.dtype;
  f.B = a.B;
  f.H = a.H;
  f.T = a.T;
  f.d = D;
  f.segments = P;
  f.chunks_per_segment = cps;
  f.k = a.k;
  f.v = a.v;
  f.log_alpha = a.log_alpha;
  f.beta = a.beta;
  f.S0 = a.S0;
  f.C0 = a.C0;
  f.ksum0 = a.ksum0;
  f.n0 = a.n0;
  f.workspace = a.workspace;  // the segment slots come first in the workspace
  if (rec(0) != hipSuccess) return hipErrorLaunchFailure;
  if (a.chunk_carry == nullptr) {  // else the forward wrote them and gdn_layout() points at its buffer
    if (P > 1) {
      const hipError_t es = launch_gdn_summary(f, s);
      if (es != hipSuccess) return es;
      hipLaunchKernelGGL((gdn_scan_state_kernel<D>), dim3(D / 16, (unsigned)chains), dim3(2 * D), 0, s, f);
      hipLaunchKernelGGL((gdn_scan_sum_kernel<D>), dim3((unsigned)((D * D + D + 255) / 256), (unsigned)chains),
                         dim3(256), 0, s, f);
    }
    hipLaunchKernelGGL((gdn_bwd_walk_kernel<D, T>), dim3((unsigned)(chains * P)), dim3(4 * D), 0, s, a, P, cps);
  }
  if (rec(1) != hipSuccess) return hipErrorLaunchFailure;
  // 2. pass A
  hipLaunchKernelGGL((gdn_bwd_a_kernel<D, T>), dim3((unsigned)(chains * NC)), dim3(4 * D), 0, s, a);
  if (rec(2) != hipSuccess) return hipErrorLaunchFailure;
  // 3. reverse scans
  hipLaunchKernelGGL((gdn_bwd_scan_s_kernel<D, T>), dim3(D / 32, (unsigned)chains), dim3(128), 0, s, a);
  if (rec(3) != hipSuccess) return hipErrorLaunchFailure;
  // 4. pass B
  hipLaunchKernelGGL((gdn_bwd_b_kernel<D, T>), dim3((unsigned)(chains * NC)), dim3(4 * D), 0, s, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return rec(4);
}

hipError_t launch_gdn_bwd(const BwdArgs& a, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.d == 128) return launch_gdn_bwd_t<128, __bf16>(a, s);
    if (a.d == 64) return launch_gdn_bwd_t<64, __bf16>(a, s);
  } else if (a.d == 64) {
    return launch_gdn_bwd_t<64, float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
