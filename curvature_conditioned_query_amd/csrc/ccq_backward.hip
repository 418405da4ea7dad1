// Chunked backward of the CCQ read step on a GLA backbone (gfx950): the gradients of a loss
// L(o, final carry) with respect to q, k, v, log alpha, the gate parameters and the carry in,
// with the forward carry recomputed per chunk.
//
// The pages train CCQ models from scratch (10100.com write-up, section "方法解析" point 3),
// which needs this pass; the forward it differentiates is the one of the chunked prefill
// (gist.science summary of arXiv 2606.01294, §2 "理论推导", "机制", "集成"; GLA write rule
// S_t = S_{t-1} diag(alpha_t) + v_t k_t^T).
//
// Per token (sums C_i, m_i, count n_i include token i):
//   u_i = C_i q_i / n_i - m_i sq_i / n_i^2,  sq_i = m_i . q_i,  lambda_i = sigmoid(w . q_i + b)
//   qc_i = q_i - lambda_i u_i,  o_i = S_i qc_i
// Adjoint of the read, with dqc_i the gradient of L with respect to qc_i:
//   dlogit_i = -(u_i . dqc_i) lambda_i (1 - lambda_i),  dr_i = -lambda_i dqc_i / n_i
//   ds_i = -(m_i . dr_i) / n_i,  dm_i = ds_i q_i - (sq_i / n_i) dr_i
//   dq_i = dqc_i + dlogit_i w + C_i dr_i + ds_i m_i
//   and C_i = C_c + sum_{j<=i} k_j k_j^T, m_i = m_c + sum_{j<=i} k_j give every earlier key
//   dk_j += sum_{i>=j} [dr_i (q_i . k_j) + q_i (dr_i . k_j) + dm_i].
// Chunk algebra (chunk c of 64 tokens, carry at its start S_c, C_c, m_c, n_c; B_i the
// chunk-local inclusive cumulative log decay per key channel, B_L its value at the last token;
// P = Q K^T, M = dR K^T, D = dO V^T, A = (Qc e^B)(K e^-B)^T, all lower-triangular incl.):
//   dQc = e^B * (dO S_c + tril(D) (K e^-B))
//   dq  = dQc + dlogit w^T + dR C_c + ds * (m_c + cumsum K) + tril(M) K
//   dk  = tril(P)^T dR + tril(M)^T Q + revcumsum(dm)                (statistics, this chunk)
//       + K (G + G^T) + dm_after                                  (statistics, later tokens)
//       + e^-B * (tril(D)^T (Qc e^B)) + e^{B_L - B} * (V dS_end)   (write rule)
//   dv  = tril(A)^T dO + (K e^{B_L - B}) dS_end^T
//   dlog alpha_i = sum_{s>=i in chunk} (qc_s * dqc_s - k_s * dk^{rule}_s)
//                + e^{B_L} * colsum(S_c * dS_end) + sum_j k_j * (e^{B_L - B_j} * (V dS_end)_j)
// where dS_end is the adjoint of the state at the chunk's end carried back from later chunks,
// G = dC_T + sum over later tokens of dr_i q_i^T, dm_after = dksum_T + sum over later tokens of
// dm_i.  The last line is the standard gate identity for a diagonal decay (the gradient of a
// token's log decay is the suffix sum of qc * dqc - k * dk plus the final column sums of
// S * dS), with the tokens after the chunk folded into S_end * dS_end and S_end written in terms
// of S_c and the chunk's own terms.
//
// Passes (one stream, in order):
//   1. chunk carries: the prefill's segment summary and scan, then a walk over each segment's
//      chunks that writes S_c, C_c (input dtype) and m_c for every chunk (workspace);
//   2. pass A, one workgroup per (chain, chunk): the forward read recomputed, dQc, the read
//      adjoint, dq (final), the chunk's own statistics part of dk (partial, into dk), and the
//      chunk's contributions R_c = dO^T (Qc e^B), dG_c = dR^T Q, sum dm, sum dlogit q, sum dlogit;
//   3. reverse scan over chunks, elementwise: dS_end(c), G(c), dm_after(c), and the carry-in
//      adjoints dS0 = dS_start(0), dC0, dksum0; dw, db summed over chunks;
//   4. pass B, one workgroup per (chain, chunk): dv, the rest of dk, dlog alpha.
// Every contraction is an MFMA with fp32 accumulation and operands of the input dtype
// (v_mfma_f32_16x16x32_bf16 for bf16 inputs, v_mfma_f32_16x16x4_f32 for fp32 inputs); wave w
// of a workgroup owns the 16 channels [16w, 16w + 16) of d: a "strip" holds, in accumulator layout, a [64 tokens] x [16 channels] block (element r of lane
// (g = lane / 16, l = lane % 16) of tile ti is token 16 ti + 4 g + r, channel 16 w + l).
#include <type_traits>

#include "ccq_internal.hpp"
#include "ccq_prefill_common.hpp"

#include "ccq_backward_common.hpp"

namespace ccq {

using namespace bk;

namespace {


// Workspace of one backward call, in this order (E = the input dtype; fp32 where noted):
//   segment slots      fp32 chains x NC x (2 D^2 + 2 D)  S | C | ksum | log decay (prefill layout;
//                                                       the first chains x P of them used)
//   chunk carries      E    chains x NC x 2 D^2          S_c | C_c
//   chunk key sums     fp32 chains x NC x D              m_c
//   adjoint matrices   E    chains x NC x 2 D^2          R_c | dG_c, then dS_end | G
//   adjoint tails      fp32 chains x NC x 4 D            dm | dw | db (D, [0] used) | B_L
//   qc, qc * dqc, dk   fp32 3 x chains x NC x 64 x D  (strip-major: a lane's 16 values contiguous)
// The carries and the adjoint matrices are MFMA operands of the input dtype anyway, so they
// are stored in it; every running sum is fp32 (in the scans' registers).
struct BwdLayoutBytes {
  size_t sum, car, carm, mat, tail, qc, qdq, dkp, total;
};

__host__ __device__ inline BwdLayoutBytes bwd_layout_bytes(size_t chains, size_t NC, size_t d, size_t E) {
  BwdLayoutBytes L;
  size_t off = 0;
  L.sum = off;
  off += chains * NC * (2 * d * d + 2 * d) * 4;
  L.car = off;
  off += chains * NC * 2 * d * d * E;
  L.carm = off;
  off += chains * NC * d * 4;
  L.mat = off;
  off += chains * NC * 2 * d * d * E;
  L.tail = off;
  off += chains * NC * 4 * d * 4;
  L.qc = off;
  off += chains * NC * kL * d * 4;
  L.qdq = off;
  off += chains * NC * kL * d * 4;
  L.dkp = off;
  off += chains * NC * kL * d * 4;
  L.total = off;
  return L;
}

template <typename T>
struct BwdLayout {
  float* sum;   // segment summaries
  T* car;       // S_c | C_c per chunk
  float* carm;  // m_c per chunk
  T* mat;       // R_c | dG_c, then dS_end | G, per chunk
  float* tail;  // dm | dw | db | B_L per chunk
  float *qc, *qdq, *dkp;  // cleaned query, qc * dqc, pass A's part of dk (strip-major)
};

template <typename T>
__device__ __forceinline__ BwdLayout<T> layout(const BwdArgs& a) {
  const BwdLayoutBytes b = bwd_layout_bytes((size_t)a.B * a.H, (size_t)a.nchunks, (size_t)a.d, sizeof(T));
  char* w = static_cast<char*>(a.workspace);
  BwdLayout<T> L{reinterpret_cast<float*>(w + b.sum), reinterpret_cast<T*>(w + b.car),
                 reinterpret_cast<float*>(w + b.carm), reinterpret_cast<T*>(w + b.mat),
                 reinterpret_cast<float*>(w + b.tail), reinterpret_cast<float*>(w + b.qc),
                 reinterpret_cast<float*>(w + b.qdq), reinterpret_cast<float*>(w + b.dkp)};
  if (a.chunk_carry != nullptr) {  // the chunk carries the forward wrote (same layout, own buffer)
    char* cc = static_cast<char*>(const_cast<void*>(a.chunk_carry));
    L.car = reinterpret_cast<T*>(cc);
    L.carm = reinterpret_cast<float*>(cc + chunk_carry_mat_bytes((size_t)a.B * a.H, (size_t)a.nchunks, (size_t)a.d, sizeof(T)));
  }
  return L;
}

template <typename T>
__device__ __forceinline__ void st4t(T* p, const f32x4& v) { st4<T>(p, v); }
template <typename T>
__device__ __forceinline__ f32x4 ld4t(const T* p) { return ld4<T>(p); }

template <int D, typename T>
struct SmemA {
  static constexpr int PQ = Cfg<D, T>::PQ, PF = pf<D>(), NW = D / 16;
  union {
    struct {
      T V[kL][PQ];
      T dO[kL][PQ];
    } in;
    float dR[kL][PF];  // once V and dO are no longer read
  } u1;
  T Q[kL][PQ];
  T K[kL][PQ];
  float P[kL][PT];
  union {
    T G[kL][PQ];
    float Dm[kL][PT];  // tril(dO V^T), then tril(dR K^T)
  } u2;
  T Sst[D][PQ];      // S_c, staged with 16-byte loads
  float red[NW][kL][2];
  f32x4 tok[kL];     // lambda, 1/n, sq/n, -
  float tok2[kL][2]; // dlogit, m_c . dr then ds
};

}  // namespace

template <int D, typename T>
__global__ __launch_bounds__(4 * D) void bwd_chunk_a_kernel(BwdArgs a) {
  using SM = SmemA<D, T>;
  using O = T;
  constexpr int NW = D / 16, NT = 64 * NW, PQ = SM::PQ, PF = SM::PF, NA = D / 16;
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), cw = 16 * w;
  const int NC = a.nchunks;
  const int chain = blockIdx.x / NC, c = blockIdx.x % NC, h = chain % a.H;
  const int t0 = c * kL, Lc = min(kL, a.T - t0);
  const size_t row0 = (size_t)chain * a.T + t0;
  const BwdLayout<T> L = layout<T>(a);
  const size_t slot = (size_t)chain * NC + c;
  const T* Sc = L.car + slot * 2 * D * D;
  const T* Cc = Sc + (size_t)D * D;
  const float* mc = L.carm + slot * D;
  T* bmat = L.mat + slot * 2 * D * D;
  float* tail = L.tail + slot * 4 * D;
  const size_t sv = (slot * NW + w) * kL * 16;  // this wave's strip in the strip-major buffers
  const int64_t nc = (a.n0 != nullptr ? a.n0[chain] : 0) + t0;

  // every read of the chunk, issued at once: the token tiles and S_c straight from HBM into LDS, the
  // wave's fragments of C_c (both products with it take them from registers) and the scalars
  dma_tile<D, T, PQ>(sm.Q, static_cast<const T*>(a.q) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.K, static_cast<const T*>(a.k) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.u2.G, static_cast<const T*>(a.log_alpha) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.u1.in.V, static_cast<const T*>(a.v) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.u1.in.dO, static_cast<const T*>(a.d_o) + row0 * D, Lc, w, NW, lane);
#pragma unroll
  for (int hh = 0; hh < D / kL; ++hh) dma_tile<D, T, PQ>(&sm.Sst[kL * hh], Sc + (size_t)kL * hh * D, kL, w, NW, lane);
  Frag<O> cf[D / 32];
  sym_frags<D, O>(Cc, cw, lane, cf);
  const float wv = a.w_lambda[(size_t)h * D + cw + l16];
  const float mv = mc[cw + l16];
  const float b_lam = a.b_lambda[h];
  vm_wait_all();
  __syncthreads();
  if (Lc < kL) {  // a ragged last chunk: rows past the end of the sequence read as zeros
    zero_tail<D, T, PQ>(sm.Q, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.K, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.u2.G, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.u1.in.V, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.u1.in.dO, Lc, tid, NT);
    __syncthreads();
  }

  f32x4 qs[4], ks[4], bs[4];
  {
    f32x4 gs[4];
    read_strip(&sm.Q[0][0], PQ, cw, lane, qs);
    read_strip(&sm.K[0][0], PQ, cw, lane, ks);
    read_strip(&sm.u2.G[0][0], PQ, cw, lane, gs);
    strip_cumsum<O, true>(gs, bs, lane);
  }
  // the read recomputed: token scalars, P = tril(Q K^T), u and the cleaned query
  f32x4 us[4], qc[4];
  read_forward<D, O, NW>(&sm.Q[0][0], &sm.K[0][0], PQ, sm.P, sm.red, sm.tok, cf, wv, mv, b_lam, nc, qs, ks, tid, us,
                         qc);
  store_strip_vec(L.qc + sv, lane, qc);

  // D = tril(dO V^T) (into the log-decay tile: every wave has read its strip of it)
  for (int idx = w; idx < 16; idx += NW) {
    const int ti = idx >> 2, tj = idx & 3;
    const f32x4 acc = tril_tile<D, O>(&sm.u1.in.dO[0][0], PQ, &sm.u1.in.V[0][0], PQ, ti, tj, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.u2.Dm[16 * ti + 4 * g + r][16 * tj + l16] = acc[r];
  }
  // R_c = dO^T (qc e^B): the read's contribution to the adjoint of S_c
  {
    f32x4 qh[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) qh[ti][r] = qc[ti][r] * __expf(bs[ti][r]);
#pragma unroll 2
    for (int ta = 0; ta < NA; ++ta) {
      const f32x4 acc = tileT_times_strip<O>(&sm.u1.in.dO[0][0], PQ, ta, qh, lane);
#pragma unroll
      for (int r = 0; r < 4; ++r) bmat[(size_t)(16 * ta + 4 * g + r) * D + cw + l16] = (T)acc[r];
    }
  }
  __syncthreads();

  // dQc = e^B * (dO S_c + tril(D) (K e^-B))
  f32x4 dqc[4];
  {
    f32x4 kh[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      dqc[ti] = zero4();
#pragma unroll
      for (int r = 0; r < 4; ++r) kh[ti][r] = ks[ti][r] * __expf(-bs[ti][r]);
    }
    strip_times_tile<D, O>(&sm.u1.in.dO[0][0], PQ, &sm.Sst[0][0], PQ, cw, lane, dqc);
    tril_times_strip<O>(&sm.u2.Dm[0][0], PT, kh, lane, dqc);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) dqc[ti][r] *= __expf(bs[ti][r]);
  }
  {
    f32x4 qdq[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) qdq[ti] = qc[ti] * dqc[ti];
    store_strip_vec(L.qdq + sv, lane, qdq);
  }
  // the read's adjoint: dq, the chunk's statistics part of dk, dG_c = dR^T Q and the chunk sums (dR
  // is written over the V and dO tiles, tril(dR K^T) over D: none is read after this)
  read_adjoint<D, O, NW, PF>(&sm.K[0][0], PQ, sm.P, sm.u1.dR, sm.u2.Dm, sm.red, sm.tok, sm.tok2, cf, wv, mv, qs, ks,
                             us, dqc, tid, Lc, a.dq + row0 * D, L.dkp + sv, bmat + (size_t)D * D, tail);
  if (g == 3) tail[3 * D + cw + l16] = bs[3][3];
}

namespace {
template <int D, typename T>
struct SmemW {
  static constexpr int PQ = Cfg<D, T>::PQ;
  T K[2][kL][PQ];
  T V[2][kL][PQ];
  T G[2][kL][PQ];  // log decay; each wave then overwrites its own channels with k e^-B
  float eBL[D];
};
}  // namespace

// Carry at every chunk start, walking the chunks of a segment from the segment's carry-in (the
// prefill's segment summary and scan; for one segment, the carry in): before chunk c it writes
// the carry (S_c, C_c in the input dtype, m_c fp32), then applies the chunk's update
//   C += K^T K,  m += sum k,  S = (S + V^T (K e^-B)) diag(e^{B_63})
// (the prefill's carry update).  One workgroup per (chain, segment); wave w keeps rows
// [16w, 16w + 16) of S (value rows) and the matching columns of C in MFMA accumulators, as the
// prefill does; the next chunk's tiles stream into the other LDS buffer (gfx950 direct
// HBM -> LDS loads) while the current chunk is applied.
template <int D, typename T>
__global__ __launch_bounds__(4 * D) void bwd_carry_walk_kernel(BwdArgs a, int P, int cps) {
  using SM = SmemW<D, T>;
  using O = T;
  constexpr int NW = D / 16, NA = D / 16, PQ = SM::PQ;
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15, cw = 16 * w;
  const int NC = a.nchunks;
  const int chain = blockIdx.x / P, seg = blockIdx.x % P;
  const int c0 = seg * cps, c1 = min(NC, c0 + cps);
  const size_t DD = (size_t)D * D;
  const BwdLayout<T> L = layout<T>(a);
  const float *S_in = nullptr, *C_in = nullptr, *m_in = nullptr;
  if (P > 1 && seg > 0) {  // the prefill's scan left the carry-in of segments 1.. in their slots
    const float* slot = L.sum + ((size_t)chain * P + seg) * (2 * DD + 2 * D);
    S_in = slot;
    C_in = slot + DD;
    m_in = slot + 2 * DD;
  } else if (a.S0 != nullptr) {
    S_in = a.S0 + (size_t)chain * DD;
    C_in = a.C0 + (size_t)chain * DD;
    m_in = a.ksum0 + (size_t)chain * D;
  }
  // Sacc[t][r] = S[cw + l16][16 t + 4 g + r] (= S^T tile), Cacc[t][r] = C[16 t + 4 g + r][cw + l16]
  f32x4 Sacc[NA], Cacc[NA];
  float mv = 0.f;  // m[cw + l16]
#pragma unroll
  for (int t = 0; t < NA; ++t) {
    Sacc[t] = S_in ? *reinterpret_cast<const f32x4*>(S_in + (size_t)(cw + l16) * D + 16 * t + 4 * g) : zero4();
    Cacc[t] = C_in ? *reinterpret_cast<const f32x4*>(C_in + (size_t)(cw + l16) * D + 16 * t + 4 * g) : zero4();
  }
  if (m_in) mv = m_in[cw + l16];
  // chunks whose update is needed: all but the segment's last (the carry after it is the next
  // segment's carry-in, or unused after the chain's last chunk)
  const int cu = c1 - 1;
  const T* kg_ = static_cast<const T*>(a.k);
  const T* vg_ = static_cast<const T*>(a.v);
  const T* gg_ = static_cast<const T*>(a.log_alpha);
  auto issue = [&](int c, int b) {
    const size_t row0 = (size_t)chain * a.T + (size_t)c * kL;
    dma_tile<D, T, PQ>(sm.K[b], kg_ + row0 * D, kL, w, NW, lane);
    dma_tile<D, T, PQ>(sm.V[b], vg_ + row0 * D, kL, w, NW, lane);
    dma_tile<D, T, PQ>(sm.G[b], gg_ + row0 * D, kL, w, NW, lane);
  };
  if (c0 < cu) issue(c0, 0);
  for (int c = c0; c < c1; ++c) {
    const size_t cs = (size_t)chain * NC + c;
    T* Sd = L.car + cs * 2 * DD;
    T* Cd = Sd + DD;
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      st4t<T>(Sd + (size_t)(cw + l16) * D + 16 * t + 4 * g, Sacc[t]);
      st4t<T>(Cd + (size_t)(cw + l16) * D + 16 * t + 4 * g, Cacc[t]);  // C symmetric: row cw + l16
    }
    if (g == 0) L.carm[cs * D + cw + l16] = mv;
    if (c >= cu) break;
    const int b = (c - c0) & 1;
    vm_wait_all();
    lds_barrier();  // chunk c's tiles have landed; the other buffer is free
    if (c + 1 < cu) issue(c + 1, b ^ 1);
    f32x4 ks[4], bs[4];
    {
      f32x4 gs[4];
      read_strip(&sm.K[b][0][0], PQ, cw, lane, ks);
      read_strip(&sm.G[b][0][0], PQ, cw, lane, gs);
      strip_cumsum<O, true>(gs, bs, lane);
    }
    mv += token_sum(ks);
    {
      f32x4 kp[4];
#pragma unroll
      for (int ti = 0; ti < 4; ++ti)
#pragma unroll
        for (int r = 0; r < 4; ++r) kp[ti][r] = ks[ti][r] * __expf(-bs[ti][r]);
      write_strip(&sm.G[b][0][0], PQ, cw, lane, kp);  // own channels only: no other wave reads them before the barrier
    }
    const float eBLv = __expf(__shfl(bs[3][3], 48 + l16, 64));  // token 63
    if (g == 0) sm.eBL[cw + l16] = eBLv;
    lds_barrier();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const Frag<O> Bk = tile_cols<O, KORD_CONTIG>(&sm.K[b][0][0], PQ, 32 * kk, cw, lane);
      const Frag<O> Bv = tile_cols<O, KORD_CONTIG>(&sm.V[b][0][0], PQ, 32 * kk, cw, lane);
#pragma unroll
      for (int t = 0; t < NA; ++t) {
        mma(Cacc[t], tile_cols<O, KORD_CONTIG>(&sm.K[b][0][0], PQ, 32 * kk, 16 * t, lane), Bk);
        mma(Sacc[t], tile_cols<O, KORD_CONTIG>(&sm.G[b][0][0], PQ, 32 * kk, 16 * t, lane), Bv);
      }
    }
#pragma unroll
    for (int t = 0; t < NA; ++t) Sacc[t] *= *reinterpret_cast<const f32x4*>(&sm.eBL[16 * t + 4 * g]);
    lds_barrier();  // eBL and the k e^-B columns are read before the next chunk rewrites them
  }
}

// Reverse scan over the chunks of a chain, in place: chunk c receives dS_end(c), G(c), dm_after(c)
// (the adjoints carried back from the chunks after c and the caller's carry-out adjoint);
// dS_end(c-1) = dS_end(c) diag(e^{B_L(c)}) + R_c, G and dm_after by plain sums.  What is left after
// chunk 0 is the carry-in adjoint.  dw and db are summed over chunks.  Running sums in fp32.
// Blocks 0 .. nmb-1 take the adjoint matrices dS | G (input dtype), one 16-byte vector per thread;
// the last block the fp32 tails dm | dw | db, 4 floats per thread.  Which part a thread scans is
// uniform over its block.
template <int D, typename T>
__global__ __launch_bounds__(256) void bwd_scan_kernel(BwdArgs a) {
  constexpr int EPV = 16 / (int)sizeof(T);          // matrix elements per thread
  constexpr int NMV = 2 * D * D / EPV;              // matrix vectors per chunk
  constexpr int NMB = (NMV + 255) / 256;            // matrix blocks
  const int chain = blockIdx.y;
  const int NC = a.nchunks;
  const BwdLayout<T> L = layout<T>(a);
  const size_t DD = (size_t)D * D;
  if ((int)blockIdx.x < NMB) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= NMV) return;
    const size_t f = (size_t)idx * EPV;
    float run[EPV];
    T* x0 = L.mat + (size_t)chain * NC * 2 * DD + f;
    if (f < DD) {  // dS: decayed by the chunk's e^{B_L} per key channel (the matrix column)
      const float* src = a.dS_T ? a.dS_T + (size_t)chain * DD + f : nullptr;
#pragma unroll
      for (int e = 0; e < EPV; ++e) run[e] = src ? src[e] : 0.f;
      rev_scan_vec<T, true>(x0, 2 * DD, NC, L.tail + (size_t)chain * NC * 4 * D + 3 * D + f % D, 4 * (size_t)D, run);
      if (a.dS0) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) a.dS0[(size_t)chain * DD + f + e] = run[e];
      }
    } else {       // G: plain sums
      const size_t o = f - DD;
      const float* src = a.dC_T ? a.dC_T + (size_t)chain * DD + o : nullptr;
#pragma unroll
      for (int e = 0; e < EPV; ++e) run[e] = src ? src[e] : 0.f;
      rev_scan_vec<T, false>(x0, 2 * DD, NC, nullptr, 0, run);
      if (a.dC0) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) a.dC0[(size_t)chain * DD + o + e] = run[e];
      }
    }
    return;
  }
  // tails dm | dw | db: dm scanned (what is left is dksum0), dw and db only summed
  const int idx = threadIdx.x;
  if (idx >= 3 * D / 4) return;
  const size_t o = (size_t)idx * 4;
  const int part = (int)(o / D);  // 0 dm, 1 dw, 2 db
  float run[4];
  const float* src = (part == 0 && a.dksum_T) ? a.dksum_T + (size_t)chain * D + o : nullptr;
#pragma unroll
  for (int e = 0; e < 4; ++e) run[e] = src ? src[e] : 0.f;
  float* x0 = L.tail + (size_t)chain * NC * 4 * D + o;
  if (part == 0) {
    rev_scan_vec<float, false>(x0, 4 * (size_t)D, NC, nullptr, 0, run);
    if (a.dksum0) *reinterpret_cast<f32x4*>(a.dksum0 + (size_t)chain * D + o) = f32x4{run[0], run[1], run[2], run[3]};
  } else {  // only summed: the per-chunk values stay (pass B does not read them)
    for (int c = 0; c < NC; ++c) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(x0 + (size_t)c * 4 * D);
#pragma unroll
      for (int e = 0; e < 4; ++e) run[e] += v[e];
    }
    if (part == 1) *reinterpret_cast<f32x4*>(a.dw + (size_t)chain * D + (o - D)) = f32x4{run[0], run[1], run[2], run[3]};
    if (part == 2 && o == 2 * (size_t)D) a.db[chain] = run[0];
  }
}

namespace {
template <int D, typename T>
struct SmemB {
  static constexpr int PQ = Cfg<D, T>::PQ, PTO = kL + 16 / (int)sizeof(T), NW = D / 16;
  union {
    struct {
      T K[kL][PQ];
      T G[kL][PQ];
    } in;
    T Kh[kL][PQ];  // k e^-B, once the key and log-decay strips are read
  } u1;
  T V[kL][PQ];
  T dO[kL][PQ];
  union {
    T Gm[D][PQ];   // the carried-back statistics adjoint G (read only before the tiles below are formed)
    struct {
      T Qh[kL][PQ];  // qc e^B
      T A[kL][PTO];  // tril((qc e^B)(k e^-B)^T)
      T Dm[kL][PTO]; // tril(dO V^T)
    } t;
  } u3;
  T Mst[D][PQ];    // dS_end
  float eBL[D];
  float red[NW][D];  // per-wave column sums of S_c * dS_end
};
}  // namespace

// Pass B.  Every global read of the chunk goes out at the workgroup's start, so the chunk waits for
// memory once: the token tiles, G and dS_end straight from HBM into LDS (direct loads), the three
// fp32 strips of pass A and this thread's 16-byte blocks of S_c (for colsum(S_c * dS_end)) into
// registers.
template <int D, typename T>
__global__ __launch_bounds__(4 * D) void bwd_chunk_b_kernel(BwdArgs a) {
  using SM = SmemB<D, T>;
  using O = T;
  constexpr int NW = D / 16, NT = 64 * NW, PQ = SM::PQ, PTO = SM::PTO;
  constexpr int EPU = 16 / (int)sizeof(T), UR = D / EPU, NP = D * UR / NT;  // S_c blocks: per row, per thread
  static_assert(sizeof(decltype(SM::u3.t)) >= sizeof(decltype(SM::u3.Gm)), "G overlays the formed tiles");
  static_assert(NP * NT == D * UR && NT % UR == 0, "S_c rows split evenly over the workgroup");
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), cw = 16 * w;
  const int NC = a.nchunks;
  const int chain = blockIdx.x / NC, c = blockIdx.x % NC;
  const int t0 = c * kL, Lc = min(kL, a.T - t0);
  const size_t row0 = (size_t)chain * a.T + t0;
  const BwdLayout<T> L = layout<T>(a);
  const size_t slot = (size_t)chain * NC + c;
  const T* Sc = L.car + slot * 2 * D * D;
  const T* dSe = L.mat + slot * 2 * D * D;
  const T* Ga = dSe + (size_t)D * D;
  const size_t sv = (slot * NW + w) * kL * 16;  // this wave's strip in the strip-major buffers

  // ---- every read of the chunk, issued at once
  dma_tile<D, T, PQ>(sm.u1.in.K, static_cast<const T*>(a.k) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.u1.in.G, static_cast<const T*>(a.log_alpha) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.V, static_cast<const T*>(a.v) + row0 * D, Lc, w, NW, lane);
  dma_tile<D, T, PQ>(sm.dO, static_cast<const T*>(a.d_o) + row0 * D, Lc, w, NW, lane);
#pragma unroll
  for (int h = 0; h < D / kL; ++h) {
    dma_tile<D, T, PQ>(&sm.u3.Gm[kL * h], Ga + (size_t)kL * h * D, kL, w, NW, lane);
    dma_tile<D, T, PQ>(&sm.Mst[kL * h], dSe + (size_t)kL * h * D, kL, w, NW, lane);
  }
  f32x4 qc[4], dkp[4], qdq[4];
  load_strip_vec(L.qc + sv, lane, qc);
  load_strip_vec(L.dkp + sv, lane, dkp);
  load_strip_vec(L.qdq + sv, lane, qdq);
  uint4 scb[NP];  // S_c[tid / UR + (NT / UR) p][EPU (tid % UR) ..]
#pragma unroll
  for (int p = 0; p < NP; ++p)
    scb[p] = *reinterpret_cast<const uint4*>(Sc + (size_t)(tid / UR + (NT / UR) * p) * D + EPU * (tid % UR));
  const float dma = L.tail[slot * 4 * D + cw + l16];
  vm_wait_all();
  __syncthreads();
  if (Lc < kL) {  // a ragged last chunk: rows past the end of the sequence read as zeros
    zero_tail<D, T, PQ>(sm.u1.in.K, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.u1.in.G, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.V, Lc, tid, NT);
    zero_tail<D, T, PQ>(sm.dO, Lc, tid, NT);
    __syncthreads();
  }

  f32x4 ks[4], bs[4], dos[4], kg[4];
  {
    f32x4 gs[4];
    read_strip(&sm.u1.in.K[0][0], PQ, cw, lane, ks);
    read_strip(&sm.u1.in.G[0][0], PQ, cw, lane, gs);
    strip_cumsum<O, true>(gs, bs, lane);
  }
  read_strip(&sm.dO[0][0], PQ, cw, lane, dos);
  const float bL = __shfl(bs[3][3], 48 + l16, 64);  // token 63
  const float eBLv = __expf(bL);
  if (g == 0) sm.eBL[cw + l16] = eBLv;
  // K (G + G^T): the statistics part of dk from later tokens
  {
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) kg[ti] = zero4();
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const Frag<O> gc = tile_cols<O, KORD_CONTIG>(&sm.u3.Gm[0][0], PQ, 32 * kk, cw, lane);  // G[c][kappa]
      const Frag<O> gr = tile_rows<O, KORD_CONTIG>(&sm.u3.Gm[0][0], PQ, cw, 32 * kk, lane);  // G[kappa][c]
      Frag<O> b;
#pragma unroll
      for (int e = 0; e < 8; ++e) b.v[e] = cvt<O>(to_f32(gc.v[e]) + to_f32(gr.v[e]));
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) mma(kg[ti], tile_rows<O, KORD_CONTIG>(&sm.u1.in.K[0][0], PQ, 16 * ti, 32 * kk, lane), b);
    }
  }
  // colsum(S_c * dS_end): this thread's blocks, then the lanes and waves that share its columns
  {
    float cs[EPU];
#pragma unroll
    for (int e = 0; e < EPU; ++e) cs[e] = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int row = tid / UR + (NT / UR) * p;
      float sc[EPU], de[EPU];
      unpack16<T>(scb[p], sc);
      unpack16<T>(*reinterpret_cast<const uint4*>(&sm.Mst[row][EPU * (tid % UR)]), de);
#pragma unroll
      for (int e = 0; e < EPU; ++e) cs[e] += sc[e] * de[e];
    }
#pragma unroll
    for (int off = UR; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < EPU; ++e) cs[e] += __shfl_xor(cs[e], off, 64);
    if (lane < UR) {
#pragma unroll
      for (int e = 0; e < EPU; ++e) sm.red[w][EPU * lane + e] = cs[e];
    }
  }
  f32x4 qh[4], ebn[4];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      qh[ti][r] = qc[ti][r] * __expf(bs[ti][r]);
      ebn[ti][r] = __expf(-bs[ti][r]);
    }
  __syncthreads();  // key, log-decay and G tiles fully read
  {
    f32x4 kh[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) kh[ti] = ks[ti] * ebn[ti];
    write_strip(&sm.u1.Kh[0][0], PQ, cw, lane, kh);
    write_strip(&sm.u3.t.Qh[0][0], PQ, cw, lane, qh);
  }
  __syncthreads();
  for (int idx = w; idx < 16; idx += NW) {
    const int ti = idx >> 2, tj = idx & 3;
    const f32x4 x = tril_tile<D, O>(&sm.u3.t.Qh[0][0], PQ, &sm.u1.Kh[0][0], PQ, ti, tj, lane);
    const f32x4 y = tril_tile<D, O>(&sm.dO[0][0], PQ, &sm.V[0][0], PQ, ti, tj, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sm.u3.t.A[16 * ti + 4 * g + r][16 * tj + l16] = (T)x[r];
      sm.u3.t.Dm[16 * ti + 4 * g + r][16 * tj + l16] = (T)y[r];
    }
  }
  __syncthreads();

  // dv = tril(A)^T dO + (k e^-B) (dS_end diag(e^{B_L}))^T
  {
    f32x4 z[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) z[ti] = zero4();
    trilT_times_strip<O>(&sm.u3.t.A[0][0], PTO, dos, lane, z);
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const Frag<O> br = tile_rows<O, KORD_CONTIG>(&sm.Mst[0][0], PQ, cw, 32 * kk, lane);  // dS_end[cw + l][kappa]
      Frag<O> b;
#pragma unroll
      for (int e = 0; e < 8; ++e) b.v[e] = cvt<O>(to_f32(br.v[e]) * sm.eBL[32 * kk + kidx<KORD_CONTIG>(g, e)]);
#pragma unroll
      for (int ti = 0; ti < 4; ++ti) mma(z[ti], tile_rows<O, KORD_CONTIG>(&sm.u1.Kh[0][0], PQ, 16 * ti, 32 * kk, lane), b);
    }
    store_strip_rows<D>(a.dv + row0 * D, Lc, cw, lane, z);
  }
  // write-rule part of dk: e^-B (tril(D)^T (qc e^B)) + e^{B_L - B} (V dS_end)
  f32x4 dkr[4], dks[4];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) dkr[ti] = dks[ti] = zero4();
  trilT_times_strip<O>(&sm.u3.t.Dm[0][0], PTO, qh, lane, dkr);
  strip_times_tile<D, O>(&sm.V[0][0], PQ, &sm.Mst[0][0], PQ, cw, lane, dks);
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
    dks[ti] = dks[ti] * ebn[ti] * eBLv;
    dkr[ti] = dkr[ti] * ebn[ti] + dks[ti];
  }
  {
    f32x4 dk[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) dk[ti] = dkr[ti] + kg[ti] + dkp[ti] + dma;
    store_strip_rows<D>(a.dk + row0 * D, Lc, cw, lane, dk);
  }
  // dlog alpha = revcumsum(qc dqc - k dk_rule) + e^{B_L} colsum(S_c dS_end) + sum_j k_j dk_state_j
  {
    f32x4 out[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      qdq[ti] -= ks[ti] * dkr[ti];
      out[ti] = zero4();
      dks[ti] *= ks[ti];
    }
    strip_revcumsum_add<O, false>(qdq, out, lane);
    float cs = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) cs += sm.red[v][cw + l16];
    const float after = eBLv * cs + token_sum(dks);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) out[ti] += after;
    store_strip_rows<D>(a.dlog_alpha + row0 * D, Lc, cw, lane, out);
  }
}

size_t bwd_workspace_bytes(int B, int H, int T, int d, int dtype) {
  const size_t chains = (size_t)B * H, NC = (size_t)((T + kL - 1) / kL);
  return bwd_layout_bytes(chains, NC, (size_t)d, dtype == 1 ? 2 : 4).total;
}

static hipError_t record_bwd_event(const BwdArgs& a, int i, hipStream_t s) {
  if (a.events == nullptr) return hipSuccess;
  return hipEventRecord(static_cast<hipEvent_t>(a.events[i]), s);
}

template <int D, typename T>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const int chains = a.B * a.H, NC = a.nchunks;
  // 1. carries at every chunk start: the prefill's summary and scan, one chunk per segment
  FwdArgs f{};
  f.rule = 0;
  f.dtype = a.dtype;
  f.B = a.B;
  f.H = a.H;
  f.T = a.T;
  f.d = D;
  f.k = a.k;
  f.v = a.v;
  f.log_alpha = a.log_alpha;
  f.S0 = a.S0;
  f.C0 = a.C0;
  f.ksum0 = a.ksum0;
  f.n0 = a.n0;
  f.workspace = a.workspace;  // the segment summaries come first in the workspace
  f.flags = 0;
  // segments: about one (chain, segment) workgroup per compute unit, as the prefill chooses
  int P = (256 + chains - 1) / chains;
  if (P > NC) P = NC;
  if (P < 1) P = 1;
  const int cps = (NC + P - 1) / P;
  P = (NC + cps - 1) / cps;
  f.segments = P;
  f.chunks_per_segment = cps;
  if (record_bwd_event(a, 0, s) != hipSuccess) return hipErrorLaunchFailure;
  hipError_t e = hipSuccess;
  if (a.chunk_carry == nullptr) {  // else the forward wrote them and layout() points at its buffer
    e = P > 1 ? launch_gla_segment_carries(f, s) : hipSuccess;
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_carry_walk_kernel<D, T>), dim3((unsigned)(chains * P)), dim3(4 * D), 0, s, a, P, cps);
  }
  if (record_bwd_event(a, 1, s) != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL((bwd_chunk_a_kernel<D, T>), dim3((unsigned)(chains * NC)), dim3(4 * D), 0, s, a);
  if (record_bwd_event(a, 2, s) != hipSuccess) return hipErrorLaunchFailure;
  const int nmb = (2 * D * D / (16 / (int)sizeof(T)) + 255) / 256;  // matrix blocks, then one tail block
  hipLaunchKernelGGL((bwd_scan_kernel<D, T>), dim3((unsigned)(nmb + 1), (unsigned)chains), dim3(256), 0, s, a);
  if (record_bwd_event(a, 3, s) != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL((bwd_chunk_b_kernel<D, T>), dim3((unsigned)(chains * NC)), dim3(4 * D), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return record_bwd_event(a, 4, s);
}

hipError_t launch_bwd(const BwdArgs& a, hipStream_t s) {
  if (a.rule == 1) return launch_gdn_bwd(a, s);
  if (a.dtype == 1) {
    if (a.d == 128) return launch_bwd_t<128, __bf16>(a, s);
    if (a.d == 64) return launch_bwd_t<64, __bf16>(a, s);
  } else if (a.d == 64) {
    return launch_bwd_t<64, float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ccq
