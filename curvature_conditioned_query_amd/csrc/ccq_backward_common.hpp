// Building blocks of the chunked backward kernels (gfx950), shared by the GLA and Gated DeltaNet
// backward passes: operand fragments of LDS / global tiles in either K order, "strips" (a wave's
// [64 tokens] x [16 channels] block in MFMA accumulator layout: element r of lane (g, l) of tile ti
// is token 16 ti + 4 g + r, channel cw + l), cumulative sums over tokens as MFMAs against 0/1
// fragments, masked token-token products, and the channel reductions of a strip.
#pragma once

#include <type_traits>

#include "ccq_prefill_common.hpp"

namespace ccq {
namespace bk {

// MFMA operand type O: the input dtype (bf16 operands for bf16 inputs, fp32 for fp32 inputs);
// the cumulative sums over tokens are exact for bf16 inputs and split hi + lo for computed values.

template <int KO>
__device__ __forceinline__ int kidx(int g, int e) {
  if constexpr (KO == KORD_CONTIG) {
    return 8 * g + e;
  } else {
    return 16 * (e >> 2) + 4 * g + (e & 3);
  }
}

// Lane (g, l) receives X[row0 + l][k0 + kidx(g, e)]: as an A operand, rows of X; as a B
// operand, X^T.  X row-major with the given pitch (LDS or global, any storage type).
template <typename O, int KO, typename TS>
__device__ __forceinline__ Frag<O> frag_rows(const TS* X, int pitch, int row0, int k0, int lane) {
  Frag<O> f;
  const int g = lane >> 4;
  const TS* p = X + (size_t)(row0 + (lane & 15)) * pitch + k0;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = cvt<O>(to_f32(p[kidx<KO>(g, e)]));
  return f;
}

// Lane (g, l) receives X[k0 + kidx(g, e)][n0 + l]: as a B operand, X itself; as an A operand,
// X^T.
template <typename O, int KO, typename TS>
__device__ __forceinline__ Frag<O> frag_cols(const TS* X, int pitch, int k0, int n0, int lane) {
  Frag<O> f;
  const int g = lane >> 4;
  const TS* p = X + (size_t)k0 * pitch + n0 + (lane & 15);
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = cvt<O>(to_f32(p[(size_t)kidx<KO>(g, e) * pitch]));
  return f;
}

// Upper-triangular ones U[t][t'] = (t' >= t), t = 16 ti + (lane % 16), t' over K-step kk in
// KORD_ACC order: as an A operand against a strip it forms reverse cumulative sums over tokens.
template <typename O>
__device__ __forceinline__ Frag<O> utri_frag(int ti, int kk, int lane) {
  Frag<O> f;
  const int t = 16 * ti + (lane & 15), g = lane >> 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = cvt<O>((32 * kk + kidx<KORD_ACC>(g, e) >= t) ? 1.f : 0.f);
  return f;
}

// B operands of a strip's two K-steps of 32 tokens.  EXACT: the strip's values are exactly
// representable in O (bf16 inputs read from a tile); otherwise, for bf16 operands, a second
// pair holds the low parts x - bf16(x), so a sum against 0/1 weights keeps ~16 more bits.
template <typename O, bool EXACT>
struct StripOps {
  Frag<O> hi0, hi1, lo0, lo1;
  __device__ __forceinline__ explicit StripOps(const f32x4 (&x)[4]) {
    hi0 = acc_frag<O>(x[0], x[1]);
    hi1 = acc_frag<O>(x[2], x[3]);
    if constexpr (!EXACT && sizeof(O) == 2) {
      f32x4 r[4];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) r[t][e] = x[t][e] - (float)(O)x[t][e];
      lo0 = acc_frag<O>(r[0], r[1]);
      lo1 = acc_frag<O>(r[2], r[3]);
    }
  }
  __device__ __forceinline__ void mma_k(f32x4& acc, const Frag<O>& a, int kk) const {
    mma(acc, a, kk == 0 ? hi0 : hi1);
    if constexpr (!EXACT && sizeof(O) == 2) mma(acc, a, kk == 0 ? lo0 : lo1);
  }
};

// out[ti] = sum_{j <= i} x_j (inclusive cumulative sum over the tokens of a strip).
template <typename O, bool EXACT>
__device__ __forceinline__ void strip_cumsum(const f32x4 (&x)[4], f32x4 (&out)[4], int lane) {
  const StripOps<O, EXACT> b(x);
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
    out[ti] = zero4();
    b.mma_k(out[ti], ltri_frag<O>(ti, 0, lane), 0);
    if (ti >= 2) b.mma_k(out[ti], ltri_frag<O>(ti, 1, lane), 1);
  }
}

// out[ti] += sum_{j >= i} x_j (reverse cumulative sum over the tokens of a strip).
template <typename O, bool EXACT>
__device__ __forceinline__ void strip_revcumsum_add(const f32x4 (&x)[4], f32x4 (&out)[4], int lane) {
  const StripOps<O, EXACT> b(x);
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
    if (ti < 2) b.mma_k(out[ti], utri_frag<O>(ti, 0, lane), 0);
    b.mma_k(out[ti], utri_frag<O>(ti, 1, lane), 1);
  }
}

// Strip of a row-major LDS tile: token 16 ti + 4 g + r, channel cw + l.
template <typename TS>
__device__ __forceinline__ void read_strip(const TS* X, int pitch, int cw, int lane, f32x4 (&out)[4]) {
  const int g = lane >> 4, l = lane & 15;
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int r = 0; r < 4; ++r) out[ti][r] = to_f32(X[(16 * ti + 4 * g + r) * pitch + cw + l]);
}

template <typename TS>
__device__ __forceinline__ void write_strip(TS* X, int pitch, int cw, int lane, const f32x4 (&v)[4]) {
  const int g = lane >> 4, l = lane & 15;
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int r = 0; r < 4; ++r) X[(16 * ti + 4 * g + r) * pitch + cw + l] = (TS)v[ti][r];
}

// Strip rows 0 .. rows-1 to a global [token][D] array (row 0 at p).
template <int D>
__device__ __forceinline__ void store_strip_rows(float* p, int rows, int cw, int lane, const f32x4 (&v)[4]) {
  const int g = lane >> 4, l = lane & 15;
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * g + r;
      if (i < rows) p[(size_t)i * D + cw + l] = v[ti][r];
    }
}

// A strip in the workspace's strip-major order: the 16 values of a lane are contiguous (lane
// order within the wave, waves in order within the chunk), so each lane moves 4 x 16 bytes.
__device__ __forceinline__ void store_strip_vec(float* p, int lane, const f32x4 (&v)[4]) {
  f32x4* q = reinterpret_cast<f32x4*>(p + (size_t)lane * 16);
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) q[ti] = v[ti];
}
__device__ __forceinline__ void load_strip_vec(const float* p, int lane, f32x4 (&v)[4]) {
  const f32x4* q = reinterpret_cast<const f32x4*>(p + (size_t)lane * 16);
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) v[ti] = q[ti];
}

// Rows 0 .. Lc-1 of a [ROWS][D] block (row stride D) into an LDS tile of pitch PQ, 16 bytes per
// thread and step; rows Lc .. ROWS-1 are zeroed.
template <int D, int ROWS, typename T, int PQ>
__device__ __forceinline__ void load_rows(T (*dst)[PQ], const T* src, int Lc, int tid, int nthreads) {
  constexpr int EPU = 16 / (int)sizeof(T), U = D / EPU;
  for (int u = tid; u < ROWS * U; u += nthreads) {
    const int row = u / U, col = (u % U) * EPU;
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (row < Lc) x = *reinterpret_cast<const uint4*>(src + (size_t)row * D + col);
    *reinterpret_cast<uint4*>(&dst[row][col]) = x;
  }
}

// Rows 0 .. Lc-1 of a chunk of a [token][D] tensor (64-row tile).
template <int D, typename T, int PQ>
__device__ __forceinline__ void load_tile(T (*dst)[PQ], const T* src, int Lc, int tid, int nthreads) {
  load_rows<D, kL, T, PQ>(dst, src, Lc, tid, nthreads);
}

// Fragments of LDS tiles: wide reads when the tile already holds operands of type O (16- or
// 8-byte row reads; gfx950 transposing reads for the column forms of bf16 tiles), otherwise
// element reads converted to O.
template <typename O, int KO, typename TS>
__device__ __forceinline__ Frag<O> tile_rows(const TS* X, int pitch, int row0, int k0, int lane) {
  if constexpr (std::is_same<TS, O>::value) {
    return lds_frag<O, KO>(X, pitch, row0, k0, lane);
  } else {
    return frag_rows<O, KO>(X, pitch, row0, k0, lane);
  }
}
template <typename O, int KO, typename TS>
__device__ __forceinline__ Frag<O> tile_cols(const TS* X, int pitch, int k0, int n0, int lane) {
  if constexpr (std::is_same<TS, O>::value && sizeof(O) == 2) {
    if constexpr (KO == KORD_CONTIG) {
      return tr_frag<O>(X, pitch, k0, n0, lane);
    } else {
      return tr_frag_acc<O>(X, pitch, k0, n0, lane);
    }
  } else {
    return frag_cols<O, KO>(X, pitch, k0, n0, lane);
  }
}

// Tile (ti, tj) of tril_incl(X Y^T) for row-major tiles X, Y (contraction over D channels):
// acc[r] = sum_c X[16 ti + 4 g + r][c] Y[16 tj + l][c], zero where column > row.
template <int D, typename O, typename TX, typename TY>
__device__ __forceinline__ f32x4 tril_tile(const TX* X, int px, const TY* Y, int py, int ti, int tj, int lane) {
  f32x4 acc = zero4();
  if (tj > ti) return acc;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
    mma(acc, tile_rows<O, KORD_CONTIG>(X, px, 16 * ti, 32 * kk, lane), tile_rows<O, KORD_CONTIG>(Y, py, 16 * tj, 32 * kk, lane));
  const int g = lane >> 4, l = lane & 15;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (16 * tj + l > 16 * ti + 4 * g + r) acc[r] = 0.f;
  return acc;
}

// strip[ti] += X (rows 16 ti.., all D channels of a row-major LDS tile) times the D x 16 block
// M[:, cw .. cw + 15] of a global matrix (M[a][cw + n], K running over a).
template <int D, typename O, typename TX, typename TM>
__device__ __forceinline__ void strip_times_mat(const TX* X, int px, const TM* M, int cw, int lane, f32x4 (&out)[4]) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const Frag<O> b = frag_cols<O, KORD_CONTIG>(M, D, 32 * kk, cw, lane);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) mma(out[ti], tile_rows<O, KORD_CONTIG>(X, px, 16 * ti, 32 * kk, lane), b);
  }
}

// As strip_times_mat for a symmetric global matrix M: the block is read as rows
// M[cw + n][a] (contiguous, 16 bytes per lane and K-step for bf16).
template <int D, typename O, typename TX, typename TM>
__device__ __forceinline__ void strip_times_sym(const TX* X, int px, const TM* M, int cw, int lane, f32x4 (&out)[4]) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const Frag<O> b = frag_rows<O, KORD_CONTIG>(M, D, cw, 32 * kk, lane);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) mma(out[ti], tile_rows<O, KORD_CONTIG>(X, px, 16 * ti, 32 * kk, lane), b);
  }
}

// The B-operand fragments strip_times_sym takes from a symmetric D x D matrix in global memory (rows
// cw .. cw + 15: lane (g, l) gets row cw + l, columns 32 kk + 8 g .. + 7), loaded once, with one
// 16-byte load per fragment for bf16 (two for fp32), so that several products can share them and the
// loads can go out long before the first product.
template <int D, typename O>
__device__ __forceinline__ void sym_frags(const O* M, int cw, int lane, Frag<O> (&f)[D / 32]) {
  const O* p = M + (size_t)(cw + (lane & 15)) * D + 8 * (lane >> 4);
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    if constexpr (sizeof(O) == 2) {
      f[kk].v = *reinterpret_cast<const bf16x8*>(p + 32 * kk);
    } else {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p + 32 * kk);
      const f32x4 b = *reinterpret_cast<const f32x4*>(p + 32 * kk + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[kk].v[e] = a[e];
        f[kk].v[4 + e] = b[e];
      }
    }
  }
}

// out += X C for the statistic carry C: from global memory (strip_times_sym), or from the wave's
// fragments of it already in registers (sym_frags).
template <int D, typename O, typename TX>
__device__ __forceinline__ void strip_times_carry(const TX* X, int px, const O* C, int cw, int lane, f32x4 (&out)[4]) {
  strip_times_sym<D, O>(X, px, C, cw, lane, out);
}
template <int D, typename O, typename TX>
__device__ __forceinline__ void strip_times_carry(const TX* X, int px, const Frag<O> (&f)[D / 32], int cw, int lane,
                                                  f32x4 (&out)[4]) {
  (void)cw;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk)
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) mma(out[ti], tile_rows<O, KORD_CONTIG>(X, px, 16 * ti, 32 * kk, lane), f[kk]);
}

// As strip_times_sym for a D x D matrix staged in LDS (pitch pm): out += X M[cw .. cw + 15][:]^T, the
// B operand read as rows of M.
template <int D, typename O, typename TX, typename TM>
__device__ __forceinline__ void strip_times_tile_rows(const TX* X, int px, const TM* M, int pm, int cw, int lane,
                                                      f32x4 (&out)[4]) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const Frag<O> b = tile_rows<O, KORD_CONTIG>(M, pm, cw, 32 * kk, lane);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) mma(out[ti], tile_rows<O, KORD_CONTIG>(X, px, 16 * ti, 32 * kk, lane), b);
  }
}

// As strip_times_mat for a D x D matrix staged in LDS (pitch pm).
template <int D, typename O, typename TX, typename TM>
__device__ __forceinline__ void strip_times_tile(const TX* X, int px, const TM* M, int pm, int cw, int lane,
                                                 f32x4 (&out)[4]) {
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const Frag<O> b = tile_cols<O, KORD_CONTIG>(M, pm, 32 * kk, cw, lane);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) mma(out[ti], tile_rows<O, KORD_CONTIG>(X, px, 16 * ti, 32 * kk, lane), b);
  }
}

// strip[ti] += tril(Mt) x, Mt a 64 x 64 LDS tile (lower-triangular incl., pitch pt), x a strip.
template <typename O, typename TS>
__device__ __forceinline__ void tril_times_strip(const TS* Mt, int pt, const f32x4 (&x)[4], int lane, f32x4 (&out)[4]) {
  const Frag<O> b0 = acc_frag<O>(x[0], x[1]), b1 = acc_frag<O>(x[2], x[3]);
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) {
    mma(out[ti], tile_rows<O, KORD_ACC>(Mt, pt, 16 * ti, 0, lane), b0);
    if (ti >= 2) mma(out[ti], tile_rows<O, KORD_ACC>(Mt, pt, 16 * ti, 32, lane), b1);
  }
}

// strip[tj] += tril(Mt)^T x.
template <typename O, typename TS>
__device__ __forceinline__ void trilT_times_strip(const TS* Mt, int pt, const f32x4 (&x)[4], int lane, f32x4 (&out)[4]) {
  const Frag<O> b0 = acc_frag<O>(x[0], x[1]), b1 = acc_frag<O>(x[2], x[3]);
#pragma unroll
  for (int tj = 0; tj < 4; ++tj) {
    if (tj < 2) mma(out[tj], tile_cols<O, KORD_ACC>(Mt, pt, 0, 16 * tj, lane), b0);
    mma(out[tj], tile_cols<O, KORD_ACC>(Mt, pt, 32, 16 * tj, lane), b1);
  }
}

// Rows [16 ta, 16 ta + 16) x strip columns of X^T y (contraction over the 64 tokens): X a
// row-major LDS tile (token rows), y a strip.  acc[r] = out[16 ta + 4 g + r][cw + l].
template <typename O, typename TX>
__device__ __forceinline__ f32x4 tileT_times_strip(const TX* X, int px, int ta, const f32x4 (&y)[4], int lane) {
  f32x4 acc = zero4();
  mma(acc, tile_cols<O, KORD_ACC>(X, px, 0, 16 * ta, lane), acc_frag<O>(y[0], y[1]));
  mma(acc, tile_cols<O, KORD_ACC>(X, px, 32, 16 * ta, lane), acc_frag<O>(y[2], y[3]));
  return acc;
}

// One DPP exchange within rows of 16 lanes: the value of the lane the pattern pairs with.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Reduce-scatter over the 16 channels of a lane group: v[4 ti + r] is this lane's value for
// token 16 ti + 4 g + r; lane l of the group returns the group's total for index l (token
// 16 (l / 4) + 4 g + l % 4).  Four butterfly steps pair lane l with 15 - l (row mirror),
// l ^ 7 within eight (half mirror), l ^ 3 and l ^ 1 within four (quad permutations); at each
// step a lane keeps the half of its values its partner sends the other half of, so it moves
// 8 + 4 + 2 + 1 values instead of 16 x 4.
__device__ __forceinline__ float chan_reduce16(const float (&v)[16], int l) {
  float a[8], b[4], c[2];
  const bool up8 = (l & 8) != 0, up4 = (l & 4) != 0, up2 = (l & 2) != 0, up1 = (l & 1) != 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = (up8 ? v[8 + j] : v[j]) + dpp<0x140>(up8 ? v[j] : v[8 + j]);
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = (up4 ? a[4 + j] : a[j]) + dpp<0x141>(up4 ? a[j] : a[4 + j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) c[j] = (up2 ? b[2 + j] : b[j]) + dpp<0x1B>(up2 ? b[j] : b[2 + j]);
  return (up1 ? c[1] : c[0]) + dpp<0xB1>(up1 ? c[0] : c[1]);
}

// Sum over the 64 tokens of a strip for the lane's channel (every lane gets it).
__device__ __forceinline__ float token_sum(const f32x4 (&x)[4]) {
  float s = 0.f;
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) s += x[ti][0] + x[ti][1] + x[ti][2] + x[ti][3];
  s += __shfl_xor(s, 16, 64);
  s += __shfl_xor(s, 32, 64);
  return s;
}

constexpr int PT = kL + 4;  // pitch of the fp32 64 x 64 token tiles

template <int D>
constexpr int pf() { return D + 4; }  // pitch of fp32 [64][D] tiles

// ---------------------------------------------------------------- the read, recomputed and adjoint
// (rule-independent: the statistics never see the write rule)
//
// Per token (sums C_i, m_i and count n_i include token i; carry C_c, m_c, n_c at the chunk start):
//   u_i = C_i q_i / n_i - m_i sq_i / n_i^2,  sq_i = m_i . q_i,  lambda_i = sigmoid(w . q_i + b),
//   qc_i = q_i - lambda_i u_i.
// With dqc_i the gradient of the loss with respect to qc_i:
//   dlogit_i = -(u_i . dqc_i) lambda_i (1 - lambda_i),  dr_i = -lambda_i dqc_i / n_i,
//   ds_i = -(m_i . dr_i) / n_i,  dm_i = ds_i q_i - (sq_i / n_i) dr_i,
//   dq_i = dqc_i + dlogit_i w + C_i dr_i + ds_i m_i,
// and every key j of the chunk gets sum_{i >= j in the chunk} [dr_i (q_i . k_j) + q_i (dr_i . k_j) + dm_i]
// (the later chunks' part is added from their carried-back sums).  In chunk form, with P = tril(Q K^T)
// and M2 = tril(dR K^T): dq = dQc + dlogit w^T + dR C_c + ds * (m_c + cumsum K) + M2 K and
// dk_stats = P^T dR + M2^T Q + revcumsum(dm).

// The read of a chunk recomputed: per-token gate lambda, 1/n_i and sq_i / n_i into tok; the masked Gram
// tile P = tril(Q K^T) (fp32) into Pt; the wave's strips of u and of the cleaned query qc.  Qt, Kt: the
// chunk's q and k row tiles (pitch pq); Cc: the statistic carry C_c at the chunk start, symmetric D x D
// (operand dtype), in global memory or as the wave's fragments of it (sym_frags); wv, mv: w_lambda and m_c at the lane's channel cw + l; nc: tokens
// before the chunk; qs, ks: the wave's strips of q and k.  Every thread of the workgroup calls it.
template <int D, typename O, int NW, typename TQ, typename CS>
__device__ __forceinline__ void read_forward(const TQ* Qt, const TQ* Kt, int pq, float (*Pt)[PT],
                                             float (*red)[kL][2], f32x4* tok, const CS& Cc, float wv, float mv,
                                             float b_lam, int64_t nc, const f32x4 (&qs)[4], const f32x4 (&ks)[4],
                                             int tid, f32x4 (&us)[4], f32x4 (&qc)[4]) {
  constexpr int NT = 64 * NW;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15, cw = 16 * w;
  // per-token w . q and m_c . q: this wave's channels
  const int rtok = 16 * (l16 >> 2) + 4 * g + (l16 & 3);  // the token chan_reduce16 leaves here
  {
    float v0[16], v1[16];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v0[4 * ti + r] = qs[ti][r] * wv;
        v1[4 * ti + r] = qs[ti][r] * mv;
      }
    red[w][rtok][0] = chan_reduce16(v0, l16);
    red[w][rtok][1] = chan_reduce16(v1, l16);
  }
  // P = tril(Q K^T)
  for (int idx = w; idx < 16; idx += NW) {
    const int ti = idx >> 2, tj = idx & 3;
    const f32x4 acc = tril_tile<D, O>(Qt, pq, Kt, pq, ti, tj, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) Pt[16 * ti + 4 * g + r][16 * tj + l16] = acc[r];
  }
  __syncthreads();
  // token scalars: 8 threads per token
  for (int i = tid >> 3; i < kL; i += NT / 8) {
    const int part = tid & 7;
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) rs += Pt[i][8 * part + j];
    rs = group_sum<8>(rs);
    if (part == 0) {
      float logit = b_lam, mq = 0.f;
      for (int v = 0; v < NW; ++v) {
        logit += red[v][i][0];
        mq += red[v][i][1];
      }
      const float sq = mq + rs;
      const float inv_n = 1.0f / (float)(nc + i + 1);
      tok[i] = f32x4{sigmoidf(logit), inv_n, sq * inv_n, 0.f};
    }
  }
  __syncthreads();
  // u = (Q C_c + tril(P) K - (m_c + cumsum K) sq / n) / n,  qc = q - lambda u
#pragma unroll
  for (int ti = 0; ti < 4; ++ti) us[ti] = zero4();
  strip_times_carry<D, O>(Qt, pq, Cc, cw, lane, us);
  tril_times_strip<O>(&Pt[0][0], PT, ks, lane, us);
  f32x4 ck[4];  // cumulative key sum (recomputed where it is needed again: registers are short)
  strip_cumsum<O, true>(ks, ck, lane);
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 ts = tok[16 * ti + 4 * g + r];
      const float u = (us[ti][r] - (mv + ck[ti][r]) * ts[2]) * ts[1];  // m_i = m_c + cumsum k
      us[ti][r] = u;
      qc[ti][r] = qs[ti][r] - ts[0] * u;
    }
}

// The read's adjoint for a chunk, from the wave's strip of dqc: writes dq (final, rows < Lc of the
// chunk's [64][D] fp32 block at dq_rows), this chunk's statistics part of dk (the wave's strip,
// strip-major, at dkp), dG_c = dR^T Q (D x D, operand dtype, at Gs) and the chunk sums of dm, dlogit q
// (per channel, tail[0..D), tail[D..2D)) and dlogit (tail[2D]).  dRt: fp32 [64][PF] LDS tile, written
// after the first barrier here (so it may alias tiles the caller reads before calling); Mt: fp32
// [64][PT] LDS tile for tril(dR K^T).  Every thread of the workgroup calls it.
template <int D, typename O, int NW, int PF, typename TK, typename CS>
__device__ __forceinline__ void read_adjoint(const TK* Kt, int pq, const float (*Pt)[PT], float (*dRt)[PF],
                                             float (*Mt)[PT], float (*red)[kL][2], const f32x4* tok,
                                             float (*tok2)[2], const CS& Cc, float wv, float mv,
                                             const f32x4 (&qs)[4], const f32x4 (&ks)[4], const f32x4 (&us)[4],
                                             const f32x4 (&dqc)[4], int tid, int Lc, float* dq_rows, float* dkp,
                                             O* Gs, float* tail) {
  constexpr int NT = 64 * NW, NA = D / 16;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15, cw = 16 * w;
  const int rtok = 16 * (l16 >> 2) + 4 * g + (l16 & 3);
  // per-token u . dqc and m_c . dqc
  {
    float v0[16], v1[16];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v0[4 * ti + r] = us[ti][r] * dqc[ti][r];
        v1[4 * ti + r] = mv * dqc[ti][r];
      }
    red[w][rtok][0] = chan_reduce16(v0, l16);
    red[w][rtok][1] = chan_reduce16(v1, l16);
  }
  // dR = -lambda dqc / n
  f32x4 dr[4];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const f32x4 ts = tok[16 * ti + 4 * g + r];
      dr[ti][r] = -ts[0] * ts[1] * dqc[ti][r];
    }
  __syncthreads();  // the caller's tiles under dRt are no longer read; red is complete
  write_strip(&dRt[0][0], PF, cw, lane, dr);
  for (int i = tid; i < kL; i += NT) {
    float udq = 0.f, mdq = 0.f;
    for (int v = 0; v < NW; ++v) {
      udq += red[v][i][0];
      mdq += red[v][i][1];
    }
    const f32x4 ts = tok[i];
    tok2[i][0] = -udq * ts[0] * (1.f - ts[0]);  // dlogit
    tok2[i][1] = -ts[0] * ts[1] * mdq;          // m_c . dr
  }
  __syncthreads();
  // M2 = tril(dR K^T)
  for (int idx = w; idx < 16; idx += NW) {
    const int ti = idx >> 2, tj = idx & 3;
    const f32x4 acc = tril_tile<D, O>(&dRt[0][0], PF, Kt, pq, ti, tj, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) Mt[16 * ti + 4 * g + r][16 * tj + l16] = acc[r];
  }
  __syncthreads();
  // ds_i = -(m_c . dr_i + sum_{j<=i} M2_ij) / n_i
  for (int i = tid >> 3; i < kL; i += NT / 8) {
    const int part = tid & 7;
    float rs = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) rs += Mt[i][8 * part + j];
    rs = group_sum<8>(rs);
    if (part == 0) tok2[i][1] = -(tok2[i][1] + rs) * tok[i][1];
  }
  __syncthreads();

  // dq = dqc + dlogit w + dR C_c + ds (m_c + cumsum K) + tril(M2) K
  {
    f32x4 z[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) z[ti] = zero4();
    strip_times_carry<D, O>(&dRt[0][0], PF, Cc, cw, lane, z);
    tril_times_strip<O>(&Mt[0][0], PT, ks, lane, z);
    f32x4 ck2[4];
    strip_cumsum<O, true>(ks, ck2, lane);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * ti + 4 * g + r;
        z[ti][r] += dqc[ti][r] + tok2[i][0] * wv + tok2[i][1] * (mv + ck2[ti][r]);
      }
    store_strip_rows<D>(dq_rows, Lc, cw, lane, z);
  }
  // dm_i = ds_i q_i - (sq_i / n_i) dr_i;  this chunk's statistics part of dk:
  // tril(P)^T dR + tril(M2)^T Q + revcumsum(dm)
  f32x4 dm[4];
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * ti + 4 * g + r;
      dm[ti][r] = tok2[i][1] * qs[ti][r] - tok[i][2] * dr[ti][r];
    }
  {
    f32x4 z[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) z[ti] = zero4();
    trilT_times_strip<O>(&Pt[0][0], PT, dr, lane, z);
    trilT_times_strip<O>(&Mt[0][0], PT, qs, lane, z);
    strip_revcumsum_add<O, false>(dm, z, lane);
    store_strip_vec(dkp, lane, z);
  }
  // dG_c = dR^T Q
#pragma unroll 2
  for (int ta = 0; ta < NA; ++ta) {
    const f32x4 acc = tileT_times_strip<O>(&dRt[0][0], PF, ta, qs, lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) Gs[(size_t)(16 * ta + 4 * g + r) * D + cw + l16] = (O)acc[r];
  }
  // sum dm, sum dlogit q, sum dlogit
  {
    f32x4 dq_w[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int r = 0; r < 4; ++r) dq_w[ti][r] = tok2[16 * ti + 4 * g + r][0] * qs[ti][r];
    const float sdm = token_sum(dm), sdw = token_sum(dq_w);
    if (g == 0) {
      tail[cw + l16] = sdm;
      tail[D + cw + l16] = sdw;
    }
    if (w == 0) {
      const float db = group_sum<64>(tok2[lane][0]);
      if (lane == 0) tail[2 * D] = db;
    }
  }
}

// Four consecutive elements of T as raw bits (8 bytes for bf16, 16 for fp32) and their fp32 values:
// a prefetch kept raw is converted where it is used, so the load need not complete before then.
template <typename T> struct Raw4Of { using type = uint2; };
template <> struct Raw4Of<float> { using type = uint4; };
template <typename T> using raw4_t = typename Raw4Of<T>::type;
template <typename T>
__device__ __forceinline__ raw4_t<T> ld_raw4(const T* p) { return *reinterpret_cast<const raw4_t<T>*>(p); }
template <typename T>
__device__ __forceinline__ f32x4 raw4_f32(const raw4_t<T>& r) {
  if constexpr (sizeof(T) == 2) {
    return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
                 __uint_as_float(r.y & 0xffff0000u)};
  } else {
    return f32x4{__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z), __uint_as_float(r.w)};
  }
}

// ---- reverse scans over the chunks of a chain (the carried-back adjoints)

// The 16 / sizeof(E) elements of a 16-byte vector of type E as fp32, and back (bf16 rounded to nearest
// even).
template <typename E>
__device__ __forceinline__ void unpack16(const uint4& u, float (&f)[16 / sizeof(E)]) {
  const unsigned w[4] = {u.x, u.y, u.z, u.w};
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  }
}
template <typename E>
__device__ __forceinline__ uint4 pack16(const float (&f)[16 / sizeof(E)]) {
  if constexpr (sizeof(E) == 2) {
    const bf16x8 v = {(__bf16)f[0], (__bf16)f[1], (__bf16)f[2], (__bf16)f[3],
                      (__bf16)f[4], (__bf16)f[5], (__bf16)f[6], (__bf16)f[7]};
    return __builtin_bit_cast(uint4, v);
  } else {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
}

// Reverse exclusive scan, over the NC chunks of a chain, of one 16-byte vector of a per-chunk array
// (chunk c's vector at x0 + c * stride): chunk c's vector is replaced by run, the value carried back
// from the chunks after it (on entry: the caller's adjoint of the carry out, or zeros), and then
// run = run * e^{dec(c)} + x(c) with dec(c) the fp32 log decays at dec0 + c * dec_stride (DECAY), or
// run + x(c).  On return run holds what is carried back past chunk 0.  Chunks go in batches of kB
// whose loads are all issued before the first is used (no conditional loads inside a batch, so the
// waits are counted exactly); a shorter first batch (NC not a multiple of kB) goes one chunk at a
// time.  Every branch depends only on NC, so the path is uniform.
template <typename E, bool DECAY>
__device__ __forceinline__ void rev_scan_vec(E* x0, size_t stride, int NC, const float* dec0, size_t dec_stride,
                                             float (&run)[16 / sizeof(E)]) {
  constexpr int N = 16 / (int)sizeof(E), kB = 8;
  auto step = [&](int cc, uint4 xv, const float (&dl)[N]) {  // xv by value: the store below overwrites its source
    *reinterpret_cast<uint4*>(x0 + (size_t)cc * stride) = pack16<E>(run);
    float x[N];
    unpack16<E>(xv, x);
#pragma unroll
    for (int e = 0; e < N; ++e) run[e] = (DECAY ? run[e] * __expf(dl[e]) : run[e]) + x[e];
  };
  auto load_dec = [&](int cc, float (&dl)[N]) {
    if constexpr (DECAY) {
#pragma unroll
      for (int q = 0; q < N / 4; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(dec0 + (size_t)cc * dec_stride + 4 * q);
#pragma unroll
        for (int r = 0; r < 4; ++r) dl[4 * q + r] = v[r];
      }
    } else {
#pragma unroll
      for (int e = 0; e < N; ++e) dl[e] = 0.f;
    }
  };
  int c = NC - 1;
  for (; c >= 0 && (c + 1) % kB != 0; --c) {  // the ragged batch at the end, one chunk at a time
    float dl[N];
    load_dec(c, dl);
    const uint4 xv = *reinterpret_cast<const uint4*>(x0 + (size_t)c * stride);
    step(c, xv, dl);
  }
  for (; c >= 0; c -= kB) {  // c + 1 is a multiple of kB: chunks c, c - 1, .., c - kB + 1
    uint4 xv[kB];
    float dl[kB][N];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      xv[j] = *reinterpret_cast<const uint4*>(x0 + (size_t)(c - j) * stride);
      load_dec(c - j, dl[j]);
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) step(c - j, xv[j], dl[j]);
  }
}

}  // namespace bk
}  // namespace ccq
