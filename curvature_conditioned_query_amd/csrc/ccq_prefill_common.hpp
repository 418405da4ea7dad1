// Helpers and rule-independent phases shared by the chunked-prefill kernels (gfx950).
//
// Tiles of a 64-token chunk sit in LDS row-major ([token][channel]).  The CCQ statistics
// part of a chunk does not depend on the write rule: it is the gate, the causal Gram
// matrix P = Q K^T with its row sums, and the cleaned query (gist.science summary of
// arXiv 2606.01294, §2 "理论推导" and §2 "机制"):
//   s_i  = m0 + sum_{j<=i} k_j,  n_i = n0 + i + 1,  sq_i = s_i . q_i = m0 . q_i + sum_{j<=i} P_ij
//   u_i  = (Q C0 + tril_incl(P - c 1^T) K)_i / n_i - m0 sq_i / n_i^2,  c_i = sq_i / n_i
//        (row i of Q C0 + tril_incl(P) K is C_i q_i, so u_i = Sigma_i q_i)
//   qc_i = q_i - lambda_i u_i,  lambda_i = sigmoid(w . q_i + b)
// Any shared-memory struct with the members used below (Qs, Wt, Pm, tok, m0, Qa) can host
// them; the key tile and the bf16 low part of the cleaned query are passed in.
#pragma once

#include "ccq_device.hpp"
#include "ccq_internal.hpp"

namespace ccq {

constexpr int kL = 64;  // chunk length

template <int D, typename T>
struct Cfg {
  static constexpr int NW = D / 16;          // waves per workgroup (16 channels each)
  static constexpr int NA = D / 16;          // 16-wide tiles along d
  static constexpr int NK = D / 32;          // K-steps of 32 along d
  static constexpr int PQ = D + 16 / sizeof(T);    // pitch of [64][D] row tiles
  static constexpr int PT = kL + 16 / sizeof(T);   // pitch of the [64][64] token tile
  static constexpr int LO = (sizeof(T) == 2) ? kL : 1;  // rows of the bf16 lo tiles
};

template <typename T>
__device__ __forceinline__ void st4(T* p, const f32x4& v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}

// The carry at the start of chunk ch of a chain into the chunk-carry buffer (the chunked backward's
// layout): `row` of S (mat 0) or of the symmetric C (mat 1), from NA accumulator tiles whose element
// r of lane (g, .) is column 16 t + 4 g + r of that row.
template <int D, typename T, int NA>
__device__ __forceinline__ void put_carry_row(const FwdArgs& a, int chain, int ch, int mat, int row, int g,
                                              const f32x4 (&acc)[NA]) {
  const size_t NC = (size_t)((a.T + kL - 1) / kL);
  T* base = static_cast<T*>(a.chunk_carry) + ((size_t)chain * NC + ch) * 2 * D * D + (size_t)mat * D * D +
            (size_t)row * D + 4 * g;
#pragma unroll
  for (int t = 0; t < NA; ++t) st4<T>(base + 16 * t, acc[t]);
}
// m_c (the key sum before chunk ch), channel c.
template <int D, typename T>
__device__ __forceinline__ void put_carry_ksum(const FwdArgs& a, int chain, int ch, int c, float m) {
  const size_t chains = (size_t)a.B * a.H, NC = (size_t)((a.T + kL - 1) / kL);
  float* km = reinterpret_cast<float*>(static_cast<char*>(a.chunk_carry) + chunk_carry_mat_bytes(chains, NC, D, sizeof(T)));
  km[((size_t)chain * NC + ch) * D + c] = m;
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

// Fragment whose K index runs down the rows of a row-major LDS tile X[row][col]: lane
// (g, i = lane % 16) receives X[k0 + 8g + e][n0 + i] for e = 0..7 (KORD_CONTIG).  As a B
// operand that is X[k][n]; as an A operand it is X^T.  For bf16 it is two gfx950
// transposing reads: within each 16-lane group, lane s points at row k0+8g+s/4, column
// n0+4(s%4), and lane i receives element i%4 of lanes i/4, i/4+4, i/4+8, i/4+12.
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
template <typename T>
__device__ __forceinline__ Frag<T> tr_frag(const T* X, int pitch, int k0, int n0, int lane) {
  Frag<T> f;
  const int g = lane >> 4, i = lane & 15;
  if constexpr (sizeof(T) == 2) {
    const T* p = X + (k0 + 8 * g + (i >> 2)) * pitch + n0 + 4 * (i & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 4 * pitch));
    f.v = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    const T* p = X + (k0 + 8 * g) * pitch + n0 + i;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = p[e * pitch];
  }
  return f;
}

// As tr_frag, in KORD_ACC order: lane (g, i) receives X[k0 + 16 (e / 4) + 4 g + e % 4][n0 + i],
// the K order of an operand built from a pair of accumulator tiles (acc_frag).
template <typename T>
__device__ __forceinline__ Frag<T> tr_frag_acc(const T* X, int pitch, int k0, int n0, int lane) {
  Frag<T> f;
  const int g = lane >> 4, i = lane & 15;
  if constexpr (sizeof(T) == 2) {
    const T* p = X + (k0 + 4 * g + (i >> 2)) * pitch + n0 + 4 * (i & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 16 * pitch));
    f.v = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    const T* p = X + (k0 + 4 * g) * pitch + n0 + i;
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = p[(16 * (e >> 2) + (e & 3)) * pitch];
  }
  return f;
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
  if constexpr (sizeof(T) == 2) {
    // at most one element is one: e = l + 16h - 8g, in dword e / 2, half e % 2 (bf16 1.0 = 0x3F80)
    const int e = l + 16 * h - 8 * g;
    const unsigned one = (e & 1) ? 0x3F800000u : 0x3F80u;
    const int j = e >> 1;
    const u32x4 x{j == 0 ? one : 0u, j == 1 ? one : 0u, j == 2 ? one : 0u, j == 3 ? one : 0u};
    f.v = __builtin_bit_cast(bf16x8, x);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = cvt<T>((8 * g + e == l + 16 * h) ? 1.0f : 0.0f);
  }
  return f;
}

// Lower-triangular ones L[t][t'] = (t' <= t), t = 16 ti + (lane % 16), over
// t' = 32 kk + 16 (e / 4) + 4 g + e % 4 (KORD_ACC).
template <typename T>
__device__ __forceinline__ Frag<T> ltri_frag(int ti, int kk, int lane) {
  Frag<T> f;
  const int t = 16 * ti + (lane & 15), g = lane >> 4;
  if constexpr (sizeof(T) == 2) {
    // element 4 hf + r is one where r <= d = t - 32 kk - 16 hf - 4 g: two bf16 ones per dword
    u32x4 x;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int d = t - 32 * kk - 16 * hf - 4 * g;
      x[2 * hf] = d >= 1 ? 0x3F803F80u : (d >= 0 ? 0x3F80u : 0u);
      x[2 * hf + 1] = d >= 3 ? 0x3F803F80u : (d >= 2 ? 0x3F80u : 0u);
    }
    f.v = __builtin_bit_cast(bf16x8, x);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tp = 32 * kk + 16 * (e >> 2) + 4 * g + (e & 3);
      f.v[e] = cvt<T>(tp <= t ? 1.0f : 0.0f);
    }
  }
  return f;
}

__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4& v) {
  return bf16x4{(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}

// Lower-triangular 16x16 tiles of a 64x64 token-token matrix, numbered row by row:
// idx -> (row tile, col tile) = (0,0) (1,0) (1,1) (2,0) (2,1) (2,2) (3,0) ... (3,3).  Computed
// rather than read from a table: a memory read here would wait behind the in-flight prefetch.
__device__ __forceinline__ int tri_row(int idx) { return (idx >= 1) + (idx >= 3) + (idx >= 6); }
__device__ __forceinline__ int tri_col(int idx) {
  const int r = tri_row(idx);
  return idx - r * (r + 1) / 2;
}

// Rows 0..63 of one chunk of a [token][D] tensor (src = its row 0) straight into an LDS tile
// of pitch PQ with gfx950's global_load_lds_dwordx4, which writes lane i's 16 bytes to the
// LDS address M0 + 16 i.  Instruction j of a tile therefore fills the tile's 16-byte units
// [64 j, 64 j + 64); unit u is row u / U, slot u % U of a row of U units, the last
// U - D * sizeof(T) / 16 of them padding.  Padding slots and rows at or past Lc (beyond the
// end of the sequence) load row 0 instead: the padding is never read and the rows past the
// end are zeroed by zero_tail once the loads have landed.  Waves w, w + nw, ... issue the
// tile's U instructions.
// The instruction is issued from inline assembly so that the compiler does not track it:
// its wait-count pass would otherwise make every later LDS read that it cannot prove
// disjoint from the (runtime-selected) destination wait for the load.  Callers therefore
// wait themselves: s_waitcnt vmcnt(0), then a barrier, before the tile is read.  Loads the
// compiler does issue are still waited for correctly (the counter drains in order, so loads
// it does not know about only make its own waits stricter).
// Instruction j (0 <= j < PQ * sizeof(T) / 16) of such a tile load; does nothing for larger j.
template <int D, typename T, int PQ>
__device__ __forceinline__ void dma_unit(T (*dst)[PQ], const T* src, int Lc, int j, int lane) {
  constexpr int U = PQ * (int)sizeof(T) / 16, DU = D * (int)sizeof(T) / 16, EPU = 16 / (int)sizeof(T);
  static_assert(PQ * sizeof(T) % 16 == 0, "rows must be whole 16-byte units");
  if (j >= U) return;
  const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) T*)&dst[0][0];
  const int u = 64 * j + lane;
  const int row = u / U, slot = u - row * U;
  const bool ok = row < Lc && slot < DU;
  const T* p = src + (ok ? row * D + slot * EPU : 0);
  const unsigned m0 = __builtin_amdgcn_readfirstlane(base + 1024u * (unsigned)j);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(p) : "memory", "m0");
}

template <int D, typename T, int PQ>
__device__ __forceinline__ void dma_tile(T (*dst)[PQ], const T* src, int Lc, int w, int nw, int lane) {
  constexpr int U = PQ * (int)sizeof(T) / 16;
  for (int j = w; j < U; j += nw) dma_unit<D, T, PQ>(dst, src, Lc, j, lane);
}

// All ROWS rows (row stride D elements) of a block into an LDS tile of pitch PQ, every row valid:
// ceil(ROWS * U / 64) instructions, the last one with only the lanes that have a unit.  Waves w,
// w + nw, ... issue them.  Same untracked loads as dma_unit (the caller waits).
template <int D, typename T, int PQ, int ROWS>
__device__ __forceinline__ void dma_block(T (*dst)[PQ], const T* src, int w, int nw, int lane) {
  constexpr int U = PQ * (int)sizeof(T) / 16, DU = D * (int)sizeof(T) / 16, EPU = 16 / (int)sizeof(T);
  constexpr int NI = (ROWS * U + 63) / 64;
  const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) T*)&dst[0][0];
  for (int j = w; j < NI; j += nw) {
    const int u = 64 * j + lane;
    if (u < ROWS * U) {
      const int row = u / U, slot = u - row * U;
      const T* p = src + (slot < DU ? row * D + slot * EPU : 0);
      const unsigned m0 = __builtin_amdgcn_readfirstlane(base + 1024u * (unsigned)j);
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(p) : "memory", "m0");
    }
  }
}

// One direct load of 16 bytes per calling lane from p into dst + 16 * lane bytes (the lanes that do
// not call write nothing).  Untracked, as above.
template <typename T>
__device__ __forceinline__ void dma_lane(T* dst, const T* p) {
  const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) T*)dst;
  const unsigned m0 = __builtin_amdgcn_readfirstlane(base);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(p) : "memory", "m0");
}

// The same tile loads with the lane's part of every instruction worked out once: instruction
// j = w + NWAVES m of wave w reads row[m] (kL for a padding unit, so it always falls back to
// row 0) at element offset off[m] of the chunk.  A tile load then costs a compare, a select
// and an address add per instruction instead of the division by the row's unit count.
template <int D, typename T, int PQ, int NWAVES>
struct DmaPlan {
  static constexpr int U = PQ * (int)sizeof(T) / 16, DU = D * (int)sizeof(T) / 16, EPU = 16 / (int)sizeof(T);
  static constexpr int M = (U + NWAVES - 1) / NWAVES;  // instructions per wave and tile (at most)
  int row[M];
  int off[M];
  __device__ __forceinline__ DmaPlan(int w, int lane) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int u = 64 * (w + NWAVES * m) + lane;
      const int r = u / U, slot = u - r * U;
      row[m] = slot < DU ? r : kL;
      off[m] = slot < DU ? r * D + slot * EPU : 0;
    }
  }
  // the wave's m-th instruction of the tile (nothing when there is none)
  __device__ __forceinline__ void load_one(T (*dst)[PQ], const T* src, int Lc, int w, int m) const {
    const int j = w + NWAVES * m;
    if (j >= U) return;
    const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) T*)&dst[0][0];
    const T* p = src + (row[m] < Lc ? off[m] : 0);
    const unsigned m0 = __builtin_amdgcn_readfirstlane(base + 1024u * (unsigned)j);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(p) : "memory", "m0");
  }
  __device__ __forceinline__ void load(T (*dst)[PQ], const T* src, int Lc, int w) const {
#pragma unroll
    for (int m = 0; m < M; ++m) load_one(dst, src, Lc, w, m);
  }
};

// C[row][col .. col + 3] of a symmetric D x D matrix held as its packed upper triangle (the
// caller's carry with the packed-statistics flag).
template <int D>
__device__ __forceinline__ f32x4 ld_packed4(const float* p, int row, int col) {
  f32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = p[packed_index(row, col + e, D)];
  return v;
}

// The entries of C[row][col .. col + 3] on or above the diagonal, into a packed upper
// triangle.  Lanes that together hold every (row, col) of C once write every entry of the
// triangle once.
template <int D>
__device__ __forceinline__ void st_packed4(float* p, int row, int col, const f32x4& v) {
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (row <= col + e) p[packed_index(row, col + e, D)] = v[e];
}

// Zeroes rows Lc..63 of an LDS tile (the rows of a chunk past the end of the sequence).
template <int D, typename T, int PQ>
__device__ __forceinline__ void zero_tail(T (*dst)[PQ], int Lc, int tid, int nthreads) {
  for (int e = tid; e < (kL - Lc) * D; e += nthreads) dst[Lc + e / D][e % D] = (T)0.f;
}

// Scales rows 0..63 of an LDS key tile to unit L2 norm, k / max(|k|, 1e-12) in fp32 (the
// library-side normalisation asked for with the normalise-keys flag), 16 lanes per row.
// Every thread of the workgroup takes part; rows of zeros stay zero.  The caller puts a
// barrier after it.
template <int D, typename T, int PQ>
__device__ __forceinline__ void normalize_rows(T (*K)[PQ], int tid, int nthreads) {
  constexpr int EPL = D / 16;  // elements per lane
  const int sub = tid & 15;
  for (int row = tid >> 4; row < kL; row += nthreads >> 4) {
    float x[EPL];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      x[e] = to_f32(K[row][sub * EPL + e]);
      ss += x[e] * x[e];
    }
    ss = group_sum<16>(ss);
    const float inv = __builtin_amdgcn_rsqf(fmaxf(ss, 1e-24f));
#pragma unroll
    for (int e = 0; e < EPL; ++e) K[row][sub * EPL + e] = (T)(x[e] * inv);
  }
}

// Workgroups for the C part when a summary runs in two roles (0: the fused summary): one per
// compute unit the nS summary workgroups leave idle on the 256 of an MI355X, if that gives no C
// workgroup more than three segments (its step is about a third of a summary step).
__host__ __device__ inline int summary_c_groups(int nS) {
  constexpr int kCUs = 256;
  const int Wc = nS < kCUs - nS ? nS : kCUs - nS;
  return (Wc > 0 && 3 * Wc >= nS) ? Wc : 0;
}

// The C part of the segment summaries (both rules), C_seg = sum over the segment's chunks of K^T K,
// on its own: workgroup j (of Wc) takes units (chain, segment) j, j + Wc, ...; key tiles stream
// through two LDS buffers; the products are the summary kernels' own, in their order, so the sums
// are the same.  C goes to the unit's workspace slot (slot_f floats each) at offset D^2.
template <int D, typename T>
struct CSumSmem {
  T Ks[2][kL][Cfg<D, T>::PQ];
};
template <int D, typename T>
__device__ __forceinline__ void csum_body(const FwdArgs& a, CSumSmem<D, T>& sm, int j, int Wc, size_t slot_f) {
  using C_ = Cfg<D, T>;
  constexpr int NW = C_::NW, NA = C_::NA, PQ = C_::PQ;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int cw = 16 * w;
  const int P = a.segments, n = a.chunks_per_segment;
  const int units = a.B * a.H * (P - 1);
  const T* kg = static_cast<const T*>(a.k);
  const bool norm = (a.flags & kFlagNormalizeKeys) != 0;
  const DmaPlan<D, T, PQ, NW> plan(w, lane);
  for (int u = j; u < units; u += Wc) {
    const int chain = u / (P - 1), seg = u % (P - 1);
    const T* src = kg + ((size_t)chain * (size_t)a.T + (size_t)seg * n * kL) * D;  // whole chunks
    f32x4 Cacc[NA];
#pragma unroll
    for (int t = 0; t < NA; ++t) Cacc[t] = zero4();
    plan.load(sm.Ks[0], src, kL, w);
    for (int i = 0; i < n; ++i) {
      vm_wait_all();
      lds_barrier();  // chunk i has landed; chunk i-1's buffer is free
      if (i + 1 < n) plan.load(sm.Ks[(i + 1) & 1], src + (size_t)(i + 1) * kL * D, kL, w);
      T (*Ks)[PQ] = sm.Ks[i & 1];
      if (norm) {
        normalize_rows<D, T, PQ>(Ks, tid, 64 * NW);
        lds_barrier();
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const Frag<T> Bk = tr_frag<T>(&Ks[0][0], PQ, 32 * kk, cw, lane);
#pragma unroll
        for (int t0_ = 0; t0_ < NA; t0_ += 4) {
          Frag<T> Ak[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) Ak[v] = tr_frag<T>(&Ks[0][0], PQ, 32 * kk, 16 * (t0_ + v), lane);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int v = 0; v < 4; ++v) mma(Cacc[t0_ + v], Ak[v], Bk);
        }
      }
    }
    float* slot = static_cast<float*>(a.workspace) + ((size_t)chain * P + seg) * slot_f + (size_t)D * D;
    const int row = cw + l16;
#pragma unroll
    for (int t = 0; t < NA; ++t) *reinterpret_cast<f32x4*>(slot + (size_t)row * D + 16 * t + 4 * g) = Cacc[t];
    lds_barrier();  // the last chunk's buffer is read before the next unit loads over it
  }
}

// Gate logit and m0 . q, then the row tile of P = Q K^T, its inclusive row sums and
// Pm = tril(P - c 1^T), for the 16-token row tiles it = w, w + NWAVES, ... < 4.  Writes
// sm.Pm and sm.tok[i] = {lambda_i, 1/n_i, sq_i / n_i^2, logit_i}; nb is the number of tokens
// before the chunk.  Needs Qs, Ks, Wt staged; Pm rows must be zero above the diagonal tiles.
template <int D, typename T, int NWAVES, typename SM>
__device__ __forceinline__ void ccq_gram_rows(SM& sm, const T (*Ks)[Cfg<D, T>::PQ], int w, int lane, int64_t nb,
                                              float b_lam) {
  using C_ = Cfg<D, T>;
  constexpr int NK = C_::NK, PQ = C_::PQ;
  const int g = lane >> 4, l16 = lane & 15;
  for (int it = w; it < 4; it += NWAVES) {
    {
      f32x4 acc = zero4();  // [q] x [w_hi, w_lo, m0_hi, m0_lo]; B rows 4..15 are zero
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const Frag<T> A = lds_frag<T, KORD_CONTIG>(&sm.Qs[0][0], PQ, 16 * it, 32 * kk, lane);
        Frag<T> B = lds_frag<T, KORD_CONTIG>(&sm.Wt[0][0], PQ, (l16 < 4 ? 0 : -l16), 32 * kk, lane);
        if (l16 >= 4) B = Frag<T>{};
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
        const Frag<T> A = lds_frag<T, KORD_CONTIG>(&Ks[0][0], PQ, 16 * tj, 32 * kk, lane);
        const Frag<T> B = lds_frag<T, KORD_CONTIG>(&sm.Qs[0][0], PQ, 16 * it, 32 * kk, lane);
        mma(Pt[tj], A, B);
      }
      // Pt[tj][r] = P[i][16 tj + 4 g + r]
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Pt[tj][r] = (16 * tj + 4 * g + r <= i) ? Pt[tj][r] : 0.f;
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
}

// R = Q C0 for the wave's NH 16-channel groups cw + 16 h .. + 15 (C0 from the wave's carry
// accumulators: ctile(h, t) is the tile holding C[cw + 16 h + l16][16 t + 4 g + r]):
// R[h][ti][r] at channel cw + 16 h + 4 g + r, token 16 ti + l16.  Needs only Qs, so it can run
// beside ccq_gram_rows.  The Q fragments are read once for all NH groups (as one block ahead of
// their MFMAs when BATCH).
template <int D, typename T, int NH, bool BATCH = true, typename SM, typename CTile>
__device__ __forceinline__ void ccq_query_carry(SM& sm, CTile ctile, int lane, f32x4 (&R)[NH][4]) {
  using C_ = Cfg<D, T>;
  constexpr int NK = C_::NK, PQ = C_::PQ;
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) R[h][ti] = zero4();
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    Frag<T> A[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) A[h] = acc_frag<T>(ctile(h, 2 * kk), ctile(h, 2 * kk + 1));
    Frag<T> Bq[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) Bq[ti] = lds_frag<T, KORD_ACC>(&sm.Qs[0][0], PQ, 16 * ti, 32 * kk, lane);
    if constexpr (BATCH) __builtin_amdgcn_sched_barrier(0);  // the four reads go out together
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int h = 0; h < NH; ++h) mma(R[h][ti], A[h], Bq[ti]);
  }
}

// R += tril(P - c 1^T) K (R from ccq_query_carry), then u and the cleaned query; stores
// qc_i * scale(h, ti, r) to Qa (and its bf16 low part to Qalo when SPLIT) at token
// i = 16 ti + l16, channel cw + 16 h + 4 g + r.  Needs Qs, Ks, Pm and tok from ccq_gram_rows.
template <int D, typename T, int NH, bool SPLIT, typename SM, typename Scale>
__device__ __forceinline__ void ccq_clean_query(SM& sm, const T (*Ks)[Cfg<D, T>::PQ], T (*Qalo)[Cfg<D, T>::PQ],
                                                f32x4 (&R)[NH][4], int cw, int lane, Scale scale) {
  using C_ = Cfg<D, T>;
  constexpr int PT = C_::PT, PQ = C_::PQ;
  const int g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    Frag<T> A[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) A[h] = tr_frag<T>(&Ks[0][0], PQ, 32 * kk, cw + 16 * h, lane);  // K^T, own rows
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      if (kk == 1 && ti < 2) continue;  // tokens 32..63 never precede tokens 0..31
      const Frag<T> B = lds_frag<T, KORD_CONTIG>(&sm.Pm[0][0], PT, 16 * ti, 32 * kk, lane);
#pragma unroll
      for (int h = 0; h < NH; ++h) mma(R[h][ti], A[h], B);
    }
  }
  // R[h][ti][r]: channel cw + 16 h + 4 g + r, token 16 ti + l16
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const int m = cw + 16 * h + 4 * g;
    const f32x4 m04 = *reinterpret_cast<const f32x4*>(&sm.m0[m]);
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      const int i = 16 * ti + l16;
      const f32x4 ts = sm.tok[i];  // lambda, 1/n, sq/n^2
      const f32x4 q4 = ld4<T>(&sm.Qs[i][m]);
      f32x4 qa;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float u = R[h][ti][r] * ts[1] - m04[r] * ts[2];
        qa[r] = (q4[r] - ts[0] * u) * scale(h, ti, r);
      }
      // bf16: hi + lo (the intra-chunk attention is a sum of few, possibly cancelling
      // products when little of the sequence has been read)
      if constexpr (SPLIT) {
        const bf16x4 qh = to_bf16x4(qa);
        *reinterpret_cast<bf16x4*>(&sm.Qa[i][m]) = qh;
        f32x4 ql;
#pragma unroll
        for (int r = 0; r < 4; ++r) ql[r] = qa[r] - (float)qh[r];
        st4<T>(&Qalo[i][m], ql);
      } else {
        st4<T>(&sm.Qa[i][m], qa);
      }
    }
  }
}

}  // namespace ccq
