// Chunked prefill of the CCQ read step on a GLA backbone, d = 128, bf16: the pipelined variant
// of gla_main_kernel (same chunk algebra; see ccq_prefill.hip for the derivation from the
// gist.science summary of arXiv 2606.01294, §2 "理论推导", "机制" and "集成").
//
// Per chunk the statistics side (the gate, the Gram rows, Q C0, the cleaned query, C += K^T K,
// the decay factors and k e^-B) does not depend on the state S, and the state side (S0 Qc^T,
// the intra-chunk attention, S += (K e^-B)^T V) needs only the statistics side's cleaned query
// and k e^-B.  So one workgroup of 12 waves splits them: waves 0..7 ("C-waves") own 16 channels
// each of the statistic C and work on chunk c while waves 8..11 ("S-waves") own 32 value rows
// each of S and work on chunk c - 1.  Every SIMD then holds two C-waves and one S-wave whose
// work is independent within a step, so one side's MFMAs overlap the other's vector work and
// latency (three waves per SIMD leave each 168 registers: the carries alone take 32 (C) and
// 64 (S)); a step has two barriers:
//   phase A   C: gate and Gram rows (waves 0..3), Q C0, cumulative decay, k e^-B -> LDS
//             S: O = S0 (Qc e^B)^T, intra-chunk attention (Qc e^B)(K e^-B)^T -> LDS
//   phase B   C: cleaned query -> Qc e^B in place of q, C += K^T K
//             S: O += V^T A^T, o out, S <- diag(e^{B_63}) (S + (K e^-B)^T V)
// Tiles stream HBM -> LDS with global_load_lds_dwordx4 a step ahead (k, v) or half a step
// ahead (q, into the buffer the state side has just finished reading); the log decay goes
// straight into the C-waves' registers.  Rows past the end of the sequence load from a zero
// row, so no tile is ever zeroed in LDS.
//
// The first chunk of a sequence read from an empty state takes hi + lo bf16 operands in the
// intra-chunk attention (as in gla_main_kernel); the pipeline then runs that chunk's state side
// alone, with the low parts parked in the buffers of the next chunk's q and k e^-B.
#include "ccq_internal.hpp"
#include "ccq_prefill_common.hpp"

namespace ccq {

// A 16-byte row of zeros: the source of every tile row past the end of a sequence.
__device__ __align__(16) const unsigned int g_zero16[4] = {0u, 0u, 0u, 0u};

template <int D, typename T>
struct PipeSmem {
  using C_ = Cfg<D, T>;
  T QB[2][kL][C_::PQ];  // chunk c: q rows (c % 2), cleaned in place into Qc e^B
  T KB[2][kL][C_::PQ];  // chunk c: k rows
  T PB[2][kL][C_::PQ];  // chunk c: k e^-B rows (hi part for the split chunk)
  T VB[2][kL][C_::PQ];  // chunk c: v rows
  T Pm[kL][C_::PT];     // statistics side: tril(Q K^T - c 1^T)
  T Am[kL][C_::PT];     // state side: masked intra-chunk attention
  T Wt[2][4][C_::PQ];   // per chunk parity: w_lambda hi, lo; key sum hi, lo
  float m0[2][D];       // key sum before the chunk, per chunk parity
  float eBL[2][D];      // e^{B_63} of the chunk, per chunk parity
  f32x4 tok[kL];        // statistics side, per token: lambda, 1/n, sq/n^2, gate logit + b
};

// The views the shared statistics-side phases (ccq_gram_rows, ccq_query_carry,
// ccq_clean_query) read and write, for chunk parity p.
template <int D, typename T>
struct PipeView {
  using C_ = Cfg<D, T>;
  T (&Qs)[kL][C_::PQ];
  T (&Qa)[kL][C_::PQ];
  T (&Wt)[4][C_::PQ];
  T (&Pm)[kL][C_::PT];
  f32x4 (&tok)[kL];
  float (&m0)[D];
};

// Tile loads as DmaPlan's: instruction j = w + NWAVES m of wave w loads the lane's unit from
// element offset off[m] of the chunk.  A padding unit holds kL * D, so one compare against
// Lc * D sends both it and the rows at or past Lc to the zero row.
template <int D, typename T, int PQ, int NWAVES>
struct PipeDma {
  static constexpr int U = PQ * (int)sizeof(T) / 16, DU = D * (int)sizeof(T) / 16, EPU = 16 / (int)sizeof(T);
  static constexpr int M = (U + NWAVES - 1) / NWAVES;
  int off[M];
  __device__ __forceinline__ PipeDma(int w, int lane) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int u = 64 * (w + NWAVES * m) + lane;
      const int r = u / U, slot = u - r * U;
      off[m] = slot < DU ? r * D + slot * EPU : kL * D;
    }
  }
  __device__ __forceinline__ void load(T (*dst)[PQ], const T* src, int Lc, int w) const {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const int j = w + NWAVES * m;
      if (j >= U) continue;
      const unsigned base = (unsigned)(uintptr_t)(__attribute__((address_space(3))) T*)&dst[0][0];
      const void* p = off[m] < Lc * D ? static_cast<const void*>(src + off[m]) : static_cast<const void*>(g_zero16);
      const unsigned m0 = __builtin_amdgcn_readfirstlane(base + 1024u * (unsigned)j);
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0), "v"(p) : "memory", "m0");
    }
  }
};

template <int CTRL>
__device__ __forceinline__ float pipe_dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Tile shape constants of the pipelined kernel.
template <int D, typename T>
struct PipeCtx {
  using C_ = Cfg<D, T>;
  static constexpr int NA = C_::NA, NK = C_::NK, PQ = C_::PQ, PT = C_::PT;
  static constexpr int NWC = 8, NWS = 4, NWT = NWC + NWS;  // C-waves, S-waves, all
};

// CC: this instantiation writes the carry at every chunk start (FwdArgs::chunk_carry).
template <int D, typename T, bool CC>
__global__ __launch_bounds__(768) void gla_pipe_kernel(FwdArgs a) {
  using X_ = PipeCtx<D, T>;
  constexpr int NA = X_::NA, NK = X_::NK, PQ = X_::PQ, PT = X_::PT;
  constexpr int NWC = X_::NWC, NWS = X_::NWS, NWT = X_::NWT;
  static_assert(D == 128 && sizeof(T) == 2, "the pipelined prefill is built for d = 128, bf16");
  __shared__ PipeSmem<D, T> sm;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool cside = wv < NWC;
  const int P = a.segments, cps = a.chunks_per_segment;
  const int chain = blockIdx.x / P, seg = blockIdx.x % P;
  const int h = chain % a.H;
  const int nchunks = (a.T + kL - 1) / kL;
  const int cbeg = seg * cps;
  const int cend = min(nchunks, cbeg + cps);
  const size_t tok0 = (size_t)chain * (size_t)a.T;
  const T* qg = static_cast<const T*>(a.q);
  const T* kg = static_cast<const T*>(a.k);
  const T* vg = static_cast<const T*>(a.v);
  const T* gg = static_cast<const T*>(a.log_alpha);
  T* og = static_cast<T*>(a.o);
  float* slots = static_cast<float*>(a.workspace);
  const size_t slot_f = 2 * (size_t)D * D + 2 * D;
  auto chunk_len = [&](int ch) { return min(kL, a.T - ch * kL); };

  // ---- carry-in sources (the same as gla_main_kernel's)
  const bool cpacked = (a.flags & kFlagPackedCov) != 0;
  constexpr size_t kTri = (size_t)D * (D + 1) / 2;
  const float* Sin = nullptr;
  const float* Cin = nullptr;
  const float* min_ = nullptr;
  bool cin_packed = false;
  if (P > 1 && (seg > 0 || a.snapshot)) {
    const float* slot = slots + ((size_t)chain * P + seg) * slot_f;
    Sin = slot;
    Cin = slot + (size_t)D * D;
    min_ = slot + 2 * (size_t)D * D;
  } else if (a.S0 != nullptr) {
    Sin = a.S0 + (size_t)chain * D * D;
    cin_packed = cpacked;
    Cin = a.C0 + (size_t)chain * (cpacked ? kTri : (size_t)D * D);
    min_ = a.ksum0 + (size_t)chain * D;
  }
  int64_t nbase = (int64_t)cbeg * kL;  // tokens before the segment
  if (a.n0 != nullptr)
    nbase += a.snapshot ? reinterpret_cast<const int64_t*>(reinterpret_cast<const char*>(a.workspace) +
                                                             fwd_count_offset((size_t)a.B * a.H, P, slot_f * sizeof(float)))[chain]
                        : a.n0[chain];
  const int p0 = cbeg & 1;
  if (tid < D) {
    const int c = tid;
    const float m = min_ ? min_[c] : 0.f;
    const float wl = a.w_lambda[(size_t)h * D + c];
    const T whi = (T)wl, wlo = (T)(wl - (float)whi), mhi = (T)m;
    sm.m0[p0][c] = m;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      sm.Wt[p][0][c] = whi;
      sm.Wt[p][1][c] = wlo;
    }
    sm.Wt[p0][2][c] = mhi;
    sm.Wt[p0][3][c] = (T)(m - (float)mhi);
  }
  for (int e = tid; e < kL * PT; e += 64 * NWT) {
    (&sm.Pm[0][0])[e] = (T)0.f;
    (&sm.Am[0][0])[e] = (T)0.f;
  }

  // ---- the step schedule: the statistics side takes chunk c_at(s) and the state side chunk
  // s_at(s) at step s (-1: none).  With the split first chunk the state side runs that chunk
  // alone at step 1.
  const bool split0 = cbeg < cend && nbase == 0;
  const int n = cend - cbeg;
  auto c_at = [&](int s) -> int {
    if (!split0) return s < n ? cbeg + s : -1;
    if (s == 0) return cbeg;
    if (s == 1) return -1;
    return s - 1 < n ? cbeg + s - 1 : -1;
  };
  auto s_at = [&](int s) -> int {
    if (!split0) return (s >= 1 && s - 1 < n) ? cbeg + s - 1 : -1;
    if (s == 1) return cbeg;
    return (s >= 3 && s - 2 < n) ? cbeg + s - 2 : -1;
  };
  const int nsteps = n <= 0 ? 0 : n + (split0 ? 2 : 1);

  // tile loads; inside the step loops the lane's plan is built once per step from the step's
  // opaque lane index, so no per-lane plan stays live across a loop
  using Plan = PipeDma<D, T, PQ, NWT>;
  auto dma = [&](T (*dst)[PQ], const T* src, int ch, const Plan& plan) {
    plan.load(dst, src + (tok0 + (size_t)ch * kL) * D, chunk_len(ch), wv);
  };
  if (n > 0) {
    const Plan plan(wv, lane);
    dma(sm.QB[cbeg & 1], qg, cbeg, plan);
    dma(sm.KB[cbeg & 1], kg, cbeg, plan);
  }
  // Each side runs its own step loop (so that each is register-allocated on its own) with the
  // same barriers: one before the loop, two per step (s_barrier counts arrivals wherever they
  // are issued).  Inside a loop, lane-derived values come from the lane index recomputed (and
  // made opaque) every step, so the compiler recomputes LDS addresses per step instead of
  // holding dozens of them in registers across the loop.
#define CCQ_PIPE_STEP_LANE()                                                                      \
  int lane_;                                                                                     \
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_)); \
  const int g_ = lane_ >> 4, l16_ = lane_ & 15;                                                  \
  const Plan plan(wv, lane_);

  if (cside) {
    // ======================= statistics side: 16 channels of C per wave
    const int w = wv, cw = 16 * w, hb = w & 1, cb = cw - 16 * hb;
    const float b_lam = a.b_lambda[h];
    f32x4 Cacc[NA];  // C[16a + 4g + r][cw + l16]
    {
      const int row = cw + l16;
#pragma unroll
      for (int t = 0; t < NA; ++t) {
        const int col = 16 * t + 4 * g;
        if (Cin == nullptr)
          Cacc[t] = zero4();
        else if (cin_packed)
          Cacc[t] = ld_packed4<D>(Cin, row, col);
        else
          Cacc[t] = *reinterpret_cast<const f32x4*>(Cin + (size_t)row * D + col);
      }
    }
    vm_wait_all();
    lds_barrier();
    // C and the key sum at every chunk start of the segment, for the chunked backward: the first
    // one here, each later one at the end of the step that updated C to it
    if (CC && n > 0) {
      put_carry_row<D, T, NA>(a, chain, cbeg, 1, cw + l16, g, Cacc);
      if (tid < D) put_carry_ksum<D, T>(a, chain, cbeg, tid, sm.m0[p0][tid]);
    }
    typedef __attribute__((address_space(1))) const bf16x8 gbf16x8;  // global loads, not flat ones
    for (int s = 0; s < nsteps; ++s) {
      CCQ_PIPE_STEP_LANE()
      const int cc = c_at(s), nC = c_at(s + 1), nS = s_at(s + 1);
      // ---- phase A: gate and Gram rows (waves 0..3), Q C0, cumulative decay, k e^-B
      f32x4 R[1][4];   // Q C0 (+ the in-chunk part) for its channels
      f32x4 BT[4];     // B at token 16 ti + l16, channel cw + 4g + r
      if (cc >= 0) {
        const int pc = cc & 1;
        const int Lc = chunk_len(cc);
        // the log decay of its 32-channel block, read after the Gram rows and Q C0: fragment ti
        // = G[16 ti + l16][cb + 8 g .. + 7], rows past the end from the zero row
        bf16x8 gfr[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          const int t = 16 * ti + l16_;
          const void* p = t < Lc ? static_cast<const void*>(gg + (tok0 + (size_t)cc * kL + t) * D + cb + 8 * g_)
                                 : static_cast<const void*>(g_zero16);
          gfr[ti] = *(gbf16x8*)p;
        }
        T (*Ks)[PQ] = sm.KB[pc];
        PipeView<D, T> vw{sm.QB[pc], sm.QB[pc], sm.Wt[pc], sm.Pm, sm.tok, sm.m0[pc]};
        const int64_t nb = nbase + (int64_t)(cc - cbeg) * kL;
        ccq_gram_rows<D, T, NWC>(vw, Ks, w, lane_, nb, b_lam);
        ccq_query_carry<D, T, 1>(vw, [&](int, int t) -> const f32x4& { return Cacc[t]; }, lane_, R);
        const bool csplit = split0 && cc == cbeg;
        T (*Klo)[PQ] = sm.PB[pc ^ 1];  // split chunk only
        const Frag<T> Ih = ident_frag<T>(hb, lane_);
        f32x4 GT[4];
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          GT[ti] = zero4();
          Frag<T> gf;
          gf.v = gfr[ti];
          mma(GT[ti], gf, Ih);
        }
        const Frag<T> Ga = acc_frag<T>(GT[0], GT[1]);
        const Frag<T> Gb = acc_frag<T>(GT[2], GT[3]);
        // cumulative sums over tokens: L(ti, kk) is tril on the diagonal 16-token blocks and all
        // ones left of them, so two patterns (L0, L1) and the ones occur
        {
          const Frag<T> L0 = ltri_frag<T>(0, 0, lane_), L1 = ltri_frag<T>(1, 0, lane_);
          Frag<T> ones;
#pragma unroll
          for (int e = 0; e < 8; ++e) ones.v[e] = (T)1.0f;
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) BT[ti] = zero4();
          mma(BT[0], Ga, L0);
          mma(BT[1], Ga, L1);
          mma(BT[2], Ga, ones);
          mma(BT[2], Gb, L0);
          mma(BT[3], Ga, ones);
          mma(BT[3], Gb, L1);
        }
        f32x4 ks = zero4();
#pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
          f32x4 KC = zero4();  // k at token 16 ti + l16, channel cw + 4g + r
          mma(KC, Ih, lds_frag<T, KORD_CONTIG>(&Ks[0][0], PQ, 16 * ti, cb, lane_));
          ks += KC;
          f32x4 kp;
#pragma unroll
          for (int r = 0; r < 4; ++r) kp[r] = KC[r] * __expf(-BT[ti][r]);
          const int t = 16 * ti + l16_;
          const bf16x4 kh = to_bf16x4(kp);
          *reinterpret_cast<bf16x4*>(&sm.PB[pc][t][cw + 4 * g_]) = kh;
          if (csplit) {
            f32x4 kl;
#pragma unroll
            for (int r = 0; r < 4; ++r) kl[r] = kp[r] - (float)kh[r];
            st4<T>(&Klo[t][cw + 4 * g_], kl);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {  // sum over the 16 tokens of the lane's row
          ks[r] += pipe_dpp<0xB1>(ks[r]);
          ks[r] += pipe_dpp<0x4E>(ks[r]);
          ks[r] += pipe_dpp<0x141>(ks[r]);
          ks[r] += pipe_dpp<0x140>(ks[r]);
        }
        const int c = cw + 4 * g_;
        if (l16_ == 0) {  // key sum after the chunk, for the next chunk's parity
          const f32x4 mn = *reinterpret_cast<const f32x4*>(&sm.m0[pc][c]) + ks;
          *reinterpret_cast<f32x4*>(&sm.m0[pc ^ 1][c]) = mn;
          const bf16x4 mh = to_bf16x4(mn);
          *reinterpret_cast<bf16x4*>(&sm.Wt[pc ^ 1][2][c]) = mh;
          f32x4 ml;
#pragma unroll
          for (int r = 0; r < 4; ++r) ml[r] = mn[r] - (float)mh[r];
          st4<T>(&sm.Wt[pc ^ 1][3][c], ml);
        }
        if (l16_ == 15) {  // token 63
#pragma unroll
          for (int r = 0; r < 4; ++r) sm.eBL[pc][c + r] = __expf(BT[3][r]);
        }
      }
      lds_barrier();
      // ---- phase B: cleaned query -> Qc e^B in place of q, C += K^T K
      (void)plan;  // the state waves issue every tile load of the step (below)
      if (cc >= 0) {
        const int pc = cc & 1;
        T (*Ks)[PQ] = sm.KB[pc];
        PipeView<D, T> vw{sm.QB[pc], sm.QB[pc], sm.Wt[pc], sm.Pm, sm.tok, sm.m0[pc]};
        T (*Qalo)[PQ] = sm.QB[pc ^ 1];  // split chunk only
        if (split0 && cc == cbeg)
          ccq_clean_query<D, T, 1, true>(vw, Ks, Qalo, R, cw, lane_,
                                         [&](int, int ti, int r) { return __expf(BT[ti][r]); });
        else
          ccq_clean_query<D, T, 1, false>(vw, Ks, Qalo, R, cw, lane_,
                                          [&](int, int ti, int r) { return __expf(BT[ti][r]); });
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const Frag<T> Bk = tr_frag<T>(&Ks[0][0], PQ, 32 * kk, cw, lane_);
#pragma unroll
          for (int t0_ = 0; t0_ < NA; t0_ += 4) {
            Frag<T> Ak[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) Ak[u] = tr_frag<T>(&Ks[0][0], PQ, 32 * kk, 16 * (t0_ + u), lane_);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < 4; ++u) mma(Cacc[t0_ + u], Ak[u], Bk);
          }
        }
      }
      vm_wait_all();  // every tile of the next step has landed
      lds_barrier();
      // C and the key sum at the next chunk's start, for the chunked backward (after the step's
      // wait: the stores complete during the next step); the key sum was formed in phase A
      if (CC && cc >= 0 && cc + 1 < cend) {
        put_carry_row<D, T, NA>(a, chain, cc + 1, 1, cw + l16_, g_, Cacc);
        if (tid < D) put_carry_ksum<D, T>(a, chain, cc + 1, tid, sm.m0[(cc + 1) & 1][tid]);
      }
    }
    // ---- carry C out (last segment of the chain)
    if (seg == P - 1 && a.S_out != nullptr) {
      const int row = cw + l16;
      float* Cout = a.C_out + (size_t)chain * (cpacked ? kTri : (size_t)D * D);
#pragma unroll
      for (int t = 0; t < NA; ++t) {
        const int col = 16 * t + 4 * g;
        if (cpacked)
          st_packed4<D>(Cout, row, col, Cacc[t]);
        else
          *reinterpret_cast<f32x4*>(Cout + (size_t)row * D + col) = Cacc[t];
      }
      if (tid < D) a.ksum_out[(size_t)chain * D + tid] = sm.m0[n > 0 ? (cend & 1) : p0][tid];
      if (tid == 0) a.n_out[chain] = nbase + (int64_t)max(0, min(a.T, cend * kL) - cbeg * kL);
    }
  } else {
    // ======================= state side: 32 value rows of S per wave
    const int w = wv - NWC, cw = 32 * w;
    f32x4 Sacc[2][NA];  // S^T[16a + 4g + r][cw + 16 hh + l16]
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int row = cw + 16 * hh + l16;
#pragma unroll
      for (int t = 0; t < NA; ++t)
        Sacc[hh][t] = Sin ? *reinterpret_cast<const f32x4*>(Sin + (size_t)row * D + 16 * t + 4 * g) : zero4();
    }
    vm_wait_all();
    lds_barrier();
    // S at every chunk start of the segment, for the chunked backward: the first one here, each
    // later one at the end of the step that updated S to it (after the step's wait, so that the
    // stores complete during the next step)
    if (CC && n > 0) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) put_carry_row<D, T, NA>(a, chain, cbeg, 0, cw + 16 * hh + l16, g, Sacc[hh]);
    }
    // S += (K e^-B)^T V over tokens 32 kk .. 32 kk + 31 of chunk parity ps (each k e^-B fragment
    // serves both row halves); the decay e^{B_63} follows once both halves are in
    auto s_update = [&](int ps, int kk) {
      int ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      T (*Vs)[PQ] = sm.VB[ps];
      const Frag<T> Bv0 = tr_frag<T>(&Vs[0][0], PQ, 32 * kk, cw, ln);
      const Frag<T> Bv1 = tr_frag<T>(&Vs[0][0], PQ, 32 * kk, cw + 16, ln);
#pragma unroll
      for (int t0_ = 0; t0_ < NA; t0_ += 4) {
        Frag<T> Ap[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) Ap[u] = tr_frag<T>(&sm.PB[ps][0][0], PQ, 32 * kk, 16 * (t0_ + u), ln);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          mma(Sacc[0][t0_ + u], Ap[u], Bv0);
          mma(Sacc[1][t0_ + u], Ap[u], Bv1);
        }
      }
    };
    for (int s = 0; s < nsteps; ++s) {
      CCQ_PIPE_STEP_LANE()
      const int sc = s_at(s), nC = c_at(s + 1), nS = s_at(s + 1);
      f32x4 O[2][4];  // O^T for its value rows cw + 16 hh ..
      // ---- phase A: O = S0 (Qc e^B)^T, intra-chunk attention -> Am
      // The state waves issue every tile load of the step (k and v here, q at phase B's start): the
      // statistics waves, whose phase A is the step's longest path, then issue none (3-5 % off the
      // kernel against all twelve waves sharing each tile's instructions).  The shared barrier after
      // both sides' closing waits still publishes the tiles to every wave.
      const PipeDma<D, T, PQ, NWS> splan(w, lane_);
      auto sdma = [&](T (*dst)[PQ], const T* src, int ch) {
        splan.load(dst, src + (tok0 + (size_t)ch * kL) * D, chunk_len(ch), w);
      };
      if (nC >= 0) sdma(sm.KB[nC & 1], kg, nC);
      if (nS >= 0) sdma(sm.VB[nS & 1], vg, nS);
      if (sc >= 0) {
        const int ps = sc & 1;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) O[hh][ti] = zero4();
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {  // each q fragment serves both row halves
          Frag<T> Bq[4];
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) Bq[ti] = lds_frag<T, KORD_ACC>(&sm.QB[ps][0][0], PQ, 16 * ti, 32 * kk, lane_);
          const Frag<T> A0 = acc_frag<T>(Sacc[0][2 * kk], Sacc[0][2 * kk + 1]);
          const Frag<T> A1 = acc_frag<T>(Sacc[1][2 * kk], Sacc[1][2 * kk + 1]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            mma(O[0][ti], A0, Bq[ti]);
            mma(O[1][ti], A1, Bq[ti]);
          }
        }
        // intra-chunk attention (Qc e^B)(K e^-B)^T on the lower tiles -> Am (masked)
        const bool ssplit = split0 && sc == cbeg;  // hi + lo operands
        for (int idx = w; idx < 10; idx += NWS) {
          const int ti = tri_row(idx), tj = tri_col(idx);
          f32x4 acc = zero4();
          Frag<T> Af[NK], Bf[NK];
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) {
            Af[kk] = lds_frag<T, KORD_CONTIG>(&sm.PB[ps][0][0], PQ, 16 * tj, 32 * kk, lane_);
            Bf[kk] = lds_frag<T, KORD_CONTIG>(&sm.QB[ps][0][0], PQ, 16 * ti, 32 * kk, lane_);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) mma(acc, Af[kk], Bf[kk]);
          if (ssplit) {  // + k_hi q_lo + k_lo q_hi
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) {
              const Frag<T> Al = lds_frag<T, KORD_CONTIG>(&sm.PB[ps ^ 1][0][0], PQ, 16 * tj, 32 * kk, lane_);
              const Frag<T> Bl = lds_frag<T, KORD_CONTIG>(&sm.QB[ps ^ 1][0][0], PQ, 16 * ti, 32 * kk, lane_);
              mma(acc, Af[kk], Bl);
              mma(acc, Al, Bf[kk]);
            }
          }
          const int i = 16 * ti + l16_;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] = (16 * tj + 4 * g_ + r <= i) ? acc[r] : 0.f;
          st4<T>(&sm.Am[i][16 * tj + 4 * g_], acc);
        }
        // the state update's first half (tokens 0..31) here, where the state side would wait for
        // the statistics side's Gram rows; O above has read S0 already.  k e^-B and v of chunk sc
        // have been in LDS since the previous step.
        s_update(ps, 0);
      }
      lds_barrier();
      // ---- phase B: O += V^T A^T, o out, S <- diag(e^{B_63}) (S + (K e^-B)^T V)
      // The state side is phase B's longest path: its waves take issue priority over the
      // statistics waves that share their SIMDs until the step's end (measured ~2% on the pass).
      __builtin_amdgcn_s_setprio(2);
      if (nC >= 0) sdma(sm.QB[nC & 1], qg, nC);
      if (sc >= 0) {
        const int ps = sc & 1;
        const int Lc = chunk_len(sc);
        T (*Vs)[PQ] = sm.VB[ps];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {  // each attention fragment serves both row halves
          const Frag<T> A0 = tr_frag<T>(&Vs[0][0], PQ, 32 * kk, cw, lane_);
          const Frag<T> A1 = tr_frag<T>(&Vs[0][0], PQ, 32 * kk, cw + 16, lane_);
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            if (kk == 1 && ti < 2) continue;
            const Frag<T> B = lds_frag<T, KORD_CONTIG>(&sm.Am[0][0], PT, 16 * ti, 32 * kk, lane_);
            mma(O[0][ti], A0, B);
            mma(O[1][ti], A1, B);
          }
        }
        const size_t t0 = tok0 + (size_t)sc * kL;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int ti = 0; ti < 4; ++ti) {
            const int i = 16 * ti + l16_;
            if (i < Lc) st4<T>(og + (t0 + i) * D + cw + 16 * hh + 4 * g_, O[hh][ti]);
          }
        s_update(ps, 1);  // tokens 32..63 (tokens 0..31 went in phase A)
#pragma unroll
        for (int t = 0; t < NA; ++t) {
          const f32x4 e4 = *reinterpret_cast<const f32x4*>(&sm.eBL[ps][16 * t + 4 * g_]);
          Sacc[0][t] *= e4;
          Sacc[1][t] *= e4;
        }
      }
      __builtin_amdgcn_s_setprio(0);
      vm_wait_all();
      lds_barrier();
      if (CC && sc >= 0 && sc + 1 < cend) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) put_carry_row<D, T, NA>(a, chain, sc + 1, 0, cw + 16 * hh + l16_, g_, Sacc[hh]);
      }
    }
    // ---- carry S out (last segment of the chain)
    if (seg == P - 1 && a.S_out != nullptr) {
      float* Sout = a.S_out + (size_t)chain * D * D;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int t = 0; t < NA; ++t)
          *reinterpret_cast<f32x4*>(Sout + (size_t)(cw + 16 * hh + l16) * D + 16 * t + 4 * g) = Sacc[hh][t];
    }
  }
#undef CCQ_PIPE_STEP_LANE
}

hipError_t launch_gla_pipe(const FwdArgs& a, hipStream_t s) {
  if (a.chunk_carry != nullptr)
    hipLaunchKernelGGL((gla_pipe_kernel<128, __bf16, true>), dim3((unsigned)(a.B * a.H * a.segments)), dim3(768), 0, s, a);
  else
    hipLaunchKernelGGL((gla_pipe_kernel<128, __bf16, false>), dim3((unsigned)(a.B * a.H * a.segments)), dim3(768), 0, s,
                       a);
  return hipGetLastError();
}

}  // namespace ccq
