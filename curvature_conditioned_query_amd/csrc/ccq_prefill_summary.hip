// Segment summaries and the carry scan of the GLA chunked prefill (gfx950): the kernels that
// turn every segment but the last into its net effect on the carry, and those effects into each
// segment's carry-in, so the main kernel (ccq_prefill.hip) can run all segments of a chain at
// once.  The chunk algebra is the one stated at the top of ccq_prefill.hip (same source pages);
// this file sits in its own translation unit so that it can be built with its own LLVM
// scheduling strategy.
#include "ccq_internal.hpp"
#include "ccq_prefill_common.hpp"

namespace ccq {

// ---------------------------------------------------------------- segment summaries

// Segment summary (segments 0 .. P-2 of a chain, which always consist of whole chunks): from
// a zero carry, C = sum K^T K and S^T = sum over chunks of diag(e^{B_63}) (S^T + (K e^-B)^T V)
// (the carry update of the chunk algebra above), the key sum and the total log decay.
// Nothing here depends on the queries, so the chunk loop is software-pipelined with one
// barrier per chunk: in chunk i's interval every wave forms chunk i+1's decayed keys
// (cumulative decay by MFMA, k e^-B, e^{B_63}) while it accumulates chunk i into the carries,
// and the values of chunk i+1 and the keys and log decay of chunk i+2 stream into LDS.  Keys
// are triple-buffered (chunk i feeds K^T K while chunk i+1 feeds the decay and chunk i+2
// lands), the rest double-buffered.
template <int D, typename T>
struct SumSmem {
  using C_ = Cfg<D, T>;
  T Ks[3][kL][C_::PQ];
  T Vs[2][kL][C_::PQ];
  T Gs[2][kL][C_::PQ];
  T Kp[2][kL][C_::PQ];  // k e^-B
  float eBL[2][D];      // e^{B_63} per key channel
};

// WITH_C: the workgroup also accumulates C = sum K^T K (otherwise csum_body does, beside it).
template <int D, typename T, bool WITH_C>
__device__ __forceinline__ void gla_summary_body(const FwdArgs& a, SumSmem<D, T>& sm, int bid) {
  using C_ = Cfg<D, T>;
  constexpr int NW = C_::NW, NA = C_::NA, PQ = C_::PQ;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, l16 = lane & 15;
  const int cw = 16 * w, hb = w & 1, cb = cw - 16 * hb;
  const int P = a.segments, n = a.chunks_per_segment;
  const int chain = bid / (P - 1), seg = bid % (P - 1);
  const int cbeg = seg * n;
  const size_t tok0 = (size_t)chain * (size_t)a.T;
  const T* kg = static_cast<const T*>(a.k);
  const T* vg = static_cast<const T*>(a.v);
  const T* gg = static_cast<const T*>(a.log_alpha);
  const bool norm = (a.flags & kFlagNormalizeKeys) != 0;
  const DmaPlan<D, T, PQ, NW> plan(w, lane);
  auto dma = [&](T (*dst)[PQ], const T* src, int i) {
    plan.load(dst, src + (tok0 + (size_t)(cbeg + i) * kL) * D, kL, w);
  };
  // the m-th load instruction this wave issues for a tile (waves w, w + NW, ... share a tile)
  auto dma_part = [&](T (*dst)[PQ], const T* src, int i, int m) {
    plan.load_one(dst, src + (tok0 + (size_t)(cbeg + i) * kL) * D, kL, w, m);
  };
  constexpr int kParts = DmaPlan<D, T, PQ, NW>::M;  // instructions per wave and tile
  // Loads of an interval in the order they are issued: values of chunk i+1, then keys and log
  // decay of chunk i+2.
  auto issue = [&](int i, int q) {
    if (q < kParts) {
      if (i + 1 < n) dma_part(sm.Vs[(i + 1) & 1], vg, i + 1, q);
    } else if (q < 2 * kParts) {
      if (i + 2 < n) dma_part(sm.Ks[(i + 2) % 3], kg, i + 2, q - kParts);
    } else if (q < 3 * kParts) {
      if (i + 2 < n) dma_part(sm.Gs[i & 1], gg, i + 2, q - 2 * kParts);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x4 Cacc[NA], Sacc[NA];
#pragma unroll
  for (int t = 0; t < NA; ++t) Cacc[t] = Sacc[t] = zero4();
  f32x4 ksum = zero4(), ldec = zero4();  // own channels cw + 4g + r (ldec valid where l16 == 15)
  const Frag<T> Ih = ident_frag<T>(hb, lane);

  // Chunk i's decayed keys into Kp[i & 1] and e^{B_63} into eBL[i & 1], for the wave's own
  // channels; BT[ti][r] = B at token 16 ti + l16, channel cw + 4g + r.
  auto decay_keys = [&](int i) {
    T (*Ks)[PQ] = sm.Ks[i % 3];
    T (*Gs)[PQ] = sm.Gs[i & 1];
    T (*Kp)[PQ] = sm.Kp[i & 1];
    f32x4 GT[4], KC[4];
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      GT[ti] = zero4();  // log alpha at token 16 ti + 4 g + r, channel cw + l16
      mma(GT[ti], lds_frag<T, KORD_CONTIG>(&Gs[0][0], PQ, 16 * ti, cb, lane), Ih);
      KC[ti] = zero4();  // k at token 16 ti + l16, channel cw + 4g + r
      mma(KC[ti], Ih, lds_frag<T, KORD_CONTIG>(&Ks[0][0], PQ, 16 * ti, cb, lane));
    }
    const Frag<T> Ga = acc_frag<T>(GT[0], GT[1]);
    const Frag<T> Gb = acc_frag<T>(GT[2], GT[3]);
    f32x4 BT[4], ks = zero4();
#pragma unroll
    for (int ti = 0; ti < 4; ++ti) {
      BT[ti] = zero4();
      mma(BT[ti], Ga, ltri_frag<T>(ti, 0, lane));
      if (ti >= 2) mma(BT[ti], Gb, ltri_frag<T>(ti, 1, lane));
      ks += KC[ti];
      f32x4 kp;
#pragma unroll
      for (int r = 0; r < 4; ++r) kp[r] = KC[ti][r] * __expf(-BT[ti][r]);
      st4<T>(&Kp[16 * ti + l16][cw + 4 * g], kp);
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
#pragma unroll
      for (int r = 0; r < 4; ++r) ks[r] += __shfl_xor(ks[r], off, 64);
    }
    ksum += ks;
    ldec += BT[3];
    if (l16 == 15) {  // token 63
      const int c = cw + 4 * g;
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.eBL[i & 1][c + r] = __expf(BT[3][r]);
    }
  };

  // prologue: chunks 0 and 1 of keys and log decay, chunk 0 of values; chunk 0's decay
  dma(sm.Ks[0], kg, 0);
  dma(sm.Gs[0], gg, 0);
  dma(sm.Vs[0], vg, 0);
  if (n > 1) {
    dma(sm.Ks[1], kg, 1);
    dma(sm.Gs[1], gg, 1);
  }
  vm_wait_all();
  lds_barrier();
  if (norm) {
    normalize_rows<D, T, PQ>(sm.Ks[0], tid, 64 * NW);
    if (n > 1) normalize_rows<D, T, PQ>(sm.Ks[1], tid, 64 * NW);
    lds_barrier();
  }
  decay_keys(0);
  lds_barrier();

  for (int i = 0; i < n; ++i) {
    // Every buffer a load writes here was last read in the previous interval.  One tile's
    // instructions go out before the decay step, the next tile's after it and the last tile's
    // one at a time between the first MFMA groups of the carry update, so none is left for the
    // interval's end, where the closing wait would take its whole latency (the summary is 4 %
    // faster than with three of them there, and than with all of them issued at once).
#pragma unroll
    for (int q = 0; q < kParts; ++q) issue(i, q);
    if (i + 1 < n) decay_keys(i + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = kParts; q < 2 * kParts; ++q) issue(i, q);

    // carry update of chunk i: C += K^T K;  S^T = diag(e^{B_63}) (S^T + (K e^-B)^T V)
    T (*Ks)[PQ] = sm.Ks[i % 3];
    T (*Kp)[PQ] = sm.Kp[i & 1];
    T (*Vs)[PQ] = sm.Vs[i & 1];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      Frag<T> Bk{};
      if constexpr (WITH_C) Bk = tr_frag<T>(&Ks[0][0], PQ, 32 * kk, cw, lane);
      const Frag<T> Bv = tr_frag<T>(&Vs[0][0], PQ, 32 * kk, cw, lane);
#pragma unroll
      for (int t0_ = 0; t0_ < NA; t0_ += 4) {
        Frag<T> Ak[4], Ap[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if constexpr (WITH_C) Ak[u] = tr_frag<T>(&Ks[0][0], PQ, 32 * kk, 16 * (t0_ + u), lane);
          Ap[u] = tr_frag<T>(&Kp[0][0], PQ, 32 * kk, 16 * (t0_ + u), lane);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if constexpr (WITH_C) mma(Cacc[t0_ + u], Ak[u], Bk);
          mma(Sacc[t0_ + u], Ap[u], Bv);
        }
        if (2 * kParts + kk * (NA / 4) + t0_ / 4 < 3 * kParts) issue(i, 2 * kParts + kk * (NA / 4) + t0_ / 4);
      }
    }
#pragma unroll
    for (int q = 2 * kParts + 2 * (NA / 4); q < 3 * kParts; ++q) issue(i, q);
#pragma unroll
    for (int t = 0; t < NA; ++t) Sacc[t] *= *reinterpret_cast<const f32x4*>(&sm.eBL[i & 1][16 * t + 4 * g]);

    vm_wait_all();
    lds_barrier();
    if (norm && i + 2 < n) {  // chunk i+2's keys have landed: unit rows before their first use
      normalize_rows<D, T, PQ>(sm.Ks[(i + 2) % 3], tid, 64 * NW);
      lds_barrier();
    }
  }

  // slot of (chain, seg): S | C | ksum | log decay
  float* slot = static_cast<float*>(a.workspace) + ((size_t)chain * P + seg) * (2 * (size_t)D * D + 2 * D);
  {
    const int row = cw + l16;
#pragma unroll
    for (int t = 0; t < NA; ++t) {
      const int col = 16 * t + 4 * g;
      *reinterpret_cast<f32x4*>(slot + (size_t)row * D + col) = Sacc[t];
      if constexpr (WITH_C) *reinterpret_cast<f32x4*>(slot + (size_t)D * D + (size_t)row * D + col) = Cacc[t];
    }
    const int c = cw + 4 * g;
    if (l16 == 0) *reinterpret_cast<f32x4*>(slot + 2 * (size_t)D * D + c) = ksum;
    if (l16 == 15) *reinterpret_cast<f32x4*>(slot + 2 * (size_t)D * D + D + c) = ldec;
  }
}

template <int D, typename T>
__global__ __launch_bounds__(4 * D) void gla_summary_kernel(FwdArgs a) {
  __shared__ SumSmem<D, T> sm;
  gla_summary_body<D, T, true>(a, sm, blockIdx.x);
}

// The summary in two roles of one launch: workgroups 0 .. chains (P-1) - 1 summarise S (and the key
// sums and log decays) without C, the rest accumulate C on compute units the summary would leave
// idle.  The C products are a fifth of a summary chunk's latency chain; moving them out of it
// leaves the S workgroups a shorter step.
template <int D, typename T>
union SplitSumSmem {
  SumSmem<D, T> s;
  CSumSmem<D, T> c;
};
template <int D, typename T>
__global__ __launch_bounds__(4 * D) void gla_summary_split_kernel(FwdArgs a) {
  __shared__ SplitSumSmem<D, T> sm;
  const int nS = a.B * a.H * (a.segments - 1);
  if ((int)blockIdx.x < nS)
    gla_summary_body<D, T, false>(a, sm.s, blockIdx.x);
  else
    csum_body<D, T>(a, sm.c, blockIdx.x - nS, gridDim.x - nS, 2 * (size_t)D * D + 2 * D);
}

// Exclusive scan of segment summaries into carry-ins, in place.  Slot p holds the summary
// of segment p (p < P-1) and receives the carry-in of segment p (1 <= p <= P-1):
//   carry_in[0] = carry0 (stored in slot 0 only when the carry out overlaps the carry in;
//                 otherwise segment 0 reads the caller's carry);
//   carry_in[p+1] = (S_in[p] diag(e^{ldec[p]}) + dS[p], C + dC, m + dm).
// One thread per 4 consecutive floats of the S | C | ksum part of a slot.
template <int D>
__global__ __launch_bounds__(256) void gla_scan_kernel(FwdArgs a) {
  const int chain = blockIdx.y;
  const int P = a.segments;
  const size_t slot_f = 2 * (size_t)D * D + 2 * D;
  const int nf4 = (2 * D * D + D) / 4;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= nf4) return;
  const size_t f = (size_t)idx * 4;
  float* base = static_cast<float*>(a.workspace) + (size_t)chain * P * slot_f;
  if (a.snapshot && idx == 0) {  // the caller's token count, for every segment of the main kernel
    int64_t* counts = reinterpret_cast<int64_t*>(static_cast<char*>(a.workspace) +
                                                 fwd_count_offset((size_t)a.B * a.H, P, slot_f * sizeof(float)));
    counts[chain] = a.n0 != nullptr ? a.n0[chain] : 0;
  }
  const bool isS = f < (size_t)D * D;
  const int col = (int)(f % D);
  f32x4 run = zero4();
  if (a.S0 != nullptr) {
    const float* src;
    if (isS)
      src = a.S0 + (size_t)chain * D * D + f;
    else if (f < 2 * (size_t)D * D)
      src = a.C0 + (size_t)chain * D * D + (f - (size_t)D * D);
    else
      src = a.ksum0 + (size_t)chain * D + (f - 2 * (size_t)D * D);
    if (!isS && f < 2 * (size_t)D * D && (a.flags & kFlagPackedCov)) {
      const int e = (int)(f - (size_t)D * D);
      run = ld_packed4<D>(a.C0 + (size_t)chain * D * (D + 1) / 2, e / D, e % D);
    } else {
      run = *reinterpret_cast<const f32x4*>(src);
    }
  }
  // Slots in batches of 8: the batch's summaries (and log decays) are loaded together before
  // the dependent updates, so a long chain waits for memory once per batch, not once per slot.
  constexpr int kBatch = 8;
  for (int p0 = 0; p0 < P; p0 += kBatch) {
    f32x4 sum[kBatch], ld[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int p = p0 + j;
      const float* slot = base + (size_t)p * slot_f;
      sum[j] = (p < P - 1) ? *reinterpret_cast<const f32x4*>(slot + f) : zero4();
      ld[j] = (isS && p < P - 1) ? *reinterpret_cast<const f32x4*>(slot + 2 * (size_t)D * D + D + col) : zero4();
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int p = p0 + j;
      if (p >= P) break;
      if (p > 0 || a.snapshot) *reinterpret_cast<f32x4*>(base + (size_t)p * slot_f + f) = run;
      if (p < P - 1) {
        if (isS) run = run * f32x4{__expf(ld[j][0]), __expf(ld[j][1]), __expf(ld[j][2]), __expf(ld[j][3])};
        run += sum[j];
      }
    }
  }
}

template <int D, typename T>
static void launch_summary_t(const FwdArgs& a, hipStream_t s) {
  const int nS = a.B * a.H * (a.segments - 1);
  const int Wc = summary_c_groups(nS);
  if (Wc > 0)
    hipLaunchKernelGGL((gla_summary_split_kernel<D, T>), dim3((unsigned)(nS + Wc)), dim3(4 * D), 0, s, a);
  else
    hipLaunchKernelGGL((gla_summary_kernel<D, T>), dim3((unsigned)nS), dim3(4 * D), 0, s, a);
}

template <int D>
static void launch_scan_t(const FwdArgs& a, hipStream_t s) {
  const int nf4 = (2 * D * D + D) / 4;
  hipLaunchKernelGGL((gla_scan_kernel<D>), dim3((unsigned)((nf4 + 255) / 256), (unsigned)(a.B * a.H)), dim3(256), 0,
                     s, a);
}

void launch_gla_summary(const FwdArgs& a, hipStream_t s) {
  if (a.dtype == 1) {
    if (a.d == 128) launch_summary_t<128, __bf16>(a, s);
    if (a.d == 64) launch_summary_t<64, __bf16>(a, s);
  } else if (a.d == 64) {
    launch_summary_t<64, float>(a, s);
  }
}

void launch_gla_scan(const FwdArgs& a, hipStream_t s) {
  if (a.d == 128) launch_scan_t<128>(a, s);
  if (a.d == 64) launch_scan_t<64>(a, s);
}

// Summary and scan only: the carry-in of every segment after the first in its workspace slot
// (the chunked backward walks each segment's chunks from there, the first from the caller's carry).
hipError_t launch_gla_segment_carries(const FwdArgs& a, hipStream_t s) {
  const bool supported = (a.dtype == 1 && (a.d == 128 || a.d == 64)) || (a.dtype != 1 && a.d == 64);
  if (!supported) return hipErrorInvalidValue;
  if (a.segments > 1) launch_gla_summary(a, s);
  launch_gla_scan(a, s);
  return hipGetLastError();
}

}  // namespace ccq
