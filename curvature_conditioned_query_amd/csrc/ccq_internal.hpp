// Internal launch interface between the C ABI (ccq_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ccq.h"

namespace ccq {

// The prefill entry points' shared host steps (ccq_api.cpp): argument validation with the
// resolved segment split, the workspace that split needs, and the launch on a given workspace.
int fwd_resolve(const ccq_fwd_params* p, int* segments, int* chunks_per_segment);
size_t fwd_workspace_for(const ccq_fwd_params* p, int segments);
int fwd_launch(const ccq_fwd_params* p, int segments, int chunks_per_segment, void* workspace, hipStream_t stream);

struct DecodeArgs {
  int rule, dtype, N, H, d, flags;
  const void *q, *k, *v, *log_alpha, *beta;
  const float *w_lambda, *b_lambda;
  float *S, *C, *ksum;
  int64_t* n;
  void* o;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// the packed-C variants (their own translation unit)
hipError_t launch_decode_packed(const DecodeArgs& a, hipStream_t stream);

// One prefill call after validation.  Segment scheme: the T tokens of every (b, h)
// chain are cut into `segments` contiguous runs of whole chunks.  With more than one
// segment, a summary kernel condenses every segment but the last, a scan kernel turns
// the summaries into each segment's carry-in (stored in the workspace), and the main
// kernel runs all segments in parallel from their carry-ins.
struct FwdArgs {
  int rule, dtype, B, H, T, d, segments, chunks_per_segment;
  const void *q, *k, *v, *log_alpha, *beta;
  const float *w_lambda, *b_lambda;
  const float *S0, *C0, *ksum0;
  const int64_t* n0;
  void* o;
  float *S_out, *C_out, *ksum_out;
  int64_t* n_out;
  void* workspace;
  void* const* events;  // optional: 4 hipEvent_t around the kernels of the pass
  int flags;             // ccq_flag bits
  // Set when segments > 1 and the carry out overlaps the carry in: the scan then copies the
  // caller's carry into slot 0 and n0 into the workspace's count area, and every segment of
  // the main kernel reads those copies, so no workgroup can read a carry another one has
  // already overwritten.
  int snapshot;
  // Optional: the carry at every chunk start, written for the chunked backward (chunk_carry_*).
  void* chunk_carry;
};

// The carry at the start of every 64-token chunk, as the chunked backward reads it: S_c then C_c
// (d x d each, row-major, the input dtype; C symmetric) per (chain, chunk), chains x NC x 2 d^2
// elements, then m_c (the key sum, d fp32) per (chain, chunk).
__host__ __device__ inline size_t chunk_carry_mat_bytes(size_t chains, size_t NC, size_t d, size_t E) {
  return chains * NC * 2 * d * d * E;
}
__host__ __device__ inline size_t chunk_carry_bytes(size_t chains, size_t NC, size_t d, size_t E) {
  return chunk_carry_mat_bytes(chains, NC, d, E) + chains * NC * d * 4;
}

// The workspace of a prefill with more than one segment: chains x P slots, then one int64
// token count per chain (the snapshot of n0, written only when `snapshot` is set).
__host__ __device__ inline size_t fwd_count_offset(size_t chains, int P, size_t slot_bytes) {
  return chains * (size_t)P * slot_bytes;
}

constexpr int kFlagNormalizeKeys = 1;
constexpr int kFlagPackedCov = 2;  // C0 / C_out / decode C hold the packed upper triangle

// Index of entry (i, j) of a symmetric d x d matrix stored as its upper triangle, row by row:
// row r starts at r d - r (r - 1) / 2.
__host__ __device__ inline int packed_index(int i, int j, int d) {
  const int r = i < j ? i : j, c = i < j ? j : i;
  return r * d - r * (r - 1) / 2 + (c - r);
}

// Key-covariance subspace diagnostic (one call after validation).
constexpr int kMaxSubspaceRank = 32;
struct SubspaceArgs {
  int dtype, B, H, T, d, r, flags;
  const float *C, *ksum;
  const int64_t* n;
  const void* k;
  const uint8_t* needle;
  float *eigvals, *basis, *align, *delta_mu;
  int32_t* iters;
};
hipError_t launch_subspace(const SubspaceArgs& a, hipStream_t stream);

// Backward of one recurrence step (one call after validation).
struct StepBackArgs {
  int rule, dtype, N, H, d;
  const void *q, *k, *v, *log_alpha, *beta;
  const float *w_lambda, *b_lambda;
  const float *S, *C, *ksum;
  const int64_t* n;
  const float* d_o;
  float *dS, *dC, *dksum;
  float *dq, *dk, *dv, *dlog_alpha, *dbeta, *dw, *db;
};
hipError_t launch_step_backward(const StepBackArgs& a, hipStream_t stream);

// Chunked backward of the GLA prefill (one call after validation).  nchunks = ceil(T / 64).
struct BwdArgs {
  int dtype, B, H, T, d, nchunks;
  int rule;              // 0 GLA, 1 Gated DeltaNet
  const void *q, *k, *v, *log_alpha;
  const void* beta;      // Gated DeltaNet: [B, H, T]
  float* dbeta;          // Gated DeltaNet: [B, H, T] fp32
  const float *w_lambda, *b_lambda;
  const float *S0, *C0, *ksum0;
  const int64_t* n0;
  const void* d_o;
  const float *dS_T, *dC_T, *dksum_T;
  float *dq, *dk, *dv, *dlog_alpha, *dw, *db;
  float *dS0, *dC0, *dksum0;
  void* workspace;
  void* const* events;  // optional: 5 hipEvent_t around the passes
  // Optional: the chunk carries a prefill of the same inputs wrote (chunk_carry_*); the backward
  // then reads them instead of recomputing them.
  const void* chunk_carry;
};
size_t bwd_workspace_bytes(int B, int H, int T, int d, int dtype);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);
// the Gated DeltaNet chunked backward (its own translation unit)
size_t gdn_bwd_workspace_bytes(int B, int H, int T, int d, int dtype);
hipError_t launch_gdn_bwd(const BwdArgs& a, hipStream_t stream);

// Segment summary and scan of the GLA prefill only: the carry-in of every segment after the
// first in its workspace slot (the chunked backward walks each segment's chunks from there, the
// first from the caller's carry).
hipError_t launch_gla_segment_carries(const FwdArgs& a, hipStream_t stream);
// the summary (segments > 1) and scan launches themselves (their own translation unit); launch
// errors are left for the caller's hipGetLastError
void launch_gla_summary(const FwdArgs& a, hipStream_t stream);
void launch_gla_scan(const FwdArgs& a, hipStream_t stream);
// The pipelined GLA main kernel (d = 128, bf16, keys as given): statistics and state on
// separate waves a chunk apart.
hipError_t launch_gla_pipe(const FwdArgs& a, hipStream_t stream);

// Bytes of one segment slot of the workspace: GLA (S, C, ksum and the segment's log decay),
// Gated DeltaNet (S, C, ksum and the segment's d x d transition matrix).
size_t fwd_slot_bytes(int d);
size_t gdn_slot_bytes(int d);
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// Gated DeltaNet prefill.
hipError_t launch_gdn(const FwdArgs& a, hipStream_t stream);
// the Gated DeltaNet segment summary kernel (its own translation unit)
hipError_t launch_gdn_summary(const FwdArgs& a, hipStream_t stream);

}  // namespace ccq
