// C ABI of libccq.so: argument validation, workspace sizing and kernel dispatch.
// Declarations and the contract live in include/ccq.h.  Nothing here allocates, keeps
// state between calls or synchronises the stream.
#include "ccq.h"

#include <hip/hip_runtime.h>

#include "ccq_internal.hpp"
#include "ccq_overlap.hpp"

static_assert(CCQ_FLAG_NORMALIZE_KEYS == ccq::kFlagNormalizeKeys && CCQ_FLAG_PACKED_COV == ccq::kFlagPackedCov,
              "flag bits of the header and the kernels agree");

namespace {

bool misaligned(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

constexpr int kChunk = 64;
// Target number of (chain, segment) workgroups for the prefill: one per compute unit of
// an MI355X (256 CUs).  A function of the shape only, so the workspace size never
// depends on which device is current.
constexpr int kTargetPrefillGroups = 256;

int supported_d(int dtype, int d) {
  if (dtype == CCQ_DTYPE_BF16) return d == 64 || d == 128;
  return d == 64;
}

// Validates p; on success fills the resolved segment count.
int validate_fwd(const ccq_fwd_params* p, int* segments_out, int* chunks_per_seg_out) {
  if (!p) return CCQ_ERR_INVALID_ARG;
  if (p->rule != CCQ_RULE_GLA && p->rule != CCQ_RULE_GDN) return CCQ_ERR_INVALID_ARG;
  if (p->dtype != CCQ_DTYPE_F32 && p->dtype != CCQ_DTYPE_BF16) return CCQ_ERR_INVALID_ARG;
  if (p->B <= 0 || p->H <= 0 || p->T <= 0 || p->d_k <= 0 || p->d_v <= 0) return CCQ_ERR_INVALID_ARG;
  if (p->chunk < 0 || p->segments < 0) return CCQ_ERR_INVALID_ARG;
  if (p->flags & ~(CCQ_FLAG_NORMALIZE_KEYS | CCQ_FLAG_PACKED_COV)) return CCQ_ERR_INVALID_ARG;
  if (p->chunk != 0 && p->chunk != kChunk) return CCQ_ERR_UNSUPPORTED;
  if (p->d_k != p->d_v || !supported_d(p->dtype, p->d_k)) return CCQ_ERR_UNSUPPORTED;
  if (!p->q || !p->k || !p->v || !p->log_alpha || !p->w_lambda || !p->b_lambda || !p->o)
    return CCQ_ERR_INVALID_ARG;
  if ((p->rule == CCQ_RULE_GDN) != (p->beta != nullptr)) return CCQ_ERR_INVALID_ARG;
  const int nin = (p->S0 != nullptr) + (p->C0 != nullptr) + (p->ksum0 != nullptr) + (p->n0 != nullptr);
  const int nout = (p->S_out != nullptr) + (p->C_out != nullptr) + (p->ksum_out != nullptr) + (p->n_out != nullptr);
  if ((nin != 0 && nin != 4) || (nout != 0 && nout != 4)) return CCQ_ERR_INVALID_ARG;
  const void* ptrs[] = {p->q, p->k, p->v, p->log_alpha, p->beta, p->w_lambda, p->b_lambda, p->S0, p->C0,
                        p->ksum0, p->n0, p->o, p->S_out, p->C_out, p->ksum_out, p->n_out, p->workspace,
                        p->chunk_carry};
  for (const void* q : ptrs)
    if (misaligned(q)) return CCQ_ERR_MISALIGNED;
  const long long chains = (long long)p->B * p->H;
  if (chains > (1LL << 24)) return CCQ_ERR_UNSUPPORTED;
  const int nchunks = (p->T + kChunk - 1) / kChunk;
  int seg = p->segments;
  if (seg == 0) {
    long long want = (kTargetPrefillGroups + chains - 1) / chains;
    seg = (int)(want < nchunks ? want : nchunks);
    if (seg < 1) seg = 1;
  }
  if (seg > nchunks) seg = nchunks;
  // Rounds the segment length up to whole chunks and drops empty trailing segments.
  int cps = (nchunks + seg - 1) / seg;
  seg = (nchunks + cps - 1) / cps;
  *segments_out = seg;
  *chunks_per_seg_out = cps;
  return CCQ_OK;
}

size_t fwd_slot(const ccq_fwd_params* p) {
  return (p->rule == CCQ_RULE_GDN) ? ccq::gdn_slot_bytes(p->d_k) : ccq::fwd_slot_bytes(p->d_k);
}

size_t fwd_ws_bytes(const ccq_fwd_params* p, int seg) {
  if (seg <= 1) return 0;
  const size_t chains = (size_t)p->B * p->H;
  return ccq::fwd_count_offset(chains, seg, fwd_slot(p)) + chains * sizeof(int64_t);
}

// Whether any byte of the carry out is also a byte of the carry in.
bool carry_overlaps(const ccq_fwd_params* p) {
  const ccq::CarryRanges in{p->S0, p->C0, p->ksum0, p->n0}, out{p->S_out, p->C_out, p->ksum_out, p->n_out};
  return ccq::carry_ranges_overlap(in, out, (size_t)p->B * p->H, (size_t)p->d_k, (p->flags & CCQ_FLAG_PACKED_COV) != 0);
}

}  // namespace

namespace ccq {

int fwd_resolve(const ccq_fwd_params* p, int* segments, int* chunks_per_segment) {
  return validate_fwd(p, segments, chunks_per_segment);
}

size_t fwd_workspace_for(const ccq_fwd_params* p, int segments) { return fwd_ws_bytes(p, segments); }

int fwd_launch(const ccq_fwd_params* p, int seg, int cps, void* workspace, hipStream_t stream) {
  ccq::FwdArgs a{};
  a.rule = p->rule;
  a.dtype = p->dtype;
  a.B = p->B;
  a.H = p->H;
  a.T = p->T;
  a.d = p->d_k;
  a.segments = seg;
  a.chunks_per_segment = cps;
  a.q = p->q;
  a.k = p->k;
  a.v = p->v;
  a.log_alpha = p->log_alpha;
  a.beta = p->beta;
  a.w_lambda = p->w_lambda;
  a.b_lambda = p->b_lambda;
  a.S0 = p->S0;
  a.C0 = p->C0;
  a.ksum0 = p->ksum0;
  a.n0 = p->n0;
  a.o = p->o;
  a.S_out = p->S_out;
  a.C_out = p->C_out;
  a.ksum_out = p->ksum_out;
  a.n_out = p->n_out;
  a.workspace = workspace;
  a.events = p->phase_events;
  a.flags = p->flags;
  a.snapshot = (seg > 1 && carry_overlaps(p)) ? 1 : 0;
  a.chunk_carry = p->chunk_carry;
  const hipError_t e = ccq::launch_fwd(a, stream);
  return e == hipSuccess ? CCQ_OK : CCQ_ERR_LAUNCH;
}

}  // namespace ccq

namespace {

int validate_bwd(const ccq_bwd_params* p) {
  if (!p) return CCQ_ERR_INVALID_ARG;
  if (p->rule != CCQ_RULE_GLA && p->rule != CCQ_RULE_GDN) return CCQ_ERR_INVALID_ARG;
  if (p->dtype != CCQ_DTYPE_F32 && p->dtype != CCQ_DTYPE_BF16) return CCQ_ERR_INVALID_ARG;
  if (p->B <= 0 || p->H <= 0 || p->T <= 0 || p->d_k <= 0 || p->d_v <= 0 || p->chunk < 0) return CCQ_ERR_INVALID_ARG;
  if (p->flags & ~(CCQ_FLAG_NORMALIZE_KEYS | CCQ_FLAG_PACKED_COV)) return CCQ_ERR_INVALID_ARG;
  if (p->flags != 0) return CCQ_ERR_UNSUPPORTED;
  if (p->chunk != 0 && p->chunk != kChunk) return CCQ_ERR_UNSUPPORTED;
  if (p->d_k != p->d_v || !supported_d(p->dtype, p->d_k)) return CCQ_ERR_UNSUPPORTED;
  const long long groups = (long long)p->B * p->H * ((p->T + kChunk - 1) / kChunk);
  if (groups >= (1LL << 31) || (long long)p->B * p->H > 65535LL) return CCQ_ERR_UNSUPPORTED;
  if (!p->q || !p->k || !p->v || !p->log_alpha || !p->w_lambda || !p->b_lambda || !p->d_o || !p->dq || !p->dk ||
      !p->dv || !p->dlog_alpha || !p->dw_lambda || !p->db_lambda)
    return CCQ_ERR_INVALID_ARG;
  const bool gdn = p->rule == CCQ_RULE_GDN;
  if (gdn != (p->beta != nullptr) || gdn != (p->dbeta != nullptr)) return CCQ_ERR_INVALID_ARG;
  const int nin = (p->S0 != nullptr) + (p->C0 != nullptr) + (p->ksum0 != nullptr) + (p->n0 != nullptr);
  const int nadj = (p->dS_T != nullptr) + (p->dC_T != nullptr) + (p->dksum_T != nullptr);
  const int nout = (p->dS0 != nullptr) + (p->dC0 != nullptr) + (p->dksum0 != nullptr);
  if ((nin != 0 && nin != 4) || (nadj != 0 && nadj != 3) || (nout != 0 && nout != 3)) return CCQ_ERR_INVALID_ARG;
  const void* ptrs[] = {p->q, p->k, p->v, p->log_alpha, p->w_lambda, p->b_lambda, p->S0, p->C0, p->ksum0, p->n0,
                        p->d_o, p->dS_T, p->dC_T, p->dksum_T, p->dq, p->dk, p->dv, p->dlog_alpha, p->dw_lambda,
                        p->db_lambda, p->dS0, p->dC0, p->dksum0, p->workspace, p->beta, p->dbeta,
                        p->chunk_carry};
  for (const void* q : ptrs)
    if (misaligned(q)) return CCQ_ERR_MISALIGNED;
  return CCQ_OK;
}

size_t bwd_ws_bytes(const ccq_bwd_params* p) {
  return p->rule == CCQ_RULE_GDN ? ccq::gdn_bwd_workspace_bytes(p->B, p->H, p->T, p->d_k, p->dtype)
                                 : ccq::bwd_workspace_bytes(p->B, p->H, p->T, p->d_k, p->dtype);
}

}  // namespace

extern "C" {

int32_t ccq_abi_version(void) { return 11; }

const char* ccq_status_string(int32_t status) {
  switch (status) {
    case CCQ_OK: return "ok";
    case CCQ_ERR_INVALID_ARG: return "invalid argument";
    case CCQ_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case CCQ_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case CCQ_ERR_LAUNCH: return "kernel launch failed";
    case CCQ_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

size_t ccq_fwd_workspace_bytes(const ccq_fwd_params* p) {
  int seg = 0, cps = 0;
  if (validate_fwd(p, &seg, &cps) != CCQ_OK) return 0;
  return fwd_ws_bytes(p, seg);
}

int ccq_fwd_chunked(const ccq_fwd_params* p, void* hip_stream) {
  int seg = 0, cps = 0;
  const int st = validate_fwd(p, &seg, &cps);
  if (st != CCQ_OK) return st;
  const size_t need = fwd_ws_bytes(p, seg);
  if (need > 0 && (p->workspace == nullptr || p->workspace_bytes < need)) return CCQ_ERR_WORKSPACE;
  return ccq::fwd_launch(p, seg, cps, p->workspace, static_cast<hipStream_t>(hip_stream));
}

int ccq_decode_step(int32_t rule, int32_t dtype, int32_t N, int32_t H, int32_t d_k, int32_t d_v, const void* q,
                    const void* k, const void* v, const void* log_alpha, const void* beta, const float* w_lambda,
                    const float* b_lambda, float* S, float* C, float* ksum, int64_t* n, void* o,
                    int32_t flags, void* hip_stream) {
  if (rule != CCQ_RULE_GLA && rule != CCQ_RULE_GDN) return CCQ_ERR_INVALID_ARG;
  if (dtype != CCQ_DTYPE_F32 && dtype != CCQ_DTYPE_BF16) return CCQ_ERR_INVALID_ARG;
  if (N <= 0 || H <= 0 || d_k <= 0 || d_v <= 0) return CCQ_ERR_INVALID_ARG;
  if (flags & ~(CCQ_FLAG_NORMALIZE_KEYS | CCQ_FLAG_PACKED_COV)) return CCQ_ERR_INVALID_ARG;
  if (d_k != d_v || (d_k != 64 && d_k != 128)) return CCQ_ERR_UNSUPPORTED;
  if ((long long)N * H > 0x7fffffffLL) return CCQ_ERR_UNSUPPORTED;
  if (!q || !k || !v || !log_alpha || !w_lambda || !b_lambda || !S || !C || !ksum || !n || !o)
    return CCQ_ERR_INVALID_ARG;
  if ((rule == CCQ_RULE_GDN) != (beta != nullptr)) return CCQ_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, log_alpha, beta, w_lambda, b_lambda, S, C, ksum, n, o};
  for (const void* pp : ptrs)
    if (misaligned(pp)) return CCQ_ERR_MISALIGNED;
  ccq::DecodeArgs a{rule, dtype, N, H, d_k, flags, q, k, v, log_alpha, beta, w_lambda, b_lambda, S, C, ksum, n, o};
  const hipError_t e = ccq::launch_decode(a, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? CCQ_OK : CCQ_ERR_LAUNCH;
}

int ccq_key_subspace(int32_t dtype, int32_t B, int32_t H, int32_t T, int32_t d_k, int32_t r, const float* C,
                     const float* ksum, const int64_t* n, const void* k, const uint8_t* needle, float* eigvals,
                     float* basis, float* align, float* delta_mu, int32_t* iters, int32_t flags,
                     void* hip_stream) {
  if (dtype != CCQ_DTYPE_F32 && dtype != CCQ_DTYPE_BF16) return CCQ_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || T <= 0 || d_k <= 0 || r <= 0 || r > d_k) return CCQ_ERR_INVALID_ARG;
  if (flags & ~CCQ_FLAG_PACKED_COV) return CCQ_ERR_INVALID_ARG;
  if (d_k != 64 && d_k != 128) return CCQ_ERR_UNSUPPORTED;
  if (r > ccq::kMaxSubspaceRank) return CCQ_ERR_UNSUPPORTED;
  if ((long long)B * H > 65535LL) return CCQ_ERR_UNSUPPORTED;  // heads index the grid's y dimension
  if (!C || !ksum || !n || !k || !eigvals || !basis || !align) return CCQ_ERR_INVALID_ARG;
  if ((needle == nullptr) != (delta_mu == nullptr)) return CCQ_ERR_INVALID_ARG;
  const void* ptrs[] = {C, ksum, n, k, needle, eigvals, basis, align, delta_mu, iters};
  for (const void* pp : ptrs)
    if (misaligned(pp)) return CCQ_ERR_MISALIGNED;
  ccq::SubspaceArgs a{dtype, B, H, T, d_k, r, flags, C, ksum, n, k, needle, eigvals, basis, align, delta_mu,
                      iters};
  const hipError_t e = ccq::launch_subspace(a, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? CCQ_OK : CCQ_ERR_LAUNCH;
}

int ccq_step_backward(int32_t rule, int32_t dtype, int32_t N, int32_t H, int32_t d_k, int32_t d_v, const void* q,
                      const void* k, const void* v, const void* log_alpha, const void* beta, const float* w_lambda,
                      const float* b_lambda, const float* S, const float* C, const float* ksum, const int64_t* n,
                      const float* d_o, float* dS, float* dC, float* dksum, float* dq, float* dk, float* dv,
                      float* dlog_alpha, float* dbeta, float* dw_lambda, float* db_lambda, int32_t flags,
                      void* hip_stream) {
  if (rule != CCQ_RULE_GLA && rule != CCQ_RULE_GDN) return CCQ_ERR_INVALID_ARG;
  if (dtype != CCQ_DTYPE_F32 && dtype != CCQ_DTYPE_BF16) return CCQ_ERR_INVALID_ARG;
  if (N <= 0 || H <= 0 || d_k <= 0 || d_v <= 0) return CCQ_ERR_INVALID_ARG;
  if (flags & ~(CCQ_FLAG_NORMALIZE_KEYS | CCQ_FLAG_PACKED_COV)) return CCQ_ERR_INVALID_ARG;
  if (flags != 0) return CCQ_ERR_UNSUPPORTED;
  if (d_k != d_v || d_k != 128) return CCQ_ERR_UNSUPPORTED;
  if ((long long)N * H > 0x7fffffffLL) return CCQ_ERR_UNSUPPORTED;
  if (!q || !k || !v || !log_alpha || !w_lambda || !b_lambda || !S || !C || !ksum || !n || !d_o || !dS || !dC ||
      !dksum || !dq || !dk || !dv || !dlog_alpha || !dw_lambda || !db_lambda)
    return CCQ_ERR_INVALID_ARG;
  if ((rule == CCQ_RULE_GDN) != (beta != nullptr) || (rule == CCQ_RULE_GDN) != (dbeta != nullptr))
    return CCQ_ERR_INVALID_ARG;
  const void* ptrs[] = {q, k, v, log_alpha, beta, w_lambda, b_lambda, S, C, ksum, n, d_o, dS, dC,
                        dksum, dq, dk, dv, dlog_alpha, dbeta, dw_lambda, db_lambda};
  for (const void* pp : ptrs)
    if (misaligned(pp)) return CCQ_ERR_MISALIGNED;
  ccq::StepBackArgs a{rule, dtype, N, H, d_k, q, k, v, log_alpha, beta, w_lambda, b_lambda, S, C, ksum, n, d_o,
                      dS, dC, dksum, dq, dk, dv, dlog_alpha, dbeta, dw_lambda, db_lambda};
  const hipError_t e = ccq::launch_step_backward(a, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? CCQ_OK : CCQ_ERR_LAUNCH;
}

size_t ccq_chunk_carry_bytes(int32_t dtype, int32_t B, int32_t H, int32_t T, int32_t d) {
  if ((dtype != CCQ_DTYPE_F32 && dtype != CCQ_DTYPE_BF16) || B <= 0 || H <= 0 || T <= 0 || !supported_d(dtype, d))
    return 0;
  return ccq::chunk_carry_bytes((size_t)B * H, (size_t)((T + kChunk - 1) / kChunk), (size_t)d,
                                dtype == CCQ_DTYPE_BF16 ? 2 : 4);
}

size_t ccq_bwd_workspace_bytes(const ccq_bwd_params* p) {
  if (validate_bwd(p) != CCQ_OK) return 0;
  return bwd_ws_bytes(p);
}

int ccq_bwd_chunked(const ccq_bwd_params* p, void* hip_stream) {
  const int st = validate_bwd(p);
  if (st != CCQ_OK) return st;
  const size_t need = bwd_ws_bytes(p);
  if (p->workspace == nullptr || p->workspace_bytes < need) return CCQ_ERR_WORKSPACE;
  ccq::BwdArgs a{};
  a.rule = p->rule;
  a.beta = p->beta;
  a.dbeta = p->dbeta;
  a.dtype = p->dtype;
  a.B = p->B;
  a.H = p->H;
  a.T = p->T;
  a.d = p->d_k;
  a.nchunks = (p->T + kChunk - 1) / kChunk;
  a.q = p->q;
  a.k = p->k;
  a.v = p->v;
  a.log_alpha = p->log_alpha;
  a.w_lambda = p->w_lambda;
  a.b_lambda = p->b_lambda;
  a.S0 = p->S0;
  a.C0 = p->C0;
  a.ksum0 = p->ksum0;
  a.n0 = p->n0;
  a.d_o = p->d_o;
  a.dS_T = p->dS_T;
  a.dC_T = p->dC_T;
  a.dksum_T = p->dksum_T;
  a.dq = p->dq;
  a.dk = p->dk;
  a.dv = p->dv;
  a.dlog_alpha = p->dlog_alpha;
  a.dw = p->dw_lambda;
  a.db = p->db_lambda;
  a.dS0 = p->dS0;
  a.dC0 = p->dC0;
  a.dksum0 = p->dksum0;
  a.workspace = p->workspace;
  a.events = p->phase_events;
  a.chunk_carry = p->chunk_carry;
  const hipError_t e = ccq::launch_bwd(a, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? CCQ_OK : CCQ_ERR_LAUNCH;
}

}  // extern "C"
