// Host side of the C ABI declared in include/triattn.h: argument checks,
// the per-call sequence plan, workspace layout and kernel launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include <algorithm>

#include "tri_internal.hpp"
#include "triattn.h"

namespace {

using tri::SeqInfo;

thread_local std::string g_last_error;

tri_status fail(tri_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Host tables of a call reach the device through kernel arguments (no
// pinned staging, no process-wide ring; a call can be stream-captured).
// Sequences (or (sequence, layer) pairs) one call may plan: 320 KB of
// plan entries, 128 small write launches.
constexpr int64_t kMaxSeqsPerCall = 8192;
// Whether `stream` is being captured into a HIP graph.
bool capturing(void* stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing((hipStream_t)stream, &cs) == hipSuccess &&
         cs != hipStreamCaptureStatusNone;
}

hipError_t upload(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  return tri::launch_write_args(dst, src, bytes, stream);
}

// ---------------------------------------------------------------------------
// Shapes and plans
// ---------------------------------------------------------------------------
tri_status check_shape(const tri_shape* sh) {
  if (!sh) return fail(TRI_ERR_INVALID_ARGUMENT, "shape is NULL");
  const int d = sh->head_dim;
  if (d < 8 || d > tri::kMaxHeadDim || d % 8 != 0)
    return fail(TRI_ERR_INVALID_ARGUMENT,
                "head_dim must be a multiple of 8 in [8, 256] (16-byte rows, even bands)");
  if (sh->num_kv_heads < 1 || sh->num_q_heads < 1 || sh->num_layers < 1)
    return fail(TRI_ERR_INVALID_ARGUMENT, "head and layer counts must be >= 1");
  if (sh->num_q_heads % sh->num_kv_heads != 0)
    return fail(TRI_ERR_INVALID_ARGUMENT, "num_q_heads must be a multiple of num_kv_heads");
  if (sh->num_q_heads / sh->num_kv_heads > tri::kMaxGroup)
    return fail(TRI_ERR_UNSUPPORTED, "GQA group size above 16 is not supported");
  if (!(sh->rope_theta > 0.0)) return fail(TRI_ERR_INVALID_ARGUMENT, "rope_theta must be > 0");
  if (sh->rope_layout != TRI_ROPE_INTERLEAVED && sh->rope_layout != TRI_ROPE_HALF_SPLIT)
    return fail(TRI_ERR_INVALID_ARGUMENT, "rope_layout must be TRI_ROPE_INTERLEAVED or _HALF_SPLIT");
  return TRI_OK;
}

// How the offsets enter the score: the built-in set {2^0..2^16} averaged
// (tri_score), or a caller-given set averaged or maximised.
struct OffsetMode {
  const double* host = nullptr;  // NULL: built-in set, nothing uploaded
  int n = 0;
  bool max = false;
};

// Where each unit's rows live.  Packed (stride 0): units of n_s (input) or
// b_s (output) rows back to back, sequence s from row L*Hkv*cu_len[s] (or
// its output prefix) unless row0[s] is given; this is the public layout.
// Strided: every unit of sequence s at row0[s] + (l*Hkv + g)*stride, so
// units can grow in place (the decode cache).
struct PlanLayout {
  int64_t in_stride = 0, out_stride = 0;
  const int64_t* in_row0 = nullptr;   // [S] host: first input row per sequence
  const int64_t* out_row0 = nullptr;  // [S] host: first output row per sequence
  const tri::Pages* in_pages = nullptr;   // K/V/positions in a paged pool (scores stay packed)
  const tri::Pages* out_pages = nullptr;  // compacted rows into a paged pool
};

struct Plan {
  std::vector<SeqInfo> seqs;
  int S = 0, L = 0, Hkv = 0, Hq = 0, G = 0, d = 0, F = 0;
  int64_t total_rows = 0, total_out = 0;  // rows spanned by the input / output layout
  int64_t keys = 0, kept = 0;             // rows that hold keys / kept keys
  int max_n = 0, max_b = 0;
  int64_t tickets = 0;
  // workspace offsets (bytes)
  size_t off_seq = 0, off_P = 0, off_W = 0, off_E = 0, off_stats = 0, off_ctrl = 0,
         off_apack = 0, off_raw = 0, off_offsets = 0, off_ustats = 0, off_split = 0;
  int64_t n_units = 0, n_stat_slots = 0;
  int chunk = 0;  // keys per score ticket
  bool fused = false;
  bool half = false;  // half-split RoPE layout
  tri::Pages in_pg, out_pg;  // table == NULL: packed
  OffsetMode om;
  tri::MaxOffsetsPlan mp;  // max-over-offsets path
  size_t score_bytes = 0, select_bytes = 0;
};

tri_status check_offsets(const tri_shape* sh, const OffsetMode& om) {
  if (!om.host) return TRI_OK;
  if (om.n < 1 || om.n > tri::kMaxOffsets)
    return fail(TRI_ERR_INVALID_ARGUMENT, "n_offsets must be in [1, 4096]");
  for (int j = 0; j < om.n; ++j)
    if (!std::isfinite(om.host[j]))
      return fail(TRI_ERR_INVALID_ARGUMENT, "offsets must be finite");
  if (om.max && sh->head_dim % 32 != 0)
    return fail(TRI_ERR_UNSUPPORTED, "the max over offsets needs head_dim % 32 == 0");
  if (om.max && sh->rope_layout == TRI_ROPE_HALF_SPLIT && sh->head_dim % 64 != 0)
    return fail(TRI_ERR_UNSUPPORTED,
                "the max over offsets with the half-split layout needs head_dim % 64 == 0");
  return TRI_OK;
}

tri_status make_plan(const tri_shape* sh, int32_t S, const int64_t* cu_len,
                     const int32_t* cur_pos, const int32_t* budget, Plan& p,
                     const OffsetMode& om = OffsetMode(), const PlanLayout& lay = PlanLayout()) {
  tri_status st = check_shape(sh);
  if (st != TRI_OK) return st;
  st = check_offsets(sh, om);
  if (st != TRI_OK) return st;
  p.om = om;
  if (S < 0) return fail(TRI_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
  if (S > 0 && !cu_len) return fail(TRI_ERR_INVALID_ARGUMENT, "cu_len is NULL");
  if ((int64_t)S > kMaxSeqsPerCall)
    return fail(TRI_ERR_UNSUPPORTED, "too many sequences in one call (max 8192)");
  p.S = S;
  p.L = sh->num_layers;
  p.Hkv = sh->num_kv_heads;
  p.Hq = sh->num_q_heads;
  p.G = p.Hq / p.Hkv;
  p.d = sh->head_dim;
  p.F = p.d / 2;
  p.half = sh->rope_layout == TRI_ROPE_HALF_SPLIT;
  const int64_t LH = (int64_t)p.L * p.Hkv;
  p.seqs.resize(S);
  if (S > 0 && cu_len[0] < 0) return fail(TRI_ERR_INVALID_ARGUMENT, "cu_len[0] must be >= 0");
  int64_t out_acc = 0, ticket_acc = 0;
  // The fused path bounds the chunks of one unit; longer sequences take the
  // generic path, which never waits on other work-groups.
  int64_t longest = 0;
  for (int s = 0; s < S; ++s) longest = std::max<int64_t>(longest, cu_len[s + 1] - cu_len[s]);
  if (om.max) {
    p.mp = tri::plan_max_offsets(p.d, p.G, om.n);
    if (!p.mp.ok)
      return fail(TRI_ERR_UNSUPPORTED,
                  "the max over offsets: one head's offset rows exceed the LDS budget");
  }
  if (lay.in_pages) p.in_pg = *lay.in_pages;
  if (lay.out_pages) p.out_pg = *lay.out_pages;
  // The fused kernel reads a 16-key block from one page.  A unit's chunks
  // must also stay within the work-groups the device holds at once: its
  // waits need more than half that many resident, and capping a unit at
  // the resident count (occupancy x CUs, when a device answers) keeps twice
  // that margin, also on a partitioned or smaller device.
  p.fused = !om.max && tri::fused_supported(p.d, p.half) &&
            (!p.in_pg.table || p.in_pg.page_shift >= 4);
  if (p.fused) {
    const int64_t ch = tri::fused_chunk_keys(p.G, p.d);
    int64_t cap = tri::kFusedMaxUnitChunks;
    const int resident = tri::fused_resident_groups(p.d, p.half, p.in_pg.table != nullptr, p.G);
    if (resident > 0 && resident < cap) cap = resident;
    p.fused = (longest + ch - 1) / ch <= cap;
  }
  p.chunk = p.fused ? tri::fused_chunk_keys(p.G, p.d) : tri::kScoreChunk;
  for (int s = 0; s < S; ++s) {
    const int64_t n = cu_len[s + 1] - cu_len[s];
    if (n < 0) return fail(TRI_ERR_INVALID_ARGUMENT, "cu_len must be non-decreasing");
    if (n > (int64_t)0x7fffffff / 2) return fail(TRI_ERR_UNSUPPORTED, "sequence too long");
    SeqInfo& si = p.seqs[s];
    si.row_base = lay.in_row0 ? lay.in_row0[s] : LH * cu_len[s];
    si.n = (int32_t)n;
    si.in_stride = (int32_t)(lay.in_stride ? lay.in_stride : n);
    if (n > si.in_stride) return fail(TRI_ERR_INVALID_ARGUMENT, "unit longer than its stride");
    int64_t b = 0;
    if (budget) {
      if (budget[s] < 0) return fail(TRI_ERR_INVALID_ARGUMENT, "budget must be >= 0");
      b = budget[s] < n ? budget[s] : n;
    }
    si.b = (int32_t)b;
    if (n > p.max_n) p.max_n = (int)n;
    if (b > p.max_b) p.max_b = (int)b;
    si.out_base = lay.out_row0 ? lay.out_row0[s] : LH * out_acc;
    si.out_stride = (int32_t)(lay.out_stride ? lay.out_stride : b);
    if (b > si.out_stride) return fail(TRI_ERR_INVALID_ARGUMENT, "budget above the output stride");
    p.total_rows = std::max(p.total_rows, si.row_base + LH * si.in_stride);
    p.total_out = std::max(p.total_out, si.out_base + LH * si.out_stride);
    p.keys += LH * n;
    p.kept += LH * b;
    if (p.in_pg.table && ((n + (1 << p.in_pg.page_shift) - 1) >> p.in_pg.page_shift) > p.in_pg.max_pages)
      return fail(TRI_ERR_INVALID_ARGUMENT, "a sequence has more pages than the input page table holds");
    if (p.out_pg.table &&
        ((b + (1 << p.out_pg.page_shift) - 1) >> p.out_pg.page_shift) > p.out_pg.max_pages)
      return fail(TRI_ERR_INVALID_ARGUMENT, "kept keys need more pages than the output page table holds");
    out_acc += b;
    si.p_q = cur_pos ? cur_pos[s] : 0;
    si.chunk_base = (int32_t)ticket_acc;
    ticket_acc += LH * ((n + p.chunk - 1) / p.chunk);
    if (ticket_acc > 0x7fffffff) return fail(TRI_ERR_UNSUPPORTED, "batch too large for one call");
  }
  p.tickets = ticket_acc;

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  // the control words first, at a fixed place (word 1: the fused kernel's
  // wait-bound flag, read by tri_score_status; select never writes there)
  p.off_ctrl = take((size_t)tri::kCtrlHeader * sizeof(uint32_t));
  p.off_seq = take((size_t)S * sizeof(SeqInfo));
  const size_t after_seq = off;
  p.off_offsets = take(om.host ? (size_t)om.n * sizeof(double) : 0);
  p.off_P = take((size_t)p.L * p.Hq * p.F * sizeof(double2));
  p.off_W = take((size_t)p.L * p.Hq * p.F * sizeof(float));
  p.off_E = take((size_t)S * p.F * sizeof(double2));
  // generic path: (count, mean, M2) per ticket and head; fused path: (sum,
  // sum of squares) per ticket and head, reset to a sentinel per call
  p.n_stat_slots = p.fused ? p.tickets * p.G * 2 : 0;
  p.off_stats = take((size_t)p.tickets * tri::kMaxGroup * 3 * sizeof(double));
  p.n_units = (int64_t)S * LH;
  // The fused path keeps raw scores on chip; the generic path spills them.
  p.off_apack = take(om.max ? tri::max_offsets_operand_bytes(p.d, p.G, om.n, p.mp, p.n_units, p.tickets)
                            : tri::fused_operand_bytes(p.d, p.n_units));
  p.off_ustats = take(p.fused ? 0 : (size_t)p.n_units * p.G * 2 * sizeof(double));
  p.off_raw = take(p.fused ? 0 : (size_t)p.total_rows * p.G * sizeof(float));
  p.score_bytes = off;
  // select scratch (split select of long units) reuses the score region:
  // the two never run at the same time on one workspace
  p.off_split = after_seq;
  p.select_bytes = after_seq + tri::split_select_bytes(p.n_units, p.max_n);
  return TRI_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" {

const char* tri_status_string(tri_status s) {
  switch (s) {
    case TRI_OK: return "TRI_OK";
    case TRI_ERR_INVALID_ARGUMENT: return "TRI_ERR_INVALID_ARGUMENT";
    case TRI_ERR_UNSUPPORTED: return "TRI_ERR_UNSUPPORTED";
    case TRI_ERR_WORKSPACE: return "TRI_ERR_WORKSPACE";
    case TRI_ERR_HIP: return "TRI_ERR_HIP";
  }
  return "TRI_ERR_UNKNOWN";
}

const char* tri_last_error(void) { return g_last_error.c_str(); }

uint32_t tri_debug_set_wait_limit(uint32_t polls) { return tri::set_fused_wait_limit(polls); }

unsigned long long* tri_debug_set_phase_buffer(unsigned long long* device_buf) {
  return tri::set_fused_phase_buffer(device_buf);
}

int32_t tri_debug_set_resident_groups(int32_t groups) {
  return tri::set_fused_resident_override(groups > 0 ? groups : 0);
}

size_t tri_workspace_bytes(const tri_shape* shape, int32_t num_seqs, const int64_t* cu_len) {
  Plan p;
  if (make_plan(shape, num_seqs, cu_len, nullptr, nullptr, p) != TRI_OK) return 0;
  return p.score_bytes > p.select_bytes ? p.score_bytes : p.select_bytes;
}

size_t tri_workspace_bytes_offsets(const tri_shape* shape, int32_t num_seqs,
                                   const int64_t* cu_len, int32_t n_offsets, int32_t reduce) {
  if (reduce != TRI_REDUCE_MEAN && reduce != TRI_REDUCE_MAX) {
    fail(TRI_ERR_INVALID_ARGUMENT, "reduce must be TRI_REDUCE_MEAN or TRI_REDUCE_MAX");
    return 0;
  }
  // offsets are only counted here; their values are checked by the call
  std::vector<double> zeros(n_offsets > 0 && n_offsets <= tri::kMaxOffsets ? n_offsets : 0, 0.0);
  OffsetMode om;
  om.host = zeros.data();
  om.n = n_offsets;
  om.max = reduce == TRI_REDUCE_MAX;
  if (zeros.empty()) {
    fail(TRI_ERR_INVALID_ARGUMENT, "n_offsets must be in [1, 4096]");
    return 0;
  }
  Plan p;
  if (make_plan(shape, num_seqs, cu_len, nullptr, nullptr, p, om) != TRI_OK) return 0;
  return p.score_bytes > p.select_bytes ? p.score_bytes : p.select_bytes;
}

size_t tri_trig_correlation_workspace_bytes(const tri_shape* shape, int64_t n_q) {
  if (check_shape(shape) != TRI_OK) return 0;
  if (n_q < 1) {
    fail(TRI_ERR_INVALID_ARGUMENT, "n_q must be >= 1");
    return 0;
  }
  return tri::trig_corr_workspace_bytes(shape->num_layers, shape->num_q_heads, n_q);
}

tri_status tri_trig_correlation(const tri_shape* shape, const uint16_t* q, const int32_t* q_pos,
                                int64_t n_q, const uint16_t* k, const int32_t* k_pos, int64_t n_k,
                                const float* q_centre, double* r, void* workspace,
                                size_t workspace_bytes, void* stream) {
  tri_status st = check_shape(shape);
  if (st != TRI_OK) return st;
  if (shape->head_dim % 32 != 0)
    return fail(TRI_ERR_UNSUPPORTED, "the reconstruction diagnostic needs head_dim % 32 == 0");
  if (n_q < 1 || n_k < 1) return fail(TRI_ERR_INVALID_ARGUMENT, "n_q and n_k must be >= 1");
  if (n_q > (int64_t)0x7fffffff / 16 || n_k > (int64_t)0x7fffffff)
    return fail(TRI_ERR_UNSUPPORTED, "too many samples");
  if (!q || !q_pos || !k || !q_centre || !r)
    return fail(TRI_ERR_INVALID_ARGUMENT, "q, q_pos, k, q_centre and r must be non-NULL");
  if (!aligned16(q) || !aligned16(k))
    return fail(TRI_ERR_INVALID_ARGUMENT, "q and k must be 16-byte aligned");
  const size_t need = tri::trig_corr_workspace_bytes(shape->num_layers, shape->num_q_heads, n_q);
  if (!workspace || workspace_bytes < need)
    return fail(TRI_ERR_WORKSPACE,
                "workspace missing or smaller than tri_trig_correlation_workspace_bytes()");
  hipError_t e = tri::launch_trig_corr(shape->num_layers, shape->num_q_heads, shape->num_kv_heads,
                                       shape->head_dim, n_q, n_k, shape->rope_theta,
                                       shape->rope_layout == TRI_ROPE_HALF_SPLIT, q, q_pos, k,
                                       k_pos, q_centre, (double*)workspace, r, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("trig_correlation: ") + hipGetErrorString(e));
  return TRI_OK;
}

tri_status tri_stream_probe(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return TRI_OK;
  if (!src || !sink) return fail(TRI_ERR_INVALID_ARGUMENT, "src and sink must be non-NULL");
  if (bytes % 16 != 0 || !aligned16(src))
    return fail(TRI_ERR_INVALID_ARGUMENT, "src must be 16-byte aligned and bytes a multiple of 16");
  if (bytes > ((size_t)1 << 62)) return fail(TRI_ERR_INVALID_ARGUMENT, "bytes out of range");
  const hipError_t e = tri::launch_stream_probe(src, (int64_t)bytes, sink, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("stream_probe: ") + hipGetErrorString(e));
  return TRI_OK;
}

size_t tri_calibrate_workspace_bytes(const tri_shape* shape, int64_t n_samples) {
  if (check_shape(shape) != TRI_OK) return 0;
  if (n_samples < 1) {
    fail(TRI_ERR_INVALID_ARGUMENT, "n_samples must be >= 1");
    return 0;
  }
  return tri::calibrate_workspace_bytes(shape->num_layers, shape->num_q_heads, shape->head_dim,
                                        n_samples);
}

tri_status tri_calibrate(const tri_shape* shape, const uint16_t* q, const int32_t* q_pos,
                         int64_t n_samples, float* q_centre, float* q_absmean, float* q_R,
                         void* workspace, size_t workspace_bytes, void* stream) {
  tri_status st = check_shape(shape);
  if (st != TRI_OK) return st;
  if (n_samples < 1) return fail(TRI_ERR_INVALID_ARGUMENT, "n_samples must be >= 1");
  if (!q || !q_centre || !q_absmean || !q_R)
    return fail(TRI_ERR_INVALID_ARGUMENT, "q and every output must be non-NULL");
  if (!aligned16(q)) return fail(TRI_ERR_INVALID_ARGUMENT, "q must be 16-byte aligned");
  const size_t need = tri::calibrate_workspace_bytes(shape->num_layers, shape->num_q_heads,
                                                     shape->head_dim, n_samples);
  if (!workspace || workspace_bytes < need)
    return fail(TRI_ERR_WORKSPACE, "workspace missing or smaller than tri_calibrate_workspace_bytes()");
  if (((uintptr_t)workspace & 15u) != 0)
    return fail(TRI_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  hipError_t e = tri::launch_calibrate(shape->num_layers, shape->num_q_heads, shape->head_dim,
                                       shape->rope_theta, shape->rope_layout == TRI_ROPE_HALF_SPLIT,
                                       q, q_pos, n_samples, q_centre,
                                       q_absmean, q_R, workspace, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("calibrate: ") + hipGetErrorString(e));
  return TRI_OK;
}

}  // extern "C"

namespace {

// Queue the score kernels of a ready plan: upload its sequence table (and
// offsets), the prologue, then the score path the plan chose.
hipError_t run_score(const Plan& p, double theta, const OffsetMode& om, const uint16_t* k,
                     const float* q_centre, const float* q_absmean, const float* q_R,
                     float* scores, float* raw_scores, double* head_stats, char* ws,
                     hipStream_t s) {
  SeqInfo* dseq = (SeqInfo*)(ws + p.off_seq);
  // a given set equal to the built-in {2^0..2^16} under the mean takes the
  // built-in path, so the two give the same bits
  bool builtin = !om.host;
  if (om.host && !om.max && om.n == 17) {
    builtin = true;
    for (int j = 0; j < 17; ++j) builtin = builtin && om.host[j] == std::ldexp(1.0, j);
  }
  double* doff = builtin ? nullptr : (double*)(ws + p.off_offsets);
  // a plan that fits one launch's arguments travels with the first kernel
  const size_t plan_bytes = p.seqs.size() * sizeof(SeqInfo);
  const bool inline_plan = plan_bytes <= sizeof(tri::ArgWords);
  // the fused path (the averaged score) prepares in one kernel of its own
  const bool prep_fused = p.fused;
  hipError_t e = inline_plan ? hipSuccess : upload(dseq, p.seqs.data(), plan_bytes, s);
  if (e == hipSuccess && doff) e = upload(doff, om.host, (size_t)om.n * sizeof(double), s);
  if (e == hipSuccess && !prep_fused)
    e = tri::launch_prologue(p.L, p.Hq, p.d, theta, p.S, dseq,
                             inline_plan ? p.seqs.data() : nullptr, q_centre, q_absmean, q_R,
                             doff, om.n, !om.max, (double2*)(ws + p.off_P), (float*)(ws + p.off_W),
                             (double2*)(ws + p.off_E), (uint32_t*)(ws + p.off_ctrl),
                             tri::kCtrlHeader, (double*)(ws + p.off_stats), p.n_stat_slots, s);
  if (e != hipSuccess) return e;
  float* raw = raw_scores ? raw_scores : (float*)(ws + p.off_raw);
  if (om.max)
    return tri::launch_score_max(dseq, p.S, p.L, p.Hkv, p.G, p.d, om.n, p.mp, theta,
                                 (int)p.tickets, (const double2*)(ws + p.off_P),
                                 (const float*)(ws + p.off_W), (const double2*)(ws + p.off_E),
                                 doff, ws + p.off_apack, k, raw, (double*)(ws + p.off_stats),
                                 (double*)(ws + p.off_ustats), scores, head_stats, p.half,
                                 p.in_pg, s);
  if (p.fused) {
    const tri::PrepArgs pa{theta, p.Hq, q_centre, q_absmean, q_R, doff, om.n,
                           inline_plan ? p.seqs.data() : nullptr, tri::kCtrlHeader,
                           p.n_stat_slots};
    return tri::launch_score_fused(dseq, p.S, p.L, p.Hkv, p.G, p.d, p.chunk, (int)p.tickets,
                                   ws + p.off_apack, k, (double*)(ws + p.off_stats),
                                   (uint32_t*)(ws + p.off_ctrl), scores, raw_scores, head_stats,
                                   p.half, p.in_pg, pa, s);
  }
  return tri::launch_score(dseq, p.S, p.L, p.Hkv, p.G, p.d, (int)p.tickets,
                           (const double2*)(ws + p.off_P), (const float*)(ws + p.off_W),
                           (const double2*)(ws + p.off_E), k, raw, (double*)(ws + p.off_stats),
                           (double*)(ws + p.off_ustats), scores, head_stats, p.half, p.in_pg,
                           s);
}

// Queue select (and the gathers asked for) of a ready plan; the sequence
// table is written to the workspace first (by the first kernel, or a copy
// kernel of its own) unless the caller already wrote it on this stream.
hipError_t run_select_compact(const Plan& p, const float* scores, const uint16_t* k,
                              const uint16_t* v, const int32_t* k_pos, int32_t* kept_idx,
                              uint16_t* k_out, uint16_t* v_out, int32_t* pos_out, char* ws,
                              hipStream_t s, bool upload_seqs = true) {
  SeqInfo* dseq = (SeqInfo*)(ws + p.off_seq);
  const int LH = p.L * p.Hkv;
  return tri::launch_select_compact(dseq, upload_seqs ? p.seqs.data() : nullptr, p.S, LH, p.d,
                                    p.max_n, p.max_b, scores, kept_idx, ws + p.off_split, k, v,
                                    k_pos, k_out, v_out, pos_out, p.in_pg, p.out_pg, s);
}

// ---------------------------------------------------------------------------
// Scoring without allocation (tri_score_noalloc): the workspace is a
// file-scope device array, one copy per device for the life of the process.
// Host code reaches a device's copy only through the address
// hipGetSymbolAddress gives on that device, taken once per device.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_addr;

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_addr.find(dev);
  if (it != g_scratch_addr.end()) {
    *out = it->second;
    return hipSuccess;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  g_scratch_addr[dev] = ptr;
  *out = ptr;
  return hipSuccess;
}

// noalloc: the workspace is the device's scratch array.
tri_status score_impl(const tri_shape* shape, int32_t num_seqs, const int64_t* cu_len,
                      const int32_t* cur_pos, const uint16_t* k, const float* q_centre,
                      const float* q_absmean, const float* q_R, const OffsetMode& om,
                      float* scores, float* raw_scores, double* head_stats, void* workspace,
                      size_t workspace_bytes, void* stream, const tri::Pages* pages = nullptr,
                      bool noalloc = false) {
  Plan p;
  PlanLayout lay;
  lay.in_pages = pages;
  tri_status st = make_plan(shape, num_seqs, cu_len, cur_pos, nullptr, p, om, lay);
  if (st != TRI_OK) return st;
  if (num_seqs > 0 && !cur_pos) return fail(TRI_ERR_INVALID_ARGUMENT, "cur_pos is NULL");
  if (p.keys == 0) return TRI_OK;
  if (!k || !q_centre || !q_absmean || !q_R || !scores)
    return fail(TRI_ERR_INVALID_ARGUMENT, "k, statistics and scores must be non-NULL");
  if (!aligned16(k)) return fail(TRI_ERR_INVALID_ARGUMENT, "k must be 16-byte aligned");
  const size_t need = (raw_scores || p.fused) ? p.off_raw : p.score_bytes;
  if (noalloc) {
    if (need > kNoAllocScratchBytes)
      return fail(TRI_ERR_WORKSPACE, "this call needs " + std::to_string(need) +
                                         " bytes of scratch; tri_score_noalloc holds " +
                                         std::to_string(kNoAllocScratchBytes));
    const hipError_t e = scratch_address(&workspace);
    if (e != hipSuccess)
      return fail(TRI_ERR_HIP, std::string("score scratch: ") + hipGetErrorString(e));
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (!workspace || workspace_bytes < need)
    return fail(TRI_ERR_WORKSPACE, "workspace missing or smaller than tri_workspace_bytes()");
  const hipError_t e = run_score(p, shape->rope_theta, om, k, q_centre, q_absmean, q_R, scores,
                                 raw_scores, head_stats, (char*)workspace, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("score: ") + hipGetErrorString(e));
  return TRI_OK;
}

}  // namespace

extern "C" {

tri_status tri_score(const tri_shape* shape, int32_t num_seqs, const int64_t* cu_len,
                     const int32_t* cur_pos, const uint16_t* k, const int32_t* k_pos,
                     const float* q_centre, const float* q_absmean, const float* q_R,
                     float* scores, float* raw_scores, double* head_stats, void* workspace,
                     size_t workspace_bytes, void* stream) {
  (void)k_pos;
  return score_impl(shape, num_seqs, cu_len, cur_pos, k, q_centre, q_absmean, q_R,
                    OffsetMode(), scores, raw_scores, head_stats, workspace, workspace_bytes,
                    stream);
}

tri_status tri_score_noalloc(const tri_shape* shape, int32_t num_seqs, const int64_t* cu_len,
                             const int32_t* cur_pos, const uint16_t* k, const int32_t* k_pos,
                             const float* q_centre, const float* q_absmean, const float* q_R,
                             float* scores, float* raw_scores, double* head_stats, void* stream) {
  (void)k_pos;
  return score_impl(shape, num_seqs, cu_len, cur_pos, k, q_centre, q_absmean, q_R,
                    OffsetMode(), scores, raw_scores, head_stats, nullptr, 0, stream, nullptr,
                    true);
}

tri_status tri_score_status(const void* workspace, uint32_t* flags, void* stream) {
  if (!flags) return fail(TRI_ERR_INVALID_ARGUMENT, "flags is NULL");
  void* ws = const_cast<void*>(workspace);
  if (!ws) {
    const hipError_t e = scratch_address(&ws);
    if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("score status: ") + hipGetErrorString(e));
  }
  uint32_t word = 0;
  hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(&word, (const char*)ws + sizeof(uint32_t), sizeof(word),
                       hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("score status: ") + hipGetErrorString(e));
  *flags = word ? TRI_SCORE_WAIT_GAVE_UP : 0u;
  return TRI_OK;
}

tri_status tri_score_offsets(const tri_shape* shape, int32_t num_seqs, const int64_t* cu_len,
                             const int32_t* cur_pos, const uint16_t* k, const int32_t* k_pos,
                             const float* q_centre, const float* q_absmean, const float* q_R,
                             const double* offsets, int32_t n_offsets, int32_t reduce,
                             float* scores, float* raw_scores, double* head_stats,
                             void* workspace, size_t workspace_bytes, void* stream) {
  (void)k_pos;
  if (!offsets) return fail(TRI_ERR_INVALID_ARGUMENT, "offsets is NULL");
  if (reduce != TRI_REDUCE_MEAN && reduce != TRI_REDUCE_MAX)
    return fail(TRI_ERR_INVALID_ARGUMENT, "reduce must be TRI_REDUCE_MEAN or TRI_REDUCE_MAX");
  OffsetMode om;
  om.host = offsets;
  om.n = n_offsets;
  om.max = reduce == TRI_REDUCE_MAX;
  return score_impl(shape, num_seqs, cu_len, cur_pos, k, q_centre, q_absmean, q_R, om, scores,
                    raw_scores, head_stats, workspace, workspace_bytes, stream);
}

tri_status tri_select_compact(const tri_shape* shape, int32_t num_seqs, const int64_t* cu_len,
                              const int32_t* budget, const float* scores, const uint16_t* k,
                              const uint16_t* v, const int32_t* k_pos, int32_t* kept_idx,
                              uint16_t* k_out, uint16_t* v_out, int32_t* pos_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && !budget) return fail(TRI_ERR_INVALID_ARGUMENT, "budget is NULL");
  Plan p;
  tri_status st = make_plan(shape, num_seqs, cu_len, nullptr, budget, p);
  if (st != TRI_OK) return st;
  if ((k == nullptr) != (k_out == nullptr) || (v == nullptr) != (v_out == nullptr) ||
      (k_pos == nullptr) != (pos_out == nullptr))
    return fail(TRI_ERR_INVALID_ARGUMENT, "k/k_out, v/v_out and k_pos/pos_out come in pairs");
  if (p.kept == 0) return TRI_OK;
  if (!scores || !kept_idx)
    return fail(TRI_ERR_INVALID_ARGUMENT, "scores and kept_idx must be non-NULL");
  if ((k && (!aligned16(k) || !aligned16(k_out))) || (v && (!aligned16(v) || !aligned16(v_out))))
    return fail(TRI_ERR_INVALID_ARGUMENT, "K/V buffers must be 16-byte aligned");
  if (!workspace || workspace_bytes < p.select_bytes)
    return fail(TRI_ERR_WORKSPACE, "workspace missing or smaller than tri_workspace_bytes()");
  const hipError_t e = run_select_compact(p, scores, k, v, k_pos, kept_idx, k_out, v_out, pos_out,
                                          (char*)workspace, (hipStream_t)stream);
  if (e != hipSuccess)
    return fail(TRI_ERR_HIP, std::string("select_compact: ") + hipGetErrorString(e));
  return TRI_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Decode-loop driver (declared in triattn.h).  Lengths, buffer choice and
// the prune trigger live on the host; every prune is one plan over the
// sequences that reached budget + interval keys: tri_score's kernels on the
// strided cache, the protect pass, then select and compaction into each
// sequence's other buffer.  Both ping-pong buffers are halves of one
// allocation, so one plan can read sequences from either half.
// ---------------------------------------------------------------------------
struct tri_decode {
  tri_shape shape{};
  tri_decode_config cfg{};
  int S = 0, LH = 0, d = 0;
  int64_t C = 0;      // unit stride: budget + interval
  int64_t half = 0;   // rows of one buffer: S * LH * C
  const float *qc = nullptr, *qa = nullptr, *qr = nullptr;
  uint16_t *k = nullptr, *v = nullptr;  // [2 * half][d]
  int32_t* pos = nullptr;               // [2 * half]
  float* scores = nullptr;              // [2 * half]
  int32_t* kept = nullptr;              // [2 * half]
  char* ws = nullptr;                   // score/select workspace
  size_t ws_bytes = 0;
  tri::DecodeItem* items = nullptr;     // [S] per-append targets
  float* pre_scores = nullptr;          // prefill scores (packed input rows)
  size_t pre_rows = 0;
  std::vector<int32_t> len;
  std::vector<uint8_t> cur;             // buffer index per sequence
  std::vector<const uint16_t*> vk, vv;
  std::vector<const int32_t*> vpos;
  std::vector<const float*> vsc;
  std::vector<int64_t> vsc_stride;
  int64_t prunes = 0;
};

namespace {

hipError_t grow(void** p, size_t* have, size_t need) {
  if (need <= *have) return hipSuccess;
  if (*p) {
    hipError_t e = hipFree(*p);
    if (e != hipSuccess) return e;
    *p = nullptr;
    *have = 0;
  }
  hipError_t e = hipMalloc(p, need);
  if (e == hipSuccess) *have = need;
  return e;
}

void refresh_view(tri_decode* dec) {
  for (int s = 0; s < dec->S; ++s) {
    const int64_t row0 = dec->cur[s] * dec->half + (int64_t)s * dec->LH * dec->C;
    dec->vk[s] = dec->k + row0 * dec->d;
    dec->vv[s] = dec->v + row0 * dec->d;
    dec->vpos[s] = dec->pos + row0;
  }
}

}  // namespace

extern "C" {

tri_status tri_decode_create(const tri_shape* shape, int32_t num_seqs,
                             const tri_decode_config* config, const float* q_centre,
                             const float* q_absmean, const float* q_R, tri_decode** out) {
  if (!out) return fail(TRI_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  tri_status st = check_shape(shape);
  if (st != TRI_OK) return st;
  if (!config) return fail(TRI_ERR_INVALID_ARGUMENT, "config is NULL");
  const tri_decode_config c = *config;
  if (num_seqs < 1) return fail(TRI_ERR_INVALID_ARGUMENT, "num_seqs must be >= 1");
  if (c.budget < 1 || c.interval < 1 || c.protect_sink < 0 || c.protect_recent < 0)
    return fail(TRI_ERR_INVALID_ARGUMENT, "budget and interval must be >= 1, protections >= 0");
  if ((int64_t)c.protect_sink + c.protect_recent > c.budget)
    return fail(TRI_ERR_INVALID_ARGUMENT, "protect_sink + protect_recent must be <= budget");
  if ((int64_t)c.budget + c.interval > (int64_t)0x7fffffff / 2)
    return fail(TRI_ERR_UNSUPPORTED, "budget + interval too large");
  if (!q_centre || !q_absmean || !q_R)
    return fail(TRI_ERR_INVALID_ARGUMENT, "statistics must be non-NULL");
  tri_decode* dec = new tri_decode();
  dec->shape = *shape;
  dec->cfg = c;
  dec->S = num_seqs;
  dec->LH = shape->num_layers * shape->num_kv_heads;
  dec->d = shape->head_dim;
  dec->C = (int64_t)c.budget + c.interval;
  dec->half = (int64_t)num_seqs * dec->LH * dec->C;
  dec->qc = q_centre;
  dec->qa = q_absmean;
  dec->qr = q_R;
  dec->len.assign(num_seqs, 0);
  dec->cur.assign(num_seqs, 0);
  dec->vk.assign(num_seqs, nullptr);
  dec->vv.assign(num_seqs, nullptr);
  dec->vpos.assign(num_seqs, nullptr);
  dec->vsc.assign(num_seqs, nullptr);
  dec->vsc_stride.assign(num_seqs, 0);
  // workspace of a prune of every sequence at once (either half)
  std::vector<int64_t> cu(num_seqs + 1), r_in(num_seqs), r_out(num_seqs);
  std::vector<int32_t> bud(num_seqs, c.budget);
  for (int s = 0; s <= num_seqs; ++s) cu[s] = (int64_t)s * dec->C;
  for (int s = 0; s < num_seqs; ++s) {
    r_in[s] = dec->half + (int64_t)s * dec->LH * dec->C;
    r_out[s] = r_in[s];
  }
  PlanLayout lay;
  lay.in_stride = lay.out_stride = dec->C;
  lay.in_row0 = r_in.data();
  lay.out_row0 = r_out.data();
  Plan p;
  st = make_plan(shape, num_seqs, cu.data(), nullptr, bud.data(), p, OffsetMode(), lay);
  if (st != TRI_OK) {
    delete dec;
    return st;
  }
  const size_t rows = 2 * (size_t)dec->half;
  const size_t d = (size_t)dec->d;
  hipError_t e = hipMalloc((void**)&dec->k, rows * d * 2);
  if (e == hipSuccess) e = hipMalloc((void**)&dec->v, rows * d * 2);
  if (e == hipSuccess) e = hipMalloc((void**)&dec->pos, rows * 4);
  if (e == hipSuccess) e = hipMalloc((void**)&dec->scores, rows * 4);
  if (e == hipSuccess) e = hipMalloc((void**)&dec->kept, rows * 4);
  if (e == hipSuccess)
    e = grow((void**)&dec->ws, &dec->ws_bytes, std::max(p.score_bytes, p.select_bytes));
  if (e == hipSuccess) e = hipMalloc((void**)&dec->items, (size_t)num_seqs * sizeof(tri::DecodeItem));
  if (e != hipSuccess) {
    tri_decode_destroy(dec);
    return fail(TRI_ERR_HIP, std::string("decode create: ") + hipGetErrorString(e));
  }
  refresh_view(dec);
  *out = dec;
  return TRI_OK;
}

tri_status tri_decode_prefill(tri_decode* dec, const int64_t* cu_len, const int32_t* cur_pos,
                              const uint16_t* k, const uint16_t* v, const int32_t* k_pos,
                              void* stream) {
  if (!dec) return fail(TRI_ERR_INVALID_ARGUMENT, "driver is NULL");
  if (capturing(stream))
    return fail(TRI_ERR_UNSUPPORTED,
                "the decode-loop driver may allocate and cannot be stream-captured");
  if (!cu_len || !cur_pos) return fail(TRI_ERR_INVALID_ARGUMENT, "cu_len and cur_pos are required");
  const int S = dec->S;
  std::vector<int32_t> bud(S);
  std::vector<int64_t> r_out(S);
  bool any_prune = false;
  for (int s = 0; s < S; ++s) {
    const int64_t n = cu_len[s + 1] - cu_len[s];
    if (n < 0) return fail(TRI_ERR_INVALID_ARGUMENT, "cu_len must be non-decreasing");
    const bool prune = n >= dec->C;
    any_prune |= prune;
    bud[s] = prune ? dec->cfg.budget : (int32_t)n;
    r_out[s] = (int64_t)s * dec->LH * dec->C;  // buffer 0
  }
  PlanLayout lay;
  lay.out_stride = dec->C;
  lay.out_row0 = r_out.data();
  Plan p;
  tri_status st = make_plan(&dec->shape, S, cu_len, cur_pos, bud.data(), p, OffsetMode(), lay);
  if (st != TRI_OK) return st;
  if (p.keys > 0 && (!k || !v || !k_pos))
    return fail(TRI_ERR_INVALID_ARGUMENT, "k, v and k_pos are required");
  if ((k && !aligned16(k)) || (v && !aligned16(v)))
    return fail(TRI_ERR_INVALID_ARGUMENT, "K/V buffers must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = grow((void**)&dec->ws, &dec->ws_bytes, std::max(p.score_bytes, p.select_bytes));
  if (e == hipSuccess && any_prune)
    e = grow((void**)&dec->pre_scores, &dec->pre_rows, (size_t)p.total_rows * sizeof(float));
  if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("decode prefill: ") + hipGetErrorString(e));
  if (p.keys > 0) {
    float* sc = any_prune ? dec->pre_scores : dec->scores;
    if (any_prune) {
      e = run_score(p, dec->shape.rope_theta, OffsetMode(), k, dec->qc, dec->qa, dec->qr, sc,
                    nullptr, nullptr, dec->ws, s);
      if (e == hipSuccess)
        e = tri::launch_protect((const SeqInfo*)(dec->ws + p.off_seq), S, dec->LH,
                                dec->cfg.protect_sink, dec->cfg.protect_recent, sc, s);
    }
    // sequences below the trigger keep every key (b = n: the identity)
    if (e == hipSuccess)
      e = run_select_compact(p, sc, k, v, k_pos, dec->kept, dec->k, dec->v, dec->pos, dec->ws, s,
                             !any_prune);
    if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("decode prefill: ") + hipGetErrorString(e));
  }
  for (int i = 0; i < S; ++i) {
    const int64_t n = cu_len[i + 1] - cu_len[i];
    dec->len[i] = bud[i];
    dec->cur[i] = 0;
    dec->vsc[i] = n >= dec->C ? dec->pre_scores + p.seqs[i].row_base : nullptr;
    dec->vsc_stride[i] = n >= dec->C ? n : 0;
    if (n >= dec->C) ++dec->prunes;
  }
  refresh_view(dec);
  return TRI_OK;
}

tri_status tri_decode_append(tri_decode* dec, const uint16_t* k_new, const uint16_t* v_new,
                             const int32_t* pos_new, void* stream) {
  if (!dec) return fail(TRI_ERR_INVALID_ARGUMENT, "driver is NULL");
  if (capturing(stream))
    return fail(TRI_ERR_UNSUPPORTED,
                "the decode-loop driver may allocate and cannot be stream-captured");
  if (!k_new || !v_new || !pos_new)
    return fail(TRI_ERR_INVALID_ARGUMENT, "k_new, v_new and pos_new are required");
  if (!aligned16(k_new) || !aligned16(v_new))
    return fail(TRI_ERR_INVALID_ARGUMENT, "K/V buffers must be 16-byte aligned");
  const int S = dec->S;
  std::vector<tri::DecodeItem> it(S);
  std::vector<int> hit;
  for (int s = 0; s < S; ++s) {
    it[s].row0 = dec->cur[s] * dec->half + (int64_t)s * dec->LH * dec->C + dec->len[s];
    it[s].pos = pos_new[s];
    it[s].pad = 0;
    if (dec->len[s] + 1 == dec->C) hit.push_back(s);
  }
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (S <= tri::kAppendInline) {
    // the items ride in the launch: no staging copy per decode step
    e = tri::launch_append_inline(it.data(), S, dec->LH, dec->d, dec->C, k_new, v_new, dec->k,
                                  dec->v, dec->pos, st);
  } else {
    e = upload(dec->items, it.data(), it.size() * sizeof(tri::DecodeItem), st);
    if (e == hipSuccess)
      e = tri::launch_append(dec->items, S, dec->LH, dec->d, dec->C, k_new, v_new, dec->k,
                             dec->v, dec->pos, st);
  }
  if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("decode append: ") + hipGetErrorString(e));
  for (int s = 0; s < S; ++s) ++dec->len[s];
  if (hit.empty()) return TRI_OK;

  // prune the sequences that reached budget + interval keys
  const int P = (int)hit.size();
  std::vector<int64_t> cu(P + 1), r_in(P), r_out(P);
  std::vector<int32_t> cp(P), bud(P, dec->cfg.budget);
  for (int i = 0; i <= P; ++i) cu[i] = (int64_t)i * dec->C;
  for (int i = 0; i < P; ++i) {
    const int s = hit[i];
    const int64_t off = (int64_t)s * dec->LH * dec->C;
    r_in[i] = dec->cur[s] * dec->half + off;
    r_out[i] = (1 - dec->cur[s]) * dec->half + off;
    cp[i] = pos_new[s];
  }
  PlanLayout lay;
  lay.in_stride = lay.out_stride = dec->C;
  lay.in_row0 = r_in.data();
  lay.out_row0 = r_out.data();
  Plan p;
  tri_status rs = make_plan(&dec->shape, P, cu.data(), cp.data(), bud.data(), p, OffsetMode(), lay);
  if (rs != TRI_OK) return rs;
  // the two halves share one allocation: rows read and rows written never
  // overlap (input and output halves differ for every sequence)
  e = run_score(p, dec->shape.rope_theta, OffsetMode(), dec->k, dec->qc, dec->qa, dec->qr,
                dec->scores, nullptr, nullptr, dec->ws, st);
  if (e == hipSuccess)
    e = tri::launch_protect((const SeqInfo*)(dec->ws + p.off_seq), P, dec->LH,
                            dec->cfg.protect_sink, dec->cfg.protect_recent, dec->scores, st);
  if (e == hipSuccess)
    e = run_select_compact(p, dec->scores, dec->k, dec->v, dec->pos, dec->kept, dec->k, dec->v,
                           dec->pos, dec->ws, st, false);
  if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("decode prune: ") + hipGetErrorString(e));
  for (int i = 0; i < P; ++i) {
    const int s = hit[i];
    dec->vsc[s] = dec->scores + r_in[i];
    dec->vsc_stride[s] = dec->C;
    dec->cur[s] ^= 1;
    dec->len[s] = dec->cfg.budget;
  }
  dec->prunes += P;
  refresh_view(dec);
  return TRI_OK;
}

tri_status tri_decode_get_view(const tri_decode* dec, tri_decode_view* view) {
  if (!dec || !view) return fail(TRI_ERR_INVALID_ARGUMENT, "driver and view must be non-NULL");
  view->unit_stride = dec->C;
  view->k = dec->vk.data();
  view->v = dec->vv.data();
  view->pos = dec->vpos.data();
  view->len = dec->len.data();
  view->scores = dec->vsc.data();
  view->scores_stride = dec->vsc_stride.data();
  view->prunes = dec->prunes;
  return TRI_OK;
}

tri_status tri_decode_destroy(tri_decode* dec) {
  if (!dec) return TRI_OK;
  hipError_t e = hipDeviceSynchronize();
  void* bufs[] = {dec->k, dec->v, dec->pos, dec->scores, dec->kept, dec->ws, dec->items,
                  dec->pre_scores};
  for (void* b : bufs)
    if (b) {
      const hipError_t f = hipFree(b);
      if (e == hipSuccess) e = f;
    }
  delete dec;
  if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("decode destroy: ") + hipGetErrorString(e));
  return TRI_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Per-layer budgets.  Select and gather never look at the layer, so each
// (sequence, layer) becomes a pseudo-sequence of Hkv units with its own
// budget, reading the units where the packed layout has them.
// ---------------------------------------------------------------------------
extern "C" {

tri_status tri_pyramid_budgets(int32_t num_layers, double mean_budget, double ratio,
                               int32_t* budgets) {
  if (num_layers < 1 || !budgets) return fail(TRI_ERR_INVALID_ARGUMENT, "num_layers >= 1 and budgets");
  if (!(mean_budget >= 0.0) || !(ratio > 0.0) || !std::isfinite(mean_budget) ||
      !std::isfinite(ratio) || mean_budget > 1e9)
    return fail(TRI_ERR_INVALID_ARGUMENT, "mean_budget must be in [0, 1e9], ratio > 0");
  if (num_layers == 1) {
    budgets[0] = (int32_t)std::floor(mean_budget + 0.5);
    return TRI_OK;
  }
  const double b0 = 2.0 * mean_budget / (1.0 + ratio), b1 = ratio * b0;
  for (int l = 0; l < num_layers; ++l)
    budgets[l] = (int32_t)std::floor(b0 + (b1 - b0) * l / (double)(num_layers - 1) + 0.5);
  return TRI_OK;
}

size_t tri_workspace_bytes_layers(const tri_shape* shape, int32_t num_seqs,
                                  const int64_t* cu_len) {
  // pseudo-sequences of one layer each: the plan table grows by L
  if (check_shape(shape) != TRI_OK || num_seqs < 0 || (num_seqs > 0 && !cu_len)) return 0;
  const int64_t S2 = (int64_t)num_seqs * shape->num_layers;
  if (S2 > kMaxSeqsPerCall) {
    fail(TRI_ERR_UNSUPPORTED, "too many (sequence, layer) pairs in one call (max 8192)");
    return 0;
  }
  int64_t max_n = 0;
  for (int s = 0; s < num_seqs; ++s) max_n = std::max(max_n, cu_len[s + 1] - cu_len[s]);
  if (max_n > 0x7fffffff) return 0;
  return align_up((size_t)tri::kCtrlHeader * sizeof(uint32_t), 256) +
         align_up((size_t)S2 * sizeof(SeqInfo), 256) +
         tri::split_select_bytes(S2 * shape->num_kv_heads, (int)max_n);
}

tri_status tri_select_compact_layers(const tri_shape* shape, int32_t num_seqs,
                                     const int64_t* cu_len, const int32_t* budget,
                                     const float* scores, const uint16_t* k, const uint16_t* v,
                                     const int32_t* k_pos, int32_t* kept_idx, uint16_t* k_out,
                                     uint16_t* v_out, int32_t* pos_out, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  tri_status st = check_shape(shape);
  if (st != TRI_OK) return st;
  if (num_seqs < 0) return fail(TRI_ERR_INVALID_ARGUMENT, "num_seqs must be >= 0");
  if (num_seqs > 0 && (!cu_len || !budget))
    return fail(TRI_ERR_INVALID_ARGUMENT, "cu_len and budget are required");
  const int L = shape->num_layers, Hkv = shape->num_kv_heads;
  const int64_t S2 = (int64_t)num_seqs * L;
  if (S2 > kMaxSeqsPerCall)
    return fail(TRI_ERR_UNSUPPORTED, "too many (sequence, layer) pairs in one call (max 8192)");
  std::vector<int64_t> cu2(S2 + 1, 0), in0(S2), out0(S2);
  std::vector<int32_t> bud2(S2);
  int64_t out_acc = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t n = cu_len[s + 1] - cu_len[s];
    if (n < 0) return fail(TRI_ERR_INVALID_ARGUMENT, "cu_len must be non-decreasing");
    for (int l = 0; l < L; ++l) {
      const int64_t i = (int64_t)s * L + l;
      if (budget[i] < 0) return fail(TRI_ERR_INVALID_ARGUMENT, "budget must be >= 0");
      cu2[i + 1] = cu2[i] + n;
      in0[i] = (int64_t)L * Hkv * cu_len[s] + (int64_t)l * Hkv * n;
      out0[i] = out_acc;
      bud2[i] = budget[i];
      out_acc += (int64_t)Hkv * std::min<int64_t>(budget[i], n);
    }
  }
  tri_shape sh1 = *shape;
  sh1.num_layers = 1;
  PlanLayout lay;
  lay.in_row0 = in0.data();
  lay.out_row0 = out0.data();
  Plan p;
  st = make_plan(&sh1, (int32_t)S2, cu2.data(), nullptr, bud2.data(), p, OffsetMode(), lay);
  if (st != TRI_OK) return st;
  if ((k == nullptr) != (k_out == nullptr) || (v == nullptr) != (v_out == nullptr) ||
      (k_pos == nullptr) != (pos_out == nullptr))
    return fail(TRI_ERR_INVALID_ARGUMENT, "k/k_out, v/v_out and k_pos/pos_out come in pairs");
  if (p.kept == 0) return TRI_OK;
  if (!scores || !kept_idx)
    return fail(TRI_ERR_INVALID_ARGUMENT, "scores and kept_idx must be non-NULL");
  if ((k && (!aligned16(k) || !aligned16(k_out))) || (v && (!aligned16(v) || !aligned16(v_out))))
    return fail(TRI_ERR_INVALID_ARGUMENT, "K/V buffers must be 16-byte aligned");
  if (!workspace || workspace_bytes < p.select_bytes)
    return fail(TRI_ERR_WORKSPACE, "workspace missing or smaller than tri_workspace_bytes_layers()");
  const hipError_t e = run_select_compact(p, scores, k, v, k_pos, kept_idx, k_out, v_out, pos_out,
                                          (char*)workspace, (hipStream_t)stream);
  if (e != hipSuccess)
    return fail(TRI_ERR_HIP, std::string("select_compact_layers: ") + hipGetErrorString(e));
  return TRI_OK;
}

// ---------------------------------------------------------------------------
// Paged pools
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

// A tri_kv_pages descriptor as the kernels take it, after checking it.
tri_status to_pages(const tri_kv_pages* d, const tri_shape* sh, tri::Pages& pg, const char* what) {
  const std::string w(what);
  if (!d) return fail(TRI_ERR_INVALID_ARGUMENT, w + " is NULL");
  if (!d->page_table) return fail(TRI_ERR_INVALID_ARGUMENT, w + ".page_table is NULL");
  const int32_t P = d->page_size;
  if (P < 1 || P > 65536 || (P & (P - 1)) != 0)
    return fail(TRI_ERR_INVALID_ARGUMENT, w + ".page_size must be a power of two in [1, 65536]");
  if (d->max_pages < 1 || d->num_pages < 1)
    return fail(TRI_ERR_INVALID_ARGUMENT, w + ".max_pages and .num_pages must be >= 1");
  if (d->page_stride < 0 || d->token_stride < 0 || d->head_stride < 0 || d->layer_stride < 0)
    return fail(TRI_ERR_INVALID_ARGUMENT, w + " strides must be >= 0");
  // the largest row any (layer, head, page, slot) can name, times d, fits int64
  const double top = (double)(sh->num_layers - 1) * d->layer_stride +
                     (double)(sh->num_kv_heads - 1) * d->head_stride +
                     (double)(d->num_pages - 1) * d->page_stride + (double)(P - 1) * d->token_stride;
  if ((top + 1.0) * sh->head_dim * 2.0 > 9.0e18)
    return fail(TRI_ERR_UNSUPPORTED, w + " spans more rows than 64-bit offsets hold");
  pg.table = d->page_table;
  pg.max_pages = d->max_pages;
  pg.num_pages = d->num_pages;
  int shift = 0;
  while ((1 << shift) < P) ++shift;
  pg.page_shift = shift;
  pg.hkv = sh->num_kv_heads;
  pg.page_stride = d->page_stride;
  pg.token_stride = d->token_stride;
  pg.head_stride = d->head_stride;
  pg.layer_stride = d->layer_stride;
  return TRI_OK;
}

}  // namespace

extern "C" {

size_t tri_workspace_bytes_paged(const tri_shape* shape, int32_t num_seqs, const int64_t* cu_len,
                                 int32_t page_size, int32_t n_offsets, int32_t reduce) {
  if (page_size < 1 || page_size > 65536 || (page_size & (page_size - 1)) != 0) {
    fail(TRI_ERR_INVALID_ARGUMENT, "page_size must be a power of two in [1, 65536]");
    return 0;
  }
  OffsetMode om;
  std::vector<double> zeros;  // offsets are only counted here
  if (n_offsets != 0) {
    if (reduce != TRI_REDUCE_MEAN && reduce != TRI_REDUCE_MAX) {
      fail(TRI_ERR_INVALID_ARGUMENT, "reduce must be TRI_REDUCE_MEAN or TRI_REDUCE_MAX");
      return 0;
    }
    if (n_offsets < 1 || n_offsets > tri::kMaxOffsets) {
      fail(TRI_ERR_INVALID_ARGUMENT, "n_offsets must be 0 (built-in set) or in [1, 4096]");
      return 0;
    }
    zeros.assign(n_offsets, 0.0);
    om.host = zeros.data();
    om.n = n_offsets;
    om.max = reduce == TRI_REDUCE_MAX;
  }
  // the path a paged call takes depends only on the page size
  static const int32_t kNoTable = 0;
  tri::Pages pg;
  pg.table = &kNoTable;
  pg.max_pages = 0x7fffffff;
  pg.num_pages = 1;
  while ((1 << pg.page_shift) < page_size) ++pg.page_shift;
  PlanLayout lay;
  lay.in_pages = &pg;
  Plan p;
  if (make_plan(shape, num_seqs, cu_len, nullptr, nullptr, p, om, lay) != TRI_OK) return 0;
  return p.score_bytes > p.select_bytes ? p.score_bytes : p.select_bytes;
}

tri_status tri_score_paged(const tri_shape* shape, int32_t num_seqs, const int64_t* cu_len,
                           const int32_t* cur_pos, const tri_kv_pages* pages,
                           const uint16_t* k_pool, const float* q_centre, const float* q_absmean,
                           const float* q_R, const double* offsets, int32_t n_offsets,
                           int32_t reduce, float* scores, float* raw_scores, double* head_stats,
                           void* workspace, size_t workspace_bytes, void* stream) {
  tri_status st = check_shape(shape);
  if (st != TRI_OK) return st;
  tri::Pages pg;
  st = to_pages(pages, shape, pg, "pages");
  if (st != TRI_OK) return st;
  OffsetMode om;
  if (offsets) {
    if (reduce != TRI_REDUCE_MEAN && reduce != TRI_REDUCE_MAX)
      return fail(TRI_ERR_INVALID_ARGUMENT, "reduce must be TRI_REDUCE_MEAN or TRI_REDUCE_MAX");
    om.host = offsets;
    om.n = n_offsets;
    om.max = reduce == TRI_REDUCE_MAX;
  }
  return score_impl(shape, num_seqs, cu_len, cur_pos, k_pool, q_centre, q_absmean, q_R, om,
                    scores, raw_scores, head_stats, workspace, workspace_bytes, stream, &pg);
}

tri_status tri_select_compact_paged(const tri_shape* shape, int32_t num_seqs,
                                    const int64_t* cu_len, const int32_t* budget,
                                    const float* scores, const tri_kv_pages* in_pages,
                                    const uint16_t* k_pool, const uint16_t* v_pool,
                                    const int32_t* pos_pool, int32_t* kept_idx,
                                    const tri_kv_pages* out_pages, uint16_t* k_out_pool,
                                    uint16_t* v_out_pool, int32_t* pos_out_pool, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  tri_status st = check_shape(shape);
  if (st != TRI_OK) return st;
  if (num_seqs > 0 && !budget) return fail(TRI_ERR_INVALID_ARGUMENT, "budget is NULL");
  if ((k_pool == nullptr) != (k_out_pool == nullptr) ||
      (v_pool == nullptr) != (v_out_pool == nullptr) ||
      (pos_pool == nullptr) != (pos_out_pool == nullptr))
    return fail(TRI_ERR_INVALID_ARGUMENT,
                "k/k_out, v/v_out and pos/pos_out pools come in pairs");
  const bool rows = k_pool || v_pool || pos_pool;
  tri::Pages in_pg, out_pg;
  PlanLayout lay;
  if (rows) {
    st = to_pages(in_pages, shape, in_pg, "in_pages");
    if (st != TRI_OK) return st;
    st = to_pages(out_pages, shape, out_pg, "out_pages");
    if (st != TRI_OK) return st;
    lay.in_pages = &in_pg;
    lay.out_pages = &out_pg;
  }
  Plan p;
  st = make_plan(shape, num_seqs, cu_len, nullptr, budget, p, OffsetMode(), lay);
  if (st != TRI_OK) return st;
  if (p.kept == 0) return TRI_OK;
  if (!scores || !kept_idx)
    return fail(TRI_ERR_INVALID_ARGUMENT, "scores and kept_idx must be non-NULL");
  if ((k_pool && (!aligned16(k_pool) || !aligned16(k_out_pool))) ||
      (v_pool && (!aligned16(v_pool) || !aligned16(v_out_pool))))
    return fail(TRI_ERR_INVALID_ARGUMENT, "K/V pools must be 16-byte aligned");
  if (!workspace || workspace_bytes < p.select_bytes)
    return fail(TRI_ERR_WORKSPACE, "workspace missing or smaller than tri_workspace_bytes()");
  const hipError_t e = run_select_compact(p, scores, k_pool, v_pool, pos_pool, kept_idx,
                                          k_out_pool, v_out_pool, pos_out_pool, (char*)workspace,
                                          (hipStream_t)stream);
  if (e != hipSuccess)
    return fail(TRI_ERR_HIP, std::string("select_compact_paged: ") + hipGetErrorString(e));
  return TRI_OK;
}

}  // extern "C"
