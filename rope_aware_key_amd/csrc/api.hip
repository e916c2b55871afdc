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

// ---------------------------------------------------------------------------
// Pinned staging for the per-call sequence plan.  One ring per device,
// allocated on first use; a slot is reused only after the copy that last
// read it has completed (its event).
// ---------------------------------------------------------------------------
constexpr int kSlots = 16;
constexpr size_t kSlotBytes = 320 * 1024;  // 8192 sequences of 40-byte plan entries

struct Staging {
  std::mutex mu;
  char* host = nullptr;
  hipEvent_t ev[kSlots] = {};
  bool used[kSlots] = {};
  int next = 0;
};

std::mutex g_staging_mu;
std::map<int, Staging*> g_staging;

hipError_t get_staging(Staging** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_staging_mu);
  auto it = g_staging.find(dev);
  if (it != g_staging.end()) {
    *out = it->second;
    return hipSuccess;
  }
  Staging* st = new Staging();
  e = hipHostMalloc((void**)&st->host, kSlots * kSlotBytes, hipHostMallocDefault);
  if (e != hipSuccess) {
    delete st;
    return e;
  }
  for (int i = 0; i < kSlots; ++i) {
    e = hipEventCreateWithFlags(&st->ev[i], hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  g_staging[dev] = st;
  *out = st;
  return hipSuccess;
}

// Copy `bytes` of host data to `dst` on `stream` through a pinned slot.
hipError_t upload(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  Staging* st = nullptr;
  hipError_t e = get_staging(&st);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(st->mu);
  const int slot = st->next;
  st->next = (st->next + 1) % kSlots;
  if (st->used[slot]) {
    e = hipEventSynchronize(st->ev[slot]);
    if (e != hipSuccess) return e;
  }
  char* h = st->host + (size_t)slot * kSlotBytes;
  std::memcpy(h, src, bytes);
  e = hipMemcpyAsync(dst, h, bytes, hipMemcpyHostToDevice, stream);
  if (e != hipSuccess) return e;
  e = hipEventRecord(st->ev[slot], stream);
  st->used[slot] = true;
  return e;
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
// its output prefix); this is the public layout.  Strided: every unit of
// sequence s at row0[s] + (l*Hkv + g)*stride, so units can grow in place
// (the decode cache).
struct PlanLayout {
  int64_t in_stride = 0, out_stride = 0;
  const int64_t* in_row0 = nullptr;   // [S] host, strided input only
  const int64_t* out_row0 = nullptr;  // [S] host, strided output only
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
         off_apack = 0, off_raw = 0, off_offsets = 0, off_ustats = 0;
  int64_t n_units = 0, n_stat_slots = 0;
  int chunk = 0;  // keys per score ticket
  bool fused = false;
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
  if ((size_t)S * sizeof(SeqInfo) > kSlotBytes)
    return fail(TRI_ERR_UNSUPPORTED, "too many sequences in one call (max 8192)");
  p.S = S;
  p.L = sh->num_layers;
  p.Hkv = sh->num_kv_heads;
  p.Hq = sh->num_q_heads;
  p.G = p.Hq / p.Hkv;
  p.d = sh->head_dim;
  p.F = p.d / 2;
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
  p.fused = !om.max && tri::fused_supported(p.d) &&
            (longest + tri::fused_chunk_keys(p.G) - 1) / tri::fused_chunk_keys(p.G) <=
                tri::kFusedMaxUnitChunks;
  p.chunk = p.fused ? tri::fused_chunk_keys(p.G) : tri::kScoreChunk;
  for (int s = 0; s < S; ++s) {
    const int64_t n = cu_len[s + 1] - cu_len[s];
    if (n < 0) return fail(TRI_ERR_INVALID_ARGUMENT, "cu_len must be non-decreasing");
    if (n > (int64_t)0x7fffffff / 2) return fail(TRI_ERR_UNSUPPORTED, "sequence too long");
    SeqInfo& si = p.seqs[s];
    si.row_base = lay.in_stride ? lay.in_row0[s] : LH * cu_len[s];
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
    si.out_base = lay.out_stride ? lay.out_row0[s] : LH * out_acc;
    si.out_stride = (int32_t)(lay.out_stride ? lay.out_stride : b);
    if (b > si.out_stride) return fail(TRI_ERR_INVALID_ARGUMENT, "budget above the output stride");
    p.total_rows = std::max(p.total_rows, si.row_base + LH * si.in_stride);
    p.total_out = std::max(p.total_out, si.out_base + LH * si.out_stride);
    p.keys += LH * n;
    p.kept += LH * b;
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
  p.off_ctrl = take((size_t)tri::kCtrlHeader * sizeof(uint32_t));
  // The fused path keeps raw scores on chip; the generic path spills them.
  p.off_apack = take(om.max ? tri::max_offsets_operand_bytes(p.d, p.G, p.mp, p.n_units, p.tickets)
                            : tri::fused_operand_bytes(p.d, p.n_units));
  p.off_ustats = take(p.fused ? 0 : (size_t)p.n_units * p.G * 2 * sizeof(double));
  p.off_raw = take(p.fused ? 0 : (size_t)p.total_rows * p.G * sizeof(float));
  p.score_bytes = off;
  p.select_bytes = after_seq;
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

tri_status tri_calibrate(const tri_shape* shape, const uint16_t* q, const int32_t* q_pos,
                         int64_t n_samples, float* q_centre, float* q_absmean, float* q_R,
                         void* stream) {
  tri_status st = check_shape(shape);
  if (st != TRI_OK) return st;
  if (n_samples < 1) return fail(TRI_ERR_INVALID_ARGUMENT, "n_samples must be >= 1");
  if (!q || !q_centre || !q_absmean || !q_R)
    return fail(TRI_ERR_INVALID_ARGUMENT, "q and every output must be non-NULL");
  if (((uintptr_t)q & 3u) != 0) return fail(TRI_ERR_INVALID_ARGUMENT, "q must be 4-byte aligned");
  hipError_t e = tri::launch_calibrate(shape->num_layers, shape->num_q_heads, shape->head_dim,
                                       shape->rope_theta, q, q_pos, n_samples, q_centre,
                                       q_absmean, q_R, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TRI_ERR_HIP, std::string("calibrate: ") + hipGetErrorString(e));
  return TRI_OK;
}

}  // extern "C"

namespace {

tri_status score_impl(const tri_shape* shape, int32_t num_seqs, const int64_t* cu_len,
                      const int32_t* cur_pos, const uint16_t* k, const float* q_centre,
                      const float* q_absmean, const float* q_R, const OffsetMode& om,
                      float* scores, float* raw_scores, double* head_stats, void* workspace,
                      size_t workspace_bytes, void* stream) {
  Plan p;
  tri_status st = make_plan(shape, num_seqs, cu_len, cur_pos, nullptr, p, om);
  if (st != TRI_OK) return st;
  if (num_seqs > 0 && !cur_pos) return fail(TRI_ERR_INVALID_ARGUMENT, "cur_pos is NULL");
  if (p.keys == 0) return TRI_OK;
  if (!k || !q_centre || !q_absmean || !q_R || !scores)
    return fail(TRI_ERR_INVALID_ARGUMENT, "k, statistics and scores must be non-NULL");
  if (!aligned16(k)) return fail(TRI_ERR_INVALID_ARGUMENT, "k must be 16-byte aligned");
  const size_t need = (raw_scores || p.fused) ? p.off_raw : p.score_bytes;
  if (!workspace || workspace_bytes < need)
    return fail(TRI_ERR_WORKSPACE, "workspace missing or smaller than tri_workspace_bytes()");
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  SeqInfo* dseq = (SeqInfo*)(ws + p.off_seq);
  double* doff = om.host ? (double*)(ws + p.off_offsets) : nullptr;
  hipError_t e = upload(dseq, p.seqs.data(), p.seqs.size() * sizeof(SeqInfo), s);
  if (e == hipSuccess && doff) e = upload(doff, om.host, (size_t)om.n * sizeof(double), s);
  if (e == hipSuccess)
    e = tri::launch_prologue(p.L, p.Hq, p.d, shape->rope_theta, p.S, dseq, q_centre, q_absmean,
                             q_R, doff, om.n, !om.max, (double2*)(ws + p.off_P),
                             (float*)(ws + p.off_W), (double2*)(ws + p.off_E),
                             (uint32_t*)(ws + p.off_ctrl), (double*)(ws + p.off_stats),
                             p.n_stat_slots, s);
  float* raw = raw_scores ? raw_scores : (float*)(ws + p.off_raw);
  if (e != hipSuccess) {
  } else if (om.max) {
    e = tri::launch_score_max(dseq, p.S, p.L, p.Hkv, p.G, p.d, om.n, p.mp, shape->rope_theta,
                              (int)p.tickets, (const double2*)(ws + p.off_P),
                              (const float*)(ws + p.off_W), (const double2*)(ws + p.off_E), doff,
                              ws + p.off_apack, k, raw, (double*)(ws + p.off_stats),
                              (double*)(ws + p.off_ustats), scores, head_stats, s);
  } else if (p.fused) {
    e = tri::launch_score_fused(dseq, p.S, p.L, p.Hkv, p.G, p.d, p.chunk, (int)p.tickets,
                                (const double2*)(ws + p.off_P), (const float*)(ws + p.off_W),
                                (const double2*)(ws + p.off_E), ws + p.off_apack, k,
                                (double*)(ws + p.off_stats), (uint32_t*)(ws + p.off_ctrl),
                                scores, raw_scores, head_stats, s);
  } else {
    e = tri::launch_score(dseq, p.S, p.L, p.Hkv, p.G, p.d, (int)p.tickets,
                          (const double2*)(ws + p.off_P), (const float*)(ws + p.off_W),
                          (const double2*)(ws + p.off_E), k, raw, (double*)(ws + p.off_stats),
                          (double*)(ws + p.off_ustats), scores, head_stats, s);
  }
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
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  SeqInfo* dseq = (SeqInfo*)(ws + p.off_seq);
  hipError_t e = upload(dseq, p.seqs.data(), p.seqs.size() * sizeof(SeqInfo), s);
  const int LH = p.L * p.Hkv;
  if (e == hipSuccess) e = tri::launch_select(dseq, p.S, LH, p.max_n, scores, kept_idx, s);
  if (e == hipSuccess && (k_out || v_out || pos_out))
    e = tri::launch_compact(dseq, p.S, LH, p.d, p.max_b, kept_idx, k, v, k_pos, k_out, v_out,
                            pos_out, s);
  if (e != hipSuccess)
    return fail(TRI_ERR_HIP, std::string("select_compact: ") + hipGetErrorString(e));
  return TRI_OK;
}

}  // extern "C"
