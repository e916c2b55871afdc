// Internal types shared by the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tri {

// Per-sequence plan entry, built on the host from cu_len / cur_pos / budget
// and uploaded once per call.
struct SeqInfo {
  int64_t row_base;    // first input row of the sequence (packed: L*Hkv*cu_len[s])
  int64_t out_base;    // first output row (packed: L*Hkv*cu_b[s], cu_b = prefix of b)
  int32_t n;           // keys per unit
  int32_t b;           // kept keys per unit, min(budget, n)
  int32_t p_q;         // current query position
  int32_t chunk_base;  // first score ticket of the sequence
  int32_t in_stride;   // input rows from one unit of the sequence to the next (packed: n)
  int32_t out_stride;  // output rows from one unit to the next (packed: b)
};
static_assert(sizeof(SeqInfo) == 40, "SeqInfo layout");

// Keys per score work-group ticket.
constexpr int kScoreChunk = 1024;

// Score control block (uint32 words): [0] ticket counter, [1] error flag.
constexpr int kCtrlHeader = 64;

// Bit pattern (a NaN no arithmetic produces) that marks a published
// statistics slot as not yet written.
constexpr uint64_t kStatSentinel = 0x7ff4dead0000beefull;
constexpr int kMaxGroup = 16;
constexpr int kMaxHeadDim = 256;
// Most offsets in a caller-given offset set.
constexpr int kMaxOffsets = 4096;
// Dynamic LDS of the max-over-offsets score kernel (it has no static LDS):
// the whole 160 KB of a gfx950 CU.
constexpr size_t kMaxOffsetsLds = 160 * 1024;

// Paged K/V/position pool (tutorial page, deployment paragraph: paged KV
// management as in vLLM's PagedAttention).  Token i of unit (s, l, g) is
// pool row
//   l*layer_stride + g*head_stride + page*page_stride + (i % P)*token_stride,
// page = table[s*max_pages + i / P], P = 1 << page_shift; a K or V row is d
// elements, a position row one.  Page ids outside [0, num_pages) are
// clamped into it, so a bad table never reads or writes outside the pool.
// table == NULL means the packed layout.
struct Pages {
  const int32_t* table = nullptr;
  int32_t max_pages = 0, num_pages = 0, page_shift = 0;
  int32_t hkv = 1;  // KV heads: unit lg of a sequence is layer lg / hkv, head lg % hkv
  int64_t page_stride = 0, token_stride = 0, head_stride = 0, layer_stride = 0;
};

// Pool row of slot 0 of logical page j of unit (s, l, g).
__device__ __forceinline__ int64_t page_row0(const Pages& pg, int s, int l, int g, int j) {
  int p = pg.table[(int64_t)s * pg.max_pages + j];
  p = p < 0 ? 0 : (p >= pg.num_pages ? pg.num_pages - 1 : p);
  return (int64_t)l * pg.layer_stride + (int64_t)g * pg.head_stride + (int64_t)p * pg.page_stride;
}

__device__ __forceinline__ int64_t paged_row(const Pages& pg, int s, int l, int g, int i) {
  const int j = i >> pg.page_shift;
  return page_row0(pg, s, l, g, j) + (int64_t)(i - (j << pg.page_shift)) * pg.token_stride;
}

__device__ __forceinline__ int64_t paged_row_lg(const Pages& pg, int s, int lg, int i) {
  return paged_row(pg, s, lg / pg.hkv, lg % pg.hkv, i);
}

// RoPE pair layouts.  Band f of a d-vector is (x_{2f}, x_{2f+1})
// (interleaved, the talk page's rotation equation) or (x_f, x_{f+d/2})
// (half split: a storage layout the pages print no formula for, supported
// as a reading; each pair still rotates by the printed matrix).
__host__ __device__ __forceinline__ int elem_band(int e, int d, bool half) {
  return half ? (e < (d >> 1) ? e : e - (d >> 1)) : (e >> 1);
}
// 0: element e is the real part of its band, 1: the imaginary part.
__host__ __device__ __forceinline__ int elem_part(int e, int d, bool half) {
  return half ? (e >= (d >> 1)) : (e & 1);
}

// The MFMA kernels hand lane (m, q) the key elements 32 st + 8q .. +7 of
// step st as four 32-bit words.  The norm term needs one magnitude per
// (step, word) slot; slot_band names the band it stands for.  Interleaved:
// word u holds band 16 st + 4q + u whole.  Half split (an even number of
// steps): the band's two parts sit in word u of steps st and st + steps/2,
// the low halves forming band 32 st + 8q + 2u and the high halves band
// 32 st + 8q + 2u + 1; slot (st, u) takes the first for st < steps/2 and
// the second for the rest.
__host__ __device__ __forceinline__ int slot_band(int st, int q, int u, int steps, bool half) {
  if (!half) return 16 * st + 4 * q + u;
  const int h = steps >> 1;
  return st < h ? 32 * st + 8 * q + 2 * u : 32 * (st - h) + 8 * q + 2 * u + 1;
}

__device__ __forceinline__ uint32_t uint4_word(const uint4& v, int u) {
  return u == 0 ? v.x : u == 1 ? v.y : u == 2 ? v.z : v.w;
}

// The two bf16 parts of slot (st, u)'s band as one bf16 pair (real, imag),
// from the lane's key words kw[0 .. STEPS-1].
template <int STEPS, bool HALF>
__device__ __forceinline__ uint32_t slot_pair(const uint4 (&kw)[STEPS], int st, int u) {
  if (!HALF) return uint4_word(kw[st], u);
  constexpr int H = STEPS / 2;
  // one v_perm_b32 each: bytes {0,1} of a and b, or bytes {2,3} (selector
  // bytes 0-3 pick from a, 4-7 from b)
  if (st < H)
    return __builtin_amdgcn_perm(uint4_word(kw[st + H], u), uint4_word(kw[st], u), 0x05040100u);
  return __builtin_amdgcn_perm(uint4_word(kw[st], u), uint4_word(kw[st - H], u), 0x07060302u);
}

// Largest s with seqs[s].chunk_base <= t (sequences with no tickets share
// chunk_base with their successor, so the search lands on the owner).
__device__ __forceinline__ int find_seq_by_ticket(const SeqInfo* seqs, int S, int t) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (seqs[mid].chunk_base <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Largest s with seqs[s].out_base <= r among sequences that have output rows.
__device__ __forceinline__ int find_seq_by_out_row(const SeqInfo* seqs, int S, int64_t r) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (seqs[mid].out_base <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Launchers (defined in the .hip files).  Each returns the hipError_t of the
// launch.
// Calibration scratch: the (sample, band) phasor table and per-chunk sums.
size_t calibrate_workspace_bytes(int L, int Hq, int d, int64_t n_samples);
hipError_t launch_calibrate(int L, int Hq, int d, double theta, bool half, const uint16_t* q,
                            const int32_t* q_pos, int64_t n_samples, float* centre,
                            float* absmean, float* R, void* workspace, hipStream_t st);

// 32-bit words one launch carries in its arguments (2560 bytes).
constexpr int kArgWords = 640;
struct ArgWords {
  uint32_t w[kArgWords];
};

// offsets: device array of n_offsets distances, or NULL for the default set
// {2^0, ..., 2^16}.  fold: P = E[q] * mean_delta exp(i omega delta) when
// true, P = E[q] when false (the offsets are applied later, per row).
// plan_host: the S sequences' host plan when it fits one launch's argument
// words (S * 40 <= 2560 bytes): the prologue then writes it to seqs itself
// and reads the query positions from its arguments; NULL when the plan was
// uploaded to seqs before.
hipError_t launch_prologue(int L, int Hq, int d, double theta, int S,
                           const SeqInfo* seqs, const SeqInfo* plan_host,
                           const float* q_centre, const float* q_absmean, const float* q_R,
                           const double* offsets, int n_offsets, bool fold, double2* P,
                           float* W, double2* E, uint32_t* ctrl, int64_t n_ctrl,
                           double* stat_slots, int64_t n_stat_slots, hipStream_t st);

bool fused_supported(int d, bool half);
// Keys per ticket of the fused path for a GQA group of G heads.
int fused_chunk_keys(int G, int d);
// Bound on the fused kernel's wait for another work-group's chunk statistics
// (polls per slot; default 2^22); returns the previous bound.
uint32_t set_fused_wait_limit(uint32_t polls);
unsigned long long* set_fused_phase_buffer(unsigned long long* buf);
// Most chunks one unit may have on the fused path.  Its waits need more
// than half that many work-groups resident; the planner also caps a unit at
// the device's resident work-groups (fused_resident_groups), twice that
// margin.
constexpr int kFusedMaxUnitChunks = 384;
// Fused-kernel work-groups the current device holds at once for a shape
// (occupancy x CUs), or -1 when no device answers; a positive override
// (test hook) replaces the query.  Returns / sets process-wide values.
int fused_resident_groups(int d, bool half, bool paged, int G);
int set_fused_resident_override(int groups);
// Workspace bytes of the fused path's packed MFMA operands.
size_t fused_operand_bytes(int d, int64_t units);

// What the fused path's preparation kernel needs (it stands in for the
// prologue there: the averaged score, offsets folded into C_f): the
// calibration tables, the offsets (NULL: {2^0..2^16}), the plan (plan_host:
// carried in the launch's arguments and written to seqs; NULL: already in
// seqs), and the control words and statistics slots to reset.
struct PrepArgs {
  double theta;
  int Hq;
  const float* q_centre;
  const float* q_absmean;
  const float* q_R;
  const double* offsets;
  int n_offsets;
  const SeqInfo* plan_host;
  int64_t n_ctrl;
  int64_t n_stat_slots;
};

// Fused MFMA score path (head_dim % 32 == 0, the averaged score), with no
// prologue: one preparation kernel zeroes ctrl, resets chunk_stats ([tickets]
// [G][2] fp64 sum and sum of squares) to kStatSentinel, writes the plan and
// packs the operands into apack; then the fused kernel.
hipError_t launch_score_fused(const SeqInfo* seqs, int S, int L, int Hkv, int G, int d, int ch,
                              int total_tickets, void* apack, const uint16_t* k,
                              double* chunk_stats, uint32_t* ctrl, float* scores, float* raw,
                              double* head_stats, bool half, const Pages& pg,
                              const PrepArgs& prep, hipStream_t st);

// unit_stats: [units][G][2] fp64 scratch for the per-unit (mu, 1/sigma).
hipError_t launch_score(const SeqInfo* seqs, int S, int L, int Hkv, int G, int d,
                        int total_tickets, const double2* P, const float* W,
                        const double2* E, const uint16_t* k, float* raw,
                        double* chunk_stats, double* unit_stats, float* scores,
                        double* head_stats, bool half, const Pages& pg, hipStream_t st);

// z pass of the generic path: merges the (count, mean, M2) tickets of each
// unit into unit_stats ([units][G][2]: mu, 1/sigma; head_stats gets mu,
// sigma), then writes max_h z per key.
hipError_t launch_zmax(const SeqInfo* seqs, int S, int L, int Hkv, int G, int total_tickets,
                       const float* raw, const double* chunk_stats, double* unit_stats,
                       float* scores, double* head_stats, hipStream_t st);

// Max-over-offsets score path.  Accumulator row 4q+i of a 16-row tile is
// held by lanes q (MFMA layout), so rows are assigned to the four lane
// slots q: with spread == 1 head h of a pass lives in slot h % 4 (its Dp
// rows, Dp = |D| rounded up to 4, take Dp/4 consecutive tiles of that
// slot); with spread == 4 (one head's rows exceed the LDS budget) a head
// takes all four slots of Dp/16 tiles (Dp rounded up to 16) and the slots
// are merged with two cross-lane maxima.  hp heads per pass, npass passes
// over the keys, ptiles = nk * tiles_per_head tiles per pass with nk the
// number of head rounds (hp/4 rounded up, or hp).
struct MaxOffsetsPlan {
  bool ok = false;
  int spread = 1, Dp = 0, tiles_per_head = 0, hp = 0, nk = 0, npass = 0, ptiles = 0;
};
MaxOffsetsPlan plan_max_offsets(int d, int G, int n_offsets);
// Operand rows, norm weights and per-wave moment sums of the max path.
size_t max_offsets_operand_bytes(int d, int G, int nD, const MaxOffsetsPlan& mp, int64_t units,
                                 int64_t tickets);
// Generic tickets (kScoreChunk keys); raw: [rows][G] fp32 spill; chunk_stats
// as the generic path; P from the prologue with fold = false.
hipError_t launch_score_max(const SeqInfo* seqs, int S, int L, int Hkv, int G, int d, int nD,
                            const MaxOffsetsPlan& mp, double theta, int total_tickets,
                            const double2* P, const float* W, const double2* E,
                            const double* offsets, void* operands, const uint16_t* k,
                            float* raw, double* chunk_stats, double* unit_stats, float* scores,
                            double* head_stats, bool half, const Pages& pg,
                            hipStream_t st);

// Decode-loop driver: where one appended token of sequence s goes (row of
// unit 0; unit lg at row0 + lg*stride) and its position.
struct DecodeItem {
  int64_t row0;
  int32_t pos;
  int32_t pad;
};
static_assert(sizeof(DecodeItem) == 16, "DecodeItem layout");
// Sequences whose append items travel in the kernel arguments (16 bytes each).
constexpr int kAppendInline = 128;
// host_items: host memory, copied into the launch (S <= kAppendInline).
hipError_t launch_append_inline(const DecodeItem* host_items, int S, int LH, int d,
                                int64_t stride, const uint16_t* k_new, const uint16_t* v_new,
                                uint16_t* k, uint16_t* v, int32_t* pos, hipStream_t st);
hipError_t launch_append(const DecodeItem* items, int S, int LH, int d, int64_t stride,
                         const uint16_t* k_new, const uint16_t* v_new, uint16_t* k, uint16_t* v,
                         int32_t* pos, hipStream_t st);
// Scores of the first `sink` and last `recent` keys of every pruned unit
// (b < n) of the plan's sequences -> +inf.
hipError_t launch_protect(const SeqInfo* seqs, int S, int LH, int sink, int recent,
                          float* scores, hipStream_t st);

// Writes `bytes` (a multiple of 4) of host memory to dst (device) through
// kernel arguments: no staging memory, host data free once this returns.
hipError_t launch_write_args(void* dst, const void* host, size_t bytes, hipStream_t st);

// Read-bandwidth probe over bytes (a multiple of 16) of src; XORs into *sink.
hipError_t launch_stream_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t st);

// Reconstruction diagnostic (d % 32 == 0): per-(layer, query head) Pearson
// r of the trig series against the direct logits; partial is
// trig_corr_workspace_bytes() of scratch.
size_t trig_corr_workspace_bytes(int L, int Hq, int64_t n_q);
hipError_t launch_trig_corr(int L, int Hq, int Hkv, int d, int64_t n_q, int64_t n_k, double theta,
                            bool half,
                            const uint16_t* q, const int32_t* q_pos, const uint16_t* k,
                            const int32_t* k_pos, const float* q_centre, double* partial,
                            double* r, hipStream_t st);

// split_ws: split_select_bytes(units, max_n) bytes of device scratch (only
// read when max_n is above what one work-group's select holds)
size_t split_select_bytes(int64_t units, int max_n);
hipError_t launch_select(const SeqInfo* seqs, int S, int LH, int max_n, const float* scores,
                         int32_t* kept_idx, void* split_ws, hipStream_t st);

hipError_t launch_compact(const SeqInfo* seqs, int S, int LH, int d, int max_b,
                          const int32_t* kept_idx, const uint16_t* k, const uint16_t* v,
                          const int32_t* k_pos, uint16_t* k_out, uint16_t* v_out,
                          int32_t* pos_out, const Pages& in_pg, const Pages& out_pg,
                          hipStream_t st);

// Select, then the gathers asked for (any of k_out, v_out, pos_out); for
// units of 4096 < n <= 32768 keys one kernel does both, one work-group per
// unit, so that selections overlap other units' copies.  plan_host: the
// host copy of the S-entry plan, written to seqs first (when the first
// units are selected by a launch of their own and the plan fits its
// arguments, that launch carries and writes it); NULL when seqs already
// holds the plan.
hipError_t launch_select_compact(SeqInfo* seqs, const SeqInfo* plan_host, int S, int LH, int d,
                                 int max_n, int max_b, const float* scores, int32_t* kept_idx,
                                 void* split_ws, const uint16_t* k, const uint16_t* v,
                                 const int32_t* k_pos, uint16_t* k_out, uint16_t* v_out,
                                 int32_t* pos_out, const Pages& in_pg, const Pages& out_pg,
                                 hipStream_t st);

}  // namespace tri
