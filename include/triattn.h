/*
 * triattn.h -- C ABI of the TriAttention KV-cache pruning library (gfx950).
 *
 * The library scores every cached key with the TriAttention importance
 * estimate, keeps the top-B keys of each (sequence, layer, KV head) and
 * compacts K, V and positions in their original order.  All work runs as
 * hand-written HIP kernels on the stream the caller passes.
 *
 * Sources of the definitions (page title, then section or equation):
 *  - qingkeai.online talk page "聊聊 TriAttention: 面向长上下文推理的三角级数式
 *    KV Cache 压缩": RoPE rotation equation; RoPE logit decomposition;
 *    S_trig equation; S_norm equation with R_f = |E[q_f]| / E[|q_f|];
 *    S = S_trig + S_norm and its mean over the offsets D = {1, 2, ..., 2^16};
 *    keep the top-B keys.
 *  - hyper.ai summary of arXiv 2604.04921, section "方法": average over
 *    future query positions; for grouped-query attention, z-score each query
 *    head's scores, then take the max over the group; prune every 128
 *    generated tokens.
 *  - shibing624 blog review of TriAttention, section "具体操作分三步",
 *    step 1: statistics are calibrated offline, once, from ~10K tokens.
 *  - jaedaily.cn KV-cache compression tutorial, eviction step: the top-k
 *    indices are kept, sorted to keep the time order, and keys and values
 *    are gathered with them.
 *
 * Conventions shared by every call
 *  - d = head_dim, F = d/2 RoPE bands.  Band f of a vector x is the pair
 *    (x[2f], x[2f+1]) (interleaved), rotated at position p by omega_f * p,
 *    omega_f = rope_theta^(-2f/d).
 *  - G = num_q_heads / num_kv_heads; query heads [g*G, (g+1)*G) read KV
 *    head g.
 *  - A "unit" is one (sequence s, layer l, KV head g).  Packed unit-major
 *    layout: with n_s = cu_len[s+1] - cu_len[s], the rows of sequence s
 *    start at row L*Hkv*cu_len[s]; unit (l, g) holds the n_s consecutive rows
 *    starting (l*Hkv + g)*n_s after that.  Within a unit, positions must
 *    increase strictly (row order == time order).
 *  - bf16 values are passed as their raw 16-bit patterns (uint16_t).
 *  - Pointers marked [host] are host memory, read before the call returns.
 *    Every other pointer is device memory on the current HIP device.
 *  - stream is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous on it; outputs are ready once the stream reaches the end
 *    of the call.
 *  - The caller owns every buffer.  Outputs must not alias inputs.  K/V row
 *    pointers must be 16-byte aligned and d*2 a multiple of 16.
 *  - Argument errors return before any device work is queued.  A HIP error
 *    during launch returns TRI_ERR_HIP.  tri_last_error() gives a message
 *    for the last failing call of the calling thread.
 *  - Host arrays reach the device in the arguments of small copy launches
 *    (2560 bytes each): nothing on the host outlives the call and no
 *    staging memory is held.  A call's device work is kernel launches
 *    only, so tri_score, tri_score_offsets, tri_score_paged,
 *    tri_select_compact* and tri_score_noalloc may be captured into a HIP
 *    graph and replayed (the plan is fixed at capture).  The decode-loop
 *    calls may allocate and return TRI_ERR_UNSUPPORTED on a capturing
 *    stream.
 */
#ifndef TRIATTN_H
#define TRIATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TRI_OK = 0,
  TRI_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, bad alignment   */
  TRI_ERR_UNSUPPORTED = 2,      /* shape outside what the kernels handle   */
  TRI_ERR_WORKSPACE = 3,        /* workspace missing or too small          */
  TRI_ERR_HIP = 4               /* HIP runtime error while queueing work   */
} tri_status;

/*
 * RoPE pair layout of every q/k row (TRI_ROPE_*).  Band f is the complex
 * number (x_{2f}, x_{2f+1}) -- the talk page's rotation equation -- or,
 * half split, (x_f, x_{f+d/2}).  The pages print only the interleaved
 * pairing; the half split is a storage layout supported as a reading (the
 * rotation of each pair is the printed matrix either way).  The scores do
 * not depend on the layout; only where the parts are stored.
 */
enum { TRI_ROPE_INTERLEAVED = 0, TRI_ROPE_HALF_SPLIT = 1 };

typedef struct {
  int32_t head_dim;     /* d: even, multiple of 8, 8..256                 */
  int32_t num_q_heads;  /* H_q                                            */
  int32_t num_kv_heads; /* H_kv; H_q % H_kv == 0 and G = H_q/H_kv <= 16   */
  int32_t num_layers;   /* L                                              */
  double rope_theta;    /* theta > 0 (10000 in the pages)                 */
  int32_t rope_layout;  /* TRI_ROPE_INTERLEAVED (0) or TRI_ROPE_HALF_SPLIT.
                           Half split: every call supports it; the max over
                           offsets needs d % 64 == 0 there, and tri_score
                           takes its MFMA kernel only when d % 64 == 0      */
} tri_shape;

/*
 * tri_calibrate -- per-band query statistics (offline, once per model).
 *
 * Defined by the talk page's S_norm paragraph (R_f = |E[q_f]| / E[|q_f|])
 * and the hyper.ai summary, section "方法"; calibration runs once on a small
 * batch (blog review, step 1).
 *
 *  q         [L][n_samples][H_q][d] bf16 sample queries, 16-byte aligned
 *            (device).  If q_pos != NULL
 *            they are post-RoPE at positions q_pos[n_samples] (int32,
 *            device) and are de-rotated first; if q_pos == NULL they are
 *            taken as pre-RoPE.
 *  q_centre  out [L][H_q][F][2] fp32: E[q_f] (real, imaginary) pre-RoPE.
 *  q_absmean out [L][H_q][F] fp32: E[|q_f|].
 *  q_R       out [L][H_q][F] fp32: R_f = |E[q_f]| / E[|q_f|]; 1 where
 *            E[|q_f|] = 0.
 *  workspace device scratch of at least tri_calibrate_workspace_bytes(),
 *            16-byte aligned.
 * Sums are fp64: in sample order within chunks of 256 samples, then over
 * the chunks in order (deterministic).  n_samples >= 1.
 */
size_t tri_calibrate_workspace_bytes(const tri_shape* shape, int64_t n_samples);

tri_status tri_calibrate(const tri_shape* shape, const uint16_t* q,
                         const int32_t* q_pos, int64_t n_samples,
                         float* q_centre, float* q_absmean, float* q_R,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * tri_workspace_bytes -- device workspace that tri_score and
 * tri_select_compact need for this batch (the larger of the two).
 * cu_len [host][num_seqs+1].  Returns 0 on invalid arguments.
 */
size_t tri_workspace_bytes(const tri_shape* shape, int32_t num_seqs,
                           const int64_t* cu_len);

/*
 * tri_score -- TriAttention importance of every cached key.
 *
 * For query head h of unit (s, l, g) and key i, the offset-averaged score
 *   S~_h(i) = mean_{delta in D} [ S_trig(k_i, Delta_i + delta) ] + S_norm(k_i)
 *   S_trig(k, Delta) = sum_f |E q_f| |k_f| cos(omega_f Delta + arg E q_f - arg k_f)
 *   S_norm(k)        = sum_f (1 - R_f) E|q_f| |k_f|
 * with k_f the pre-RoPE key band, Delta_i = cur_pos[s] - pos_i and
 * D = {2^0, ..., 2^16} (talk page, S_trig / S_norm / averaged-score
 * equations).  Then, per unit and query head, z_h(i) = (S~_h(i) - mu_h) /
 * sigma_h over the unit's n_s keys (population sigma; sigma = 0 gives z = 0)
 * and scores[i] = max over the G heads of z_h(i) (hyper.ai summary,
 * section "方法").
 *
 * The stored key is k'_f = k_f exp(i omega_f pos_i), so the key position
 * cancels from the score: only k' and cur_pos enter.  k_pos may be NULL and
 * is not read.
 *
 *  cu_len     [host][num_seqs+1] non-decreasing row offsets (see layout).
 *  cur_pos    [host][num_seqs] current query position p_q of each sequence.
 *  k          post-RoPE bf16 keys, rows of d, packed unit-major.
 *  q_centre, q_absmean, q_R   statistics as tri_calibrate writes them.
 *  scores     out fp32, one per row (same packing, no d).
 *  raw_scores optional out fp32 [rows][G]: S~_h(i) before the z-score.
 *  head_stats optional out fp64 [units][G][2]: (mu_h, sigma_h); unit index
 *             = (s*L + l)*Hkv + g.
 *  workspace  device scratch of at least tri_workspace_bytes().
 *
 *  Work-groups of the fused kernel wait for each other's per-chunk
 *  statistics.  The wait provably ends, and it is also bounded: should the
 *  bound ever be reached, the kernel does not hang.  A head whose
 *  statistics a finalizing work-group gave up on gets mean NaN and sigma 0
 *  there, so its z-scores drop out of that chunk's maximum (scores -inf
 *  where every head of the group is affected), and head_stats, written
 *  with the unit's first chunk, show (NaN, 0) for it.  The call also raises
 *  a flag in the workspace that tri_score_status reports.  The planner
 *  keeps that case out of reach: a unit takes the fused path only if its
 *  chunks number at most the work-groups the device holds at once
 *  (occupancy x CUs, twice what the wait needs); longer units take the
 *  generic path, which never waits on other work-groups.
 */
tri_status tri_score(const tri_shape* shape, int32_t num_seqs,
                     const int64_t* cu_len, const int32_t* cur_pos,
                     const uint16_t* k, const int32_t* k_pos,
                     const float* q_centre, const float* q_absmean,
                     const float* q_R, float* scores, float* raw_scores,
                     double* head_stats, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * tri_score_noalloc -- tri_score for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, results and errors as tri_score,
 * without the workspace: the scratch tri_score would take from the
 * workspace lives in a device array of the library, 64 MiB, that each GPU
 * the library runs on holds until the process ends; the per-call sequence
 * table travels in kernel arguments (one small launch per 64 sequences) as
 * for every call.  No hipMalloc, hipFree or host-pinned allocation is made.
 *
 * Limit: a call whose tri_workspace_bytes() exceeds 64 MiB (about 3,900
 * units of head_dim 128 on the fused path) returns TRI_ERR_WORKSPACE and
 * queues nothing.  Every call on one GPU shares that GPU's array: calls
 * that overlap on one GPU (two streams, or two host threads) race and must
 * be serialised by the caller; calls in order on one stream are safe (each
 * call reinitialises what it reads).
 */
tri_status tri_score_noalloc(const tri_shape* shape, int32_t num_seqs,
                             const int64_t* cu_len, const int32_t* cur_pos,
                             const uint16_t* k, const int32_t* k_pos,
                             const float* q_centre, const float* q_absmean,
                             const float* q_R, float* scores, float* raw_scores,
                             double* head_stats, void* stream);

/*
 * tri_score_status -- whether the last tri_score (or tri_score_offsets,
 * tri_score_paged) call queued on `workspace` gave up a bounded wait (see
 * tri_score): *flags gets TRI_SCORE_WAIT_GAVE_UP if it did, else 0.
 * workspace == NULL reads tri_score_noalloc's scratch on the current device.
 * Blocks the host until `stream` has finished its queued work, then reads
 * the flag: word 1 (a uint32 at byte offset 4) of the workspace, which
 * every score call resets when it starts and select never writes.
 */
#define TRI_SCORE_WAIT_GAVE_UP 1u
tri_status tri_score_status(const void* workspace, uint32_t* flags, void* stream);

/*
 * tri_debug_set_resident_groups -- test hook: replaces the device query of
 * how many fused-kernel work-groups run at once (used by the planner's
 * per-unit chunk cap, see tri_score) with `groups`; 0 restores the query.
 * Returns the previous override.  Lets a test on any host (also without a
 * GPU) check where the planner routes long units on a smaller device.  Not
 * for production use.
 */
int32_t tri_debug_set_resident_groups(int32_t groups);

/*
 * tri_debug_set_wait_limit -- test hook: the number of polls of one
 * chunk-statistics slot after which a finalizing work-group of the fused
 * score kernel gives up on it (default 4194304, far beyond any real wait).
 * Applies to launches queued after it returns; returns the previous value.
 * A small bound forces the outcome described at tri_score from the host,
 * with every kernel still exiting normally.  Not for production use.
 */
uint32_t tri_debug_set_wait_limit(uint32_t polls);

/*
 * tri_debug_set_phase_buffer -- measurement hook: where the cycles of the
 * fused score kernel's passes go.  device_buf is device memory of 8
 * unsigned 64-bit counters, owned and zeroed by the caller; NULL (the
 * default) turns the hook off.  While it is set, every launch of the fused
 * score kernel (tri_score, tri_score_noalloc, tri_score_offsets with the
 * mean, the decode calls' pruning steps) on head_dim 128 with the
 * interleaved layout and a packed cache runs a copy of the kernel in which
 * wave 0 of every work-group adds the core-clock cycles (s_memtime) of
 * each phase of its passes to counters 0..6 -- streaming its blocks of the
 * chunk; waiting
 * for the work-group's other waves; decoding the next ticket and
 * requesting its first K blocks; the chunk's moments and their
 * publication; waiting for the unit's published statistics; z-score and
 * group max; ticket claim, next operands, score stores and the closing
 * barrier -- and its number of passes to counter 7.  Scores are the
 * same bits as without the hook.  Other shapes ignore it.  A scoring call
 * returns TRI_ERR_HIP if the counting kernel would hold fewer work-groups
 * per CU than the plain one.  Applies to launches queued after it returns;
 * returns the previous buffer.  Not for production use.
 */
unsigned long long* tri_debug_set_phase_buffer(unsigned long long* device_buf);

/*
 * Offset-set variants of tri_score.
 *
 * The hyper.ai summary, section "实验", reports an ablation over the future
 * offsets (maximum distance, number of offsets, geometric against linear
 * spacing); the shibing624 blog review, section "一个细节：未来位置的处理",
 * combines the offsets with a maximum where the talk page's averaged-score
 * equation takes their mean.  tri_score_offsets runs either reduction over
 * a caller-given set D:
 *   TRI_REDUCE_MEAN  S~_h(i) = mean_{delta in D} S_trig(k_i, Delta_i + delta) + S_norm(k_i)
 *   TRI_REDUCE_MAX   S~_h(i) = max_{delta in D}  S_trig(k_i, Delta_i + delta) + S_norm(k_i)
 * followed by the same z-score and max over the GQA group as tri_score.
 * With TRI_REDUCE_MEAN and D = {2^0, ..., 2^16} in that order the outputs
 * equal tri_score's bit for bit.
 */
typedef enum {
  TRI_REDUCE_MEAN = 0, /* average over the offsets (folds into one term)  */
  TRI_REDUCE_MAX = 1   /* maximum over the offsets (one row per offset)   */
} tri_reduce;

/*
 * tri_workspace_bytes_offsets -- workspace of tri_score_offsets and
 * tri_select_compact for this batch, n_offsets offsets and this reduction.
 * Returns 0 on invalid or unsupported arguments (tri_last_error() says
 * which).
 */
size_t tri_workspace_bytes_offsets(const tri_shape* shape, int32_t num_seqs,
                                   const int64_t* cu_len, int32_t n_offsets,
                                   int32_t reduce);

/*
 * tri_score_offsets -- tri_score over the offset set offsets[n_offsets]
 * [host] (distances in positions, any finite doubles, used in the order
 * given; 1 <= n_offsets <= 4096) combined by `reduce` (a tri_reduce).
 * Every other argument is as for tri_score.
 *
 * TRI_REDUCE_MAX needs head_dim % 32 == 0, and one head's offset rows
 * must fit the kernel's LDS budget: up to 608 offsets at d = 64, 288 at
 * d = 128, 128 at d = 256.  Heads are processed in as many
 * passes over the keys as that budget needs.  Shapes outside this return
 * TRI_ERR_UNSUPPORTED.  TRI_REDUCE_MAX spills raw scores to the workspace
 * (or to raw_scores when given).
 */
tri_status tri_score_offsets(const tri_shape* shape, int32_t num_seqs,
                             const int64_t* cu_len, const int32_t* cur_pos,
                             const uint16_t* k, const int32_t* k_pos,
                             const float* q_centre, const float* q_absmean,
                             const float* q_R, const double* offsets,
                             int32_t n_offsets, int32_t reduce, float* scores,
                             float* raw_scores, double* head_stats,
                             void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * tri_select_compact -- keep the top-B keys of every unit, in time order,
 * and gather their K, V rows and positions.
 *
 * Per unit, b_s = min(budget[s], n_s) keys are kept: the highest scores,
 * equal scores resolved toward the lower index (= lower position); -0.0
 * equals +0.0 and NaN ranks below every number (talk page, closing top-B
 * step; tutorial page, eviction step, which sorts the kept indices to keep
 * the time order).
 *
 *  budget    [host][num_seqs] B_s >= 0.
 *  scores    fp32 per row (as tri_score writes them).
 *  kept_idx  out int32, b_s per unit, ascending indices in [0, n_s);
 *            packed unit-major like the input with b_s in place of n_s.
 *  k, k_out  optional pair (both NULL or both set): K rows in / gathered out.
 *  v, v_out  optional pair: V rows in / gathered out.
 *  k_pos, pos_out  optional pair: int32 positions in / gathered out.
 *  Output rows use the same packing as kept_idx.
 */
tri_status tri_select_compact(const tri_shape* shape, int32_t num_seqs,
                              const int64_t* cu_len, const int32_t* budget,
                              const float* scores, const uint16_t* k,
                              const uint16_t* v, const int32_t* k_pos,
                              int32_t* kept_idx, uint16_t* k_out,
                              uint16_t* v_out, int32_t* pos_out,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * tri_trig_correlation -- reconstruction diagnostic (shibing624 blog
 * review, Fig. 1(D) and Fig. 7): how well the trig series built from the
 * query centres follows the real attention logits.  For layer l and query
 * head h (KV head g = h / G), over every pair of a sample query j and a
 * key i,
 *   x_ji = S_trig(k_i, p_j - p_i) = sum_f |E q_f| |k_f| cos(omega_f (p_j - p_i) + arg E q_f - arg k_f)
 *   y_ji = <q'_j, k'_i>   (post-RoPE logit, unscaled)
 * (talk page, logit decomposition and S_trig equation), and
 *   r[l][h] = Pearson(x, y) over all n_q * n_k pairs; 0 if either is constant.
 *
 *  q         [L][n_q][H_q][d] bf16 post-RoPE sample queries (tri_calibrate's
 *            layout) at positions q_pos [n_q] (int32, device).
 *  k         [L][H_kv][n_k][d] bf16 post-RoPE keys: one sequence in the
 *            packed layout.  k_pos may be NULL and is not read (the key
 *            position cancels as in tri_score).
 *  q_centre  [L][H_q][F][2] as tri_calibrate writes it.
 *  r         out fp64 [L][H_q].
 *  workspace at least tri_trig_correlation_workspace_bytes().
 * head_dim must be a multiple of 32 (TRI_ERR_UNSUPPORTED otherwise).
 * Sums are fp64 in a fixed order (deterministic).
 */
size_t tri_trig_correlation_workspace_bytes(const tri_shape* shape, int64_t n_q);

tri_status tri_trig_correlation(const tri_shape* shape, const uint16_t* q,
                                const int32_t* q_pos, int64_t n_q,
                                const uint16_t* k, const int32_t* k_pos,
                                int64_t n_k, const float* q_centre, double* r,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * tri_stream_probe -- read-bandwidth probe (a measurement aid, not part of
 * the method): reads `bytes` of device memory at src once, with 16-byte
 * non-temporal loads, one contiguous span per work-group over every
 * compute unit, and XORs all its
 * 32-bit words into *sink (so no read can be skipped).  Timing it on a
 * buffer the size of a K cache gives the rate a plain streaming read
 * reaches on the device, the practical ceiling of tri_score's K stream.
 *
 *  src    device, 16-byte aligned; bytes a multiple of 16 (else
 *         TRI_ERR_INVALID_ARGUMENT).  Read only.
 *  sink   one device uint32, owned and initialised by the caller; the
 *         probe XORs into it (it is not cleared).
 * bytes == 0 is a no-op.  Asynchronous on `stream`.
 */
tri_status tri_stream_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

/*
 * Decode-loop driver.
 *
 * Keeps the pruned K/V cache of a batch across decode steps.
 *  - tutorial page, streaming-generation paragraph: every decode step
 *    appends the new token's K and V to the cache and evicts once the
 *    cache is over budget; the most recent r tokens are protected.
 *  - the same page's renormalisation paragraph: attention-sink tokens
 *    (e.g. [BOS]) are kept.
 *  - hyper.ai summary, section "方法": score and prune once every 128
 *    generated tokens.
 *
 * Every unit of a sequence holds the same number of keys.  When a
 * sequence's units reach budget + interval keys (after an append, or at
 * prefill), the driver prunes them to `budget`:
 *  - scores come from tri_score, at the position of the newest key (at
 *    prefill: cur_pos);
 *  - the first protect_sink and last protect_recent keys are kept
 *    whatever their score;
 *  - the other keys compete as in tri_select_compact.
 * The kept rows are compacted, in time order, into the sequence's other
 * buffer: each sequence has two ping-pong buffers of budget + interval
 * rows per unit.
 *
 * Memory: the driver allocates with hipMalloc on the current device,
 * 2 * units * (budget + interval) rows of K, V (bf16) and positions
 * (int32), plus scores, indices and a score workspace.  A prefill of
 * sequences longer than budget + interval grows its own scratch.  The
 * statistics pointers given to tri_decode_create are borrowed and must
 * outlive the driver.
 *
 * Calls on one driver are not thread-safe and must be ordered, normally
 * on one stream.  All work is queued on `stream`; lengths are tracked on
 * the host, so no call waits on the device except tri_decode_destroy.
 */
typedef struct tri_decode tri_decode; /* opaque */

typedef struct {
  int32_t budget;         /* B >= 1: keys per unit after a prune            */
  int32_t interval;       /* >= 1: appends between prunes (128 in the pages) */
  int32_t protect_sink;   /* >= 0: first keys of a unit always kept         */
  int32_t protect_recent; /* >= 0: last keys of a unit always kept          */
} tri_decode_config;      /* protect_sink + protect_recent <= budget        */

typedef struct {
  int64_t unit_stride;         /* rows from one unit of a sequence to the next
                                  (budget + interval)                          */
  const uint16_t* const* k;    /* [num_seqs] device: row 0 of unit 0; unit
                                  (l, g) at + (l*Hkv + g)*unit_stride rows     */
  const uint16_t* const* v;    /* [num_seqs] device, same layout               */
  const int32_t* const* pos;   /* [num_seqs] device positions, same layout     */
  const int32_t* len;          /* [num_seqs] keys per unit now                 */
  const float* const* scores;  /* [num_seqs] device scores the sequence's last
                                  prune used (protected keys read +inf), or
                                  NULL before its first prune                  */
  const int64_t* scores_stride;/* [num_seqs] rows between units in `scores`    */
  int64_t prunes;              /* sequence prunes run so far                   */
} tri_decode_view;             /* host arrays owned by the driver, valid until
                                  its next call                                */

/* Create a driver for num_seqs sequences.  q_centre/q_absmean/q_R as for
 * tri_score (device, borrowed).  Returns TRI_ERR_HIP if allocation fails. */
tri_status tri_decode_create(const tri_shape* shape, int32_t num_seqs,
                             const tri_decode_config* config,
                             const float* q_centre, const float* q_absmean,
                             const float* q_R, tri_decode** out);

/* Load the caches from packed K, V and positions (the tri_score layout;
 * cu_len [host][num_seqs+1], cur_pos [host][num_seqs]).  Sequences of at
 * least budget + interval keys are pruned to budget at once (scored at
 * cur_pos); the others are copied whole.  Replaces any earlier contents. */
tri_status tri_decode_prefill(tri_decode* dec, const int64_t* cu_len,
                              const int32_t* cur_pos, const uint16_t* k,
                              const uint16_t* v, const int32_t* k_pos,
                              void* stream);

/* Append one token to every sequence: k_new, v_new [num_seqs][L][Hkv][d]
 * bf16 (device), pos_new [host][num_seqs] its position (above the
 * sequence's last one).  Sequences that reach budget + interval keys are
 * pruned in the same call. */
tri_status tri_decode_append(tri_decode* dec, const uint16_t* k_new,
                             const uint16_t* v_new, const int32_t* pos_new,
                             void* stream);

/* Where the caches are now. */
tri_status tri_decode_get_view(const tri_decode* dec, tri_decode_view* view);

/* Wait for the device, then free everything the driver allocated. */
tri_status tri_decode_destroy(tri_decode* dec);

/*
 * Per-layer budgets (tutorial page, budget-setting step: a KV budget per
 * layer, and PyramidKV's pyramid allocation across layers, fewer keys for
 * shallow layers and more for deep ones).
 *
 * tri_pyramid_budgets -- budgets[num_layers] growing linearly with the
 * layer index: the last is `ratio` times the first, the two ends average
 * to mean_budget, each rounded to the nearest integer (the pages give the
 * shape, not a formula).  ratio > 0; mean_budget in [0, 1e9].
 *
 * tri_select_compact_layers -- tri_select_compact with one budget per
 * (sequence, layer): budget [host][num_seqs][L].  Unit (s, l, g) keeps
 * b = min(budget[s][l], n_s) keys.  Outputs are packed by (sequence,
 * layer) in order, each pair holding its Hkv units of b rows back to back.
 * Workspace: tri_workspace_bytes_layers().  Everything else is as for
 * tri_select_compact; scores come from tri_score unchanged.
 */
tri_status tri_pyramid_budgets(int32_t num_layers, double mean_budget,
                               double ratio, int32_t* budgets);

size_t tri_workspace_bytes_layers(const tri_shape* shape, int32_t num_seqs,
                                  const int64_t* cu_len);

tri_status tri_select_compact_layers(const tri_shape* shape, int32_t num_seqs,
                                     const int64_t* cu_len, const int32_t* budget,
                                     const float* scores, const uint16_t* k,
                                     const uint16_t* v, const int32_t* k_pos,
                                     int32_t* kept_idx, uint16_t* k_out,
                                     uint16_t* v_out, int32_t* pos_out,
                                     void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Paged pools (tutorial page, deployment paragraph: engines keep the KV
 * cache in pages, as vLLM's PagedAttention does).
 *
 * A page holds page_size consecutive tokens of one sequence for every layer
 * and KV head.  page_table [device][num_seqs][max_pages] int32 gives the
 * physical page of each logical page of a sequence (one table per sequence,
 * shared by its layers and heads).  Token i of unit (s, l, g) is pool row
 *   l*layer_stride + g*head_stride + page*page_stride + (i % page_size)*token_stride,
 *   page = page_table[s][i / page_size];
 * a K or V row is head_dim bf16 elements, a position row one int32.  The
 * strides describe token-major pages ([page][slot][head]: token_stride =
 * H_kv, head_stride = 1, page_stride = page_size*H_kv) as well as head-major
 * ones ([page][head][slot]).  Page ids outside [0, num_pages) are clamped
 * into that range (never an access outside the pool; results for such
 * tokens are unspecified).  page_size: a power of two in [1, 65536];
 * max_pages must cover ceil(n / page_size) for every sequence.  The table
 * is read by the kernels; the caller keeps it alive until the stream has
 * passed the call.
 */
typedef struct {
  const int32_t* page_table; /* device [num_seqs][max_pages]               */
  int32_t max_pages;         /* entries per sequence in page_table          */
  int32_t num_pages;         /* pages in the pool                           */
  int32_t page_size;         /* tokens per page (power of two)              */
  int64_t page_stride;       /* rows from one page to the next              */
  int64_t token_stride;      /* rows from one slot of a page to the next    */
  int64_t head_stride;       /* rows from one KV head to the next           */
  int64_t layer_stride;      /* rows from one layer to the next             */
} tri_kv_pages;

/*
 * tri_score_paged -- tri_score (offsets == NULL) or tri_score_offsets
 * (offsets given, reduced by `reduce`) with the keys read from a paged
 * pool.  scores, raw_scores and head_stats keep the packed layout of
 * tri_score.  Pages of at least 16 tokens take the fused MFMA kernel
 * (head_dim % 32 == 0); smaller pages the VALU path, which needs more
 * workspace: tri_workspace_bytes_paged (n_offsets 0 for the built-in set).
 */
size_t tri_workspace_bytes_paged(const tri_shape* shape, int32_t num_seqs,
                                 const int64_t* cu_len, int32_t page_size,
                                 int32_t n_offsets, int32_t reduce);

tri_status tri_score_paged(const tri_shape* shape, int32_t num_seqs, const int64_t* cu_len,
                           const int32_t* cur_pos, const tri_kv_pages* pages,
                           const uint16_t* k_pool, const float* q_centre,
                           const float* q_absmean, const float* q_R, const double* offsets,
                           int32_t n_offsets, int32_t reduce, float* scores, float* raw_scores,
                           double* head_stats, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * tri_select_compact_paged -- tri_select_compact with K, V and positions
 * read from the paged pool in_pages describes and the kept rows written, in
 * time order, to the pool out_pages describes: kept key j of unit (s, l, g)
 * goes to that pool's row for token j of (s, l, g).  The two may share a
 * pool (distinct pages: the call reads and writes at once).  kept_idx keeps
 * the packed layout (indices are token indices within the unit).  Pools
 * come in pairs (k_pool/k_out_pool, ...); with none given, in_pages and
 * out_pages may be NULL and only kept_idx is written.  Workspace:
 * tri_workspace_bytes.
 */
tri_status tri_select_compact_paged(const tri_shape* shape, int32_t num_seqs,
                                    const int64_t* cu_len, const int32_t* budget,
                                    const float* scores, const tri_kv_pages* in_pages,
                                    const uint16_t* k_pool, const uint16_t* v_pool,
                                    const int32_t* pos_pool, int32_t* kept_idx,
                                    const tri_kv_pages* out_pages, uint16_t* k_out_pool,
                                    uint16_t* v_out_pool, int32_t* pos_out_pool,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static string). */
const char* tri_status_string(tri_status status);

/* Message describing the calling thread's last failing call ("" if none). */
const char* tri_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TRIATTN_H */
