// Fused TriAttention score kernel for head_dim a multiple of 32 (gfx950).
//
// Per key i of a unit and query head h (talk page "聊聊 TriAttention", S_trig,
// S_norm and averaged-score equations; the offset mean and current position
// are folded into A_f = E[q_f] C_f exp(i omega_f p_q) by the prologue):
//   S~_h(i) = sum_j a_h[j] k'_i[j] + sum_f w_h[f] |k'_i,f|
// with a_h[2f] = Re A_f, a_h[2f+1] = Im A_f and w_h[f] = (1 - R_f) E|q_f|.
// Then z_h(i) = (S~_h(i) - mu_h) / sigma_h over the unit and the score is the
// max over the G heads of the group (hyper.ai summary, section "方法").
//
// Mapping onto CDNA4:
//  * The dot product with the post-RoPE key is a (16 heads x d) x (d x 16
//    keys) product per block of 16 keys: v_mfma_f32_16x16x32_bf16.  The keys
//    are bf16 already; the fp64 coefficient a_h is split into two bf16 terms
//    (hi + mid, ~17 significant bits: the split moves a coefficient by at
//    most 2^-17 of itself), so two MFMAs per 32-wide step give the dot
//    product with exact bf16 x bf16 products and fp32 accumulation.  On the
//    workload shapes this moves z-scores by at most 1.5e-5 against exact
//    coefficients (fp64 check), well inside the 1e-4 score bar; a third term
//    (3e-8) costs a third more trig MFMAs and 16 registers, about 4% of the
//    kernel's time.  The split operands of every unit are packed once per
//    call, in MFMA lane order, by prep_fused_kernel.
//  * The norm term sum_f w_f |k_f| uses v_mfma_f32_16x16x4_f32 on the fp32
//    magnitudes (computed once per key band on the VALU, shared by all G
//    heads).
//  * K is read in whole 128-byte lines with non-temporal loads (eight lanes
//    per line, each line read once) and transposed to the MFMA layout
//    through a small per-wave LDS tile; the MFMA layout read directly would
//    touch every line from two instructions.  The 4 waves of a work-group
//    take interleaved blocks so the group streams one contiguous span of K.
//  * Work is cut into "tickets": one chunk of `ch` keys of one unit, with ch
//    chosen per call so that three work-groups fit in a CU's LDS.  The
//    kernel is persistent: each work-group claims tickets in order from an
//    atomic counter and keeps two chunks' raw per-head scores in LDS.  It
//    streams chunk i, publishes the chunk's per-head fp64 sum and sum of
//    squares, and finalizes chunk i only after streaming chunk i+1, so the
//    wait for the rest of chunk i's unit overlaps useful streaming.
//  * No work-group idles between chunks: while streaming chunk i+1 it has
//    already claimed chunk i+2 (an atomic whose result it reads afterwards),
//    so it requests chunk i+2's first K blocks, then publishes chunk i+1
//    and finalizes chunk i while they land.  This holds whenever chunk i+1
//    starts past the end of chunk i's unit; otherwise (rare: one group took
//    two chunks of a unit) it publishes chunk i+1, finalizes chunk i, and
//    only then claims and requests the next chunk.
//  * The steps between chunks work per head on a group of lanes inside one
//    wave (the moments of a chunk, the sums of a unit's published slots)
//    and reduce it with DPP lane moves, so a head's total forms in one lane
//    without a work-group barrier.
//  * Publishing needs no flag and no ordering wait: every published slot
//    holds a sentinel NaN (set by the prologue) until its value lands, and
//    values are written once with coherent (agent-scope) stores.  A
//    finalizing work-group reads all chunk slots of its unit (re-reading any
//    that still hold the sentinel), sums them in one fixed order and derives
//    (mu, sigma); every chunk of the unit does the same arithmetic on the
//    same numbers, so results are deterministic and equal keys score
//    equally.
//  * Waits cannot deadlock.  A work-group waits only to finalize, and then
//    holds a claimed, unpublished chunk (at most one, claimed ahead) only of
//    a later unit than the one it waits on.  Following "waits on a chunk held by" from
//    any waiter therefore passes through strictly earlier units and ends at
//    a work-group that is streaming (and will publish) or at an unclaimed
//    chunk.  Tickets are claimed in order, so an unclaimed chunk a waiter
//    needs lies in the unit holding the claim frontier; a waiter on that
//    unit holds no unpublished chunk and two published ones of it, so such
//    a chunk stays unclaimed only if every resident work-group waits with
//    two chunks of one unit, i.e. with twice the resident work-groups no
//    more than the unit's chunks.  The planner caps chunks per unit well
//    below that.  A spin bound turns a broken invariant into an error flag
//    instead of a hang.
#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

#include <cstring>

#include "tri_internal.hpp"

namespace tri {

typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// x ~= hi + mid with each term a bf16 (relative residual at most ~2^-17).
__device__ __forceinline__ void split2(double x, uint32_t& hi, uint32_t& mid) {
  hi = bf16_rne((float)x);
  const double r1 = x - (double)__uint_as_float(hi << 16);
  mid = bf16_rne((float)r1);
}

// 16-byte vectors per 32-wide step of a unit's packed operands: the bf16 hi
// and mid terms of the trig coefficients, one unused slot, the fp32 norm
// weights.  With the unused slot a unit's operands start on a 16 KB
// boundary at d = 128 (12 KB without it), and the score kernel measured
// about 1% faster that way.
constexpr int kOpVecs = 4;
constexpr int kOpNorm = 3;  // slot of the norm weights

constexpr int kFusedThreads = 256;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int kRawPad = 4;  // LDS row stride (floats) per head = ch + kRawPad
constexpr int kPrefetch = 2;  // blocks of 16 keys in flight per wave
constexpr int kPollBatch = 4;  // chunk-stat slots a finalizing lane loads at once
constexpr int kFusedLdsPerCu = 160 * 1024;
constexpr int kFusedMaxLds = 96 * 1024;  // dynamic LDS ceiling of one work-group

__device__ __forceinline__ double wave_sum_f(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// threadIdx.x through an opaque move: per-lane values derived from it in the
// once-per-chunk steps are then recomputed where used instead of being
// hoisted out of the persistent loop, where they would stay live (and hold
// registers) through the streaming loop.
__device__ __forceinline__ int local_tid() {
  int v;
  asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "v"((int)threadIdx.x));
  return v;
}

// The per-head steps between chunks give head h the lanes [h << sh, (h + 1)
// << sh) of the work-group, a group inside one wave: 64 lanes for G <= 4,
// 32 for G <= 8, else 16.
__device__ __forceinline__ int head_shift(int G) { return G <= 4 ? 6 : (G <= 8 ? 5 : 4); }

// An fp64 value moved across lanes by a DPP pattern (both 32-bit halves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Sum over a head's group of lanes: swaps within quads, rotations by 4 and 8
// within rows of 16 (DPP, no LDS), then the row pair (swizzle, xor 16) and
// the wave halves (xor 32) as the group needs.  The group's first lane
// forms its total in the same order in every work-group.
__device__ __forceinline__ double head_sum(double v, int shift) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x124>(v);  // row_ror:4
  v += dpp_f64<0x128>(v);  // row_ror:8
  if (shift >= 5) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_ds_swizzle((int)b, 0x401F);  // xor 16 within 32 lanes
    const int hi = __builtin_amdgcn_ds_swizzle((int)(b >> 32), 0x401F);
    v += __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
  }
  if (shift >= 6) v += __shfl_xor(v, 32, 64);
  return v;
}

// |k_f|^2 = x^2 + y^2 of a packed bf16 pair (x low, y high): exact bf16
// products, one fp32 rounding.
__device__ __forceinline__ float band_sq(uint32_t w) {
  bf16x2_t pr;
  __builtin_memcpy(&pr, &w, 4);
  return __builtin_amdgcn_fdot2_f32_bf16(pr, pr, 0.0f, false);
}

__device__ __forceinline__ double ld_agent(const double* p) {
  const uint64_t u = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  return __longlong_as_double((long long)u);
}
__device__ __forceinline__ void st_agent(double* p, double v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), (uint64_t)__double_as_longlong(v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent_u64(const double* p) {
  return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

struct Chunk {
  int t, s, lg, l, g, c, nch, nkeys, nkeys_unit, key0;
  int64_t row0, unit;  // row0: first score row of the chunk (and first K row when packed)
};

// Tickets a work-group claims only grow, so the sequence of a new ticket is
// found from that of the group's last one (s_from): usually it is the same
// or the next, two loads issued together; past that, a binary search.
__device__ __forceinline__ Chunk decode_chunk(const SeqInfo* seqs, int S, int L, int Hkv, int ch,
                                              int t, int s_from) {
  Chunk ck;
  ck.t = t;
  int s = s_from;
  SeqInfo si = seqs[s];
  if (s + 1 < S && seqs[s + 1].chunk_base <= t) {
    int lo = s + 1, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (seqs[mid].chunk_base <= t) lo = mid; else hi = mid - 1;
    }
    s = lo;
    si = seqs[s];
  }
  ck.s = s;
  ck.nch = (si.n + ch - 1) / ch;
  const int local = t - si.chunk_base;
  ck.lg = local / ck.nch;
  ck.c = local % ck.nch;
  ck.l = ck.lg / Hkv;
  ck.g = ck.lg % Hkv;
  ck.nkeys_unit = si.n;
  const int key0 = ck.c * ch;
  ck.key0 = key0;
  ck.nkeys = min(ch, si.n - key0);
  ck.row0 = si.row_base + (int64_t)ck.lg * si.in_stride + key0;
  ck.unit = (int64_t)ck.s * L * Hkv + ck.lg;
  return ck;
}

// Staging tile of one wave: one 128-byte line of each of a block's 16 key
// rows, padded to 9 16-byte chunks per row (conflict-free reads).
constexpr int kTileChunks = 16 * 9;

struct Shared {
  uint4 tile[kFusedWaves][kTileChunks];  // the waves' staging tiles (streaming only)
  float2 zm[kMaxGroup];                  // per head: z = raw * zm.x + zm.y
  int ticket;       // a ticket claimed between chunks, for the work-group
  int next_ticket;  // the ticket claimed ahead, posted after streaming (its
                    // own slot: waves may still be reading `ticket` then)
};

// MFMA operands of one unit, packed by prep_fused_kernel in lane order:
// vector 4*st + 0/1 is the bf16 hi/mid split of a_h over the lane's eight
// d-elements of step st, vector 4*st + 3 the four fp32 norm weights.
template <int STEPS>
__device__ __forceinline__ const uint4* unit_operands(const uint4* __restrict__ apack,
                                                      int64_t unit) {
  return apack + unit * (kOpVecs * STEPS) * 64;
}

// Paged pools (pages of at least 16 tokens): block b (16 keys) of a chunk
// lies in one page, whose table entry this returns.  Every operand of the
// address is wave-uniform and the table a restrict (never written)
// argument, so this is a scalar load, counted apart from the K loads in
// flight: waiting for it does not drain the ring.
__device__ __forceinline__ int block_page(const Chunk& ck, const Pages& pg,
                                          const int32_t* __restrict__ ptab, int b) {
  const int kb = __builtin_amdgcn_readfirstlane(ck.key0 + b * 16);
  const int s = __builtin_amdgcn_readfirstlane(ck.s);
  return ptab[(int64_t)s * pg.max_pages + (kb >> pg.page_shift)];
}

typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));

// Whole-line loads and the tile transpose: rows of whole 128-byte lines (an
// even number of steps), up to d = 192; at d = 256 the transpose's registers
// would cost a wave per SIMD.
template <int STEPS>
constexpr bool whole_lines() { return STEPS % 2 == 0 && STEPS <= 6; }

// Row (within the K array) of key `key` of a chunk's block b.  Paged:
// `page` is the block's table entry (block_page), loaded ahead.
template <bool PAGED>
__device__ __forceinline__ int64_t key_row(const Chunk& ck, const Pages& pg, int page, int b,
                                           int key) {
  if (!PAGED) return ck.row0 + key;
  const int kb = __builtin_amdgcn_readfirstlane(ck.key0 + b * 16);
  const int j = kb >> pg.page_shift;
  const int l = __builtin_amdgcn_readfirstlane(ck.l), g = __builtin_amdgcn_readfirstlane(ck.g);
  const int p = page < 0 ? 0 : (page >= pg.num_pages ? pg.num_pages - 1 : page);
  return (int64_t)l * pg.layer_stride + (int64_t)g * pg.head_stride +
         (int64_t)p * pg.page_stride +
         (int64_t)(ck.key0 + key - (j << pg.page_shift)) * pg.token_stride;
}

// Block b (16 keys) of a chunk into bv.  With whole_lines: load i brings line i/2 of rows 8*(i%2) .. +7,
// eight lanes per line, non-temporal (each line is read once, whole);
// transpose_block then puts the data in MFMA layout.  Otherwise lane
// (m, q) takes 16 bytes of key b*16 + m per step st (4 lanes cover 64
// contiguous bytes of the row), the MFMA layout directly.  Lanes past the
// chunk's last key re-read a valid row.
template <int STEPS, bool PAGED>
__device__ __forceinline__ void load_block(const Chunk& ck, const uint16_t* __restrict__ k,
                                           const Pages& pg, int page, int b,
                                           uint4 (&bv)[STEPS]) {
  constexpr int D = STEPS * 32;
  const int lane = threadIdx.x & 63;
  if constexpr (whole_lines<STEPS>()) {
    const int r8 = lane >> 3, c8 = lane & 7;
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
      int key = b * 16 + 8 * (i & 1) + r8;
      key = key < ck.nkeys ? key : ck.nkeys - 1;
      const v4u_t* rp = reinterpret_cast<const v4u_t*>(k + key_row<PAGED>(ck, pg, page, b, key) * D);
      const v4u_t w = __builtin_nontemporal_load(rp + 8 * (i >> 1) + c8);
      __builtin_memcpy(&bv[i], &w, 16);
    }
  } else {
    const int m = lane & 15, q = lane >> 4;
    int key = b * 16 + m;
    key = key < ck.nkeys ? key : ck.nkeys - 1;
    const uint4* rp = reinterpret_cast<const uint4*>(k + key_row<PAGED>(ck, pg, page, b, key) * D);
#pragma unroll
    for (int st = 0; st < STEPS; ++st) bv[st] = rp[4 * st + q];
  }
}

// Whole-line loads to MFMA layout, in place, through the wave's tile: for
// each line h, loads 2h and 2h+1 (rows 0-7, 8-15) go in, and lane (m, q)
// reads back chunks q and 4 + q of row m (steps 2h and 2h+1).  The wave's
// LDS accesses complete in order, so no barrier is needed.
template <int STEPS>
__device__ __forceinline__ void transpose_block(uint4 (&bv)[STEPS], uint4* __restrict__ tile) {
  if constexpr (whole_lines<STEPS>()) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, q = lane >> 4, r8 = lane >> 3, c8 = lane & 7;
#pragma unroll
    for (int h = 0; h < STEPS / 2; ++h) {
      tile[r8 * 9 + c8] = bv[2 * h];
      tile[(8 + r8) * 9 + c8] = bv[2 * h + 1];
      bv[2 * h] = tile[m * 9 + q];
      bv[2 * h + 1] = tile[m * 9 + 4 + q];
    }
  }
}

// Request the first kPrefetch blocks of each wave of a chunk (wave w takes
// blocks w, w + 4, ...).  chunk_raw consumes them.  Unconditional (blocks
// past the chunk's end re-read its last block) so that no earlier ring
// contents stay live across the caller's code.  Paged: pid[j] receives the
// table entry of the block ring slot j loads next (loaded ahead).
template <int STEPS, bool PAGED>
__device__ __forceinline__ void ring_prime(const Chunk& ck, const uint16_t* __restrict__ k,
                                           const Pages& pg, const int32_t* __restrict__ ptab,
                                           uint4 (&ring)[kPrefetch][STEPS], int (&pid)[kPrefetch]) {
  const int wave = threadIdx.x >> 6;
  const int nblk = (ck.nkeys + 15) >> 4;
#pragma unroll
  for (int j = 0; j < kPrefetch; ++j) {
    const int b = wave + kFusedWaves * j;
    const int bl = b < nblk ? b : nblk - 1;
    load_block<STEPS, PAGED>(ck, k, pg, PAGED ? block_page(ck, pg, ptab, bl) : 0, bl, ring[j]);
    if (PAGED) {
      const int bp = b + kFusedWaves * kPrefetch;
      pid[j] = block_page(ck, pg, ptab, bp < nblk ? bp : nblk - 1);
    }
  }
}

template <int STEPS>
struct UnitOperands {
  bf16x8_t a_hi[STEPS], a_mid[STEPS];  // trig coefficients, bf16 split
  float wn[STEPS][4];                                // norm weights
};

// The MFMA A operands of a chunk's unit (L2-resident): lane holds head m
// (zero rows beyond G), d-range of group q.
template <int STEPS>
__device__ __forceinline__ void load_operands(const Chunk& ck, const uint4* __restrict__ apack,
                                              UnitOperands<STEPS>& op) {
  const uint4* src = unit_operands<STEPS>(apack, ck.unit) + (threadIdx.x & 63);
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const uint4 vh = src[(kOpVecs * st + 0) * 64], vm = src[(kOpVecs * st + 1) * 64];
    const uint4 vw = src[(kOpVecs * st + kOpNorm) * 64];
    __builtin_memcpy(&op.a_hi[st], &vh, 16);
    __builtin_memcpy(&op.a_mid[st], &vm, 16);
    op.wn[st][0] = __uint_as_float(vw.x);
    op.wn[st][1] = __uint_as_float(vw.y);
    op.wn[st][2] = __uint_as_float(vw.z);
    op.wn[st][3] = __uint_as_float(vw.w);
  }
}

// Raw scores of one chunk into raw (LDS, [G][ch + kRawPad]).  The ring holds
// the chunk's first blocks (ring_prime); a ring of kPrefetch register buffers
// keeps that many blocks in flight per wave.
template <int STEPS, bool HALF, bool PAGED>
__device__ __forceinline__ void chunk_raw(const Chunk& ck, int G, int rs,
                                          const UnitOperands<STEPS>& op,
                                          const uint16_t* __restrict__ k, const Pages& pg,
                                          const int32_t* __restrict__ ptab, float* raw,
                                          uint4 (&ring)[kPrefetch][STEPS],
                                          int (&pid)[kPrefetch], uint4* __restrict__ tile) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int nblk = (ck.nkeys + 15) >> 4;

  for (int base = wave; base < nblk; base += kFusedWaves * kPrefetch) {
#pragma unroll
    for (int j = 0; j < kPrefetch; ++j) {
      const int b = base + kFusedWaves * j;
      if (b < nblk) {
        transpose_block<STEPS>(ring[j], tile);
        f32x4_t acc_t = {0.f, 0.f, 0.f, 0.f}, acc_n = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
          // band magnitudes first (independent VALU work), then the trig
          // MFMAs, then the norm MFMAs that consume the magnitudes; slot
          // (st, u) of the norm stands for band slot_band(st, q, u)
          float r[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) r[u] = band_sq(slot_pair<STEPS, HALF>(ring[j], st, u));
#pragma unroll
          for (int u = 0; u < 4; ++u) r[u] = __builtin_amdgcn_sqrtf(r[u]);
          bf16x8_t bk;
          __builtin_memcpy(&bk, &ring[j][st], 16);
          acc_t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.a_hi[st], bk, acc_t, 0, 0, 0);
          acc_t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op.a_mid[st], bk, acc_t, 0, 0, 0);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            acc_n = __builtin_amdgcn_mfma_f32_16x16x4f32(op.wn[st][u], r[u], acc_n, 0, 0, 0);
          // Keep the four bands' dot2 -> sqrt -> MFMA chains overlapped
          // (left alone, the scheduler funnels them through one register and
          // pads every step with wait states): the dot2s and their operand
          // clears, the trig MFMAs, the square roots, the norm MFMAs.
          __builtin_amdgcn_sched_group_barrier(0x002, HALF ? 12 : 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x400, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        const int bn = b + kFusedWaves * kPrefetch;
        if (bn < nblk) {
          load_block<STEPS, PAGED>(ck, k, pg, pid[j], bn, ring[j]);
          if (PAGED) {  // the entry for this slot's following block
            const int bp = bn + kFusedWaves * kPrefetch;
            pid[j] = block_page(ck, pg, ptab, bp < nblk ? bp : nblk - 1);
          }
        }
        // D layout: lane holds heads 4q..4q+3 of key b*16 + m (rows past
        // the chunk's end land in the buffer's padding and are never read)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 4 * q + i;
          if (h < G) raw[h * rs + b * 16 + m] = acc_t[i] + acc_n[i];
        }
      }
    }
  }
}

// Per-head fp64 sum and sum of squares of a chunk's raw scores, read back
// from LDS (after a barrier that follows chunk_raw), published with
// coherent stores by the first lane of each head's group.  No wait: readers
// recognise slots not yet written by their sentinel.
__device__ __forceinline__ void chunk_moments_publish(const Chunk& ck, int G, int rs,
                                                      const float* raw,
                                                      double* __restrict__ chunk_stats) {
  const int tid = local_tid();
  const int hs = head_shift(G), lph = 1 << hs;
  const int h = tid >> hs, k = tid & (lph - 1);
  double a = 0.0, b2 = 0.0;
  if (h < G) {
    const float* row = raw + h * rs;
    const int nk4 = ck.nkeys & ~3;
    for (int i = 4 * k; i < nk4; i += 4 * lph) {
      const f32x4_t r = *reinterpret_cast<const f32x4_t*>(row + i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double v = (double)r[e];
        a += v;
        b2 = fma(v, v, b2);
      }
    }
    for (int i = nk4 + k; i < ck.nkeys; i += lph) {
      const double v = (double)row[i];
      a += v;
      b2 = fma(v, v, b2);
    }
  }
  a = head_sum(a, hs);
  b2 = head_sum(b2, hs);
  if (h < G && k == 0) {
    double* cs = chunk_stats + ((int64_t)ck.t * G + h) * 2;
    st_agent(cs, a);
    st_agent(cs + 1, b2);
  }
}

// Read every chunk slot of the unit (waiting for any still holding the
// sentinel), derive (mu, sigma) per head, z-score the chunk and take the
// max over the group, into row 0 of raw (each key's score overwrites its
// head-0 raw value, by the thread that read the key's raw values).
// chunk_store_scores copies them out; the debug outputs are written here.
// Whether a chunk's scores move as 16-byte vectors (see chunk_finalize).
__device__ __forceinline__ bool vector_scores(const Chunk& ck, const float* scores,
                                              const float* raw_out) {
  return (reinterpret_cast<uintptr_t>(scores + ck.row0) & 15u) == 0 && !raw_out;
}

template <bool PHASES>
__device__ __forceinline__ void chunk_finalize(const Chunk& ck, int G, int rs, const float* raw,
                                               Shared& sh, const double* __restrict__ chunk_stats,
                                               uint32_t* __restrict__ err_flag,
                                               uint32_t wait_limit,
                                               float* __restrict__ scores,
                                               float* __restrict__ raw_out,
                                               double* __restrict__ head_stats, int unit_n,
                                               uint64_t& t_stats) {
  const int tid = local_tid();
  const int hs = head_shift(G), lph = 1 << hs;
  const int h = tid >> hs, k = tid & (lph - 1);
  double a = 0.0, b2 = 0.0;
  if (h < G) {
    // Lane k of head h's group sums chunks k, k + lph, ... in that order.
    // The loads of a batch are all issued before any is examined, so a unit
    // of up to lph * kPollBatch chunks costs one round trip.
    const int t0 = ck.t - ck.c;
    for (int cc0 = k; cc0 < ck.nch; cc0 += lph * kPollBatch) {
      uint64_t u[kPollBatch][2];
#pragma unroll
      for (int r = 0; r < kPollBatch; ++r) {
        const int cc = min(cc0 + r * lph, ck.nch - 1);
        const double* cs = chunk_stats + ((int64_t)(t0 + cc) * G + h) * 2;
        u[r][0] = ld_agent_u64(cs);
        u[r][1] = ld_agent_u64(cs + 1);
      }
#pragma unroll
      for (int r = 0; r < kPollBatch; ++r) {
        const int cc = cc0 + r * lph;
        if (cc < ck.nch) {
          const double* cs = chunk_stats + ((int64_t)(t0 + cc) * G + h) * 2;
          uint32_t spins = 0;
          while (u[r][0] == kStatSentinel || u[r][1] == kStatSentinel) {
            __builtin_amdgcn_s_sleep(2);
            u[r][0] = ld_agent_u64(cs);
            u[r][1] = ld_agent_u64(cs + 1);
            if (++spins > wait_limit) {
              // give up on the whole slot, even if its second half landed:
              // a NaN sum makes the head's mean NaN and its sigma 0, never a
              // finite mean with sigma 0 (one store; the second half's
              // value no longer matters)
              __hip_atomic_store(err_flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              u[r][0] = kStatSentinel;
              break;
            }
          }
          a += __longlong_as_double((long long)u[r][0]);
          b2 += __longlong_as_double((long long)u[r][1]);
        }
      }
    }
  }
  const double sa = head_sum(a, hs), sb = head_sum(b2, hs);
  if (h < G && k == 0) {
    // population moments over the unit's keys; fp64 keeps the cancellation
    // in sum x^2 - n mu^2 far below the fp32 resolution of the raw scores
    const double n = (double)unit_n;
    const double mu = sa / n;
    const double var = fmax(sb / n - mu * mu, 0.0);
    const double sigma = sqrt(var);
    const double inv = sigma > 0.0 ? 1.0 / sigma : 0.0;
    sh.zm[h] = make_float2((float)inv, (float)(-mu * inv));
    if (ck.c == 0 && head_stats) {
      head_stats[(ck.unit * G + h) * 2] = mu;
      head_stats[(ck.unit * G + h) * 2 + 1] = sigma;
    }
  }
  __syncthreads();
  if constexpr (PHASES) t_stats = __builtin_amdgcn_s_memtime();
  // Four keys per thread with 16-byte LDS accesses where the chunk's first
  // score is 16-byte aligned in global memory (rs and the buffers are
  // multiples of four floats); the same fmaf/fmaxf per key as the scalar
  // loop below.
  float* out = const_cast<float*>(raw);
  int i0 = 0;
  if (vector_scores(ck, scores, raw_out)) {
    const int nk4 = ck.nkeys & ~3;
    for (int i = 4 * tid; i < nk4; i += 4 * kFusedThreads) {
      f32x4_t best = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll 4
      for (int hh = 0; hh < G; ++hh) {
        const f32x4_t r = *reinterpret_cast<const f32x4_t*>(raw + hh * rs + i);
        const float2 z = sh.zm[hh];
#pragma unroll
        for (int e = 0; e < 4; ++e) best[e] = fmaxf(best[e], fmaf(r[e], z.x, z.y));
      }
      *reinterpret_cast<f32x4_t*>(out + i) = best;
    }
    i0 = nk4;
  }
  for (int i = i0 + tid; i < ck.nkeys; i += kFusedThreads) {
    float best = -__builtin_inff();
    for (int hh = 0; hh < G; ++hh) {
      const float2 z = sh.zm[hh];
      best = fmaxf(best, fmaf(raw[hh * rs + i], z.x, z.y));
    }
    if (raw_out)
      for (int hh = 0; hh < G; ++hh) raw_out[(ck.row0 + i) * G + hh] = raw[hh * rs + i];
    out[i] = best;
  }
}

// Copy a finalized chunk's scores (row 0 of raw) to global memory, each key
// by the thread that computed it in chunk_finalize.  Non-temporal stores:
// scores written through the L2 like the K stream's loads leave it no dirty
// lines to hold and write back (the score kernel runs about 1.5% faster).
__device__ __forceinline__ void chunk_store_scores(const Chunk& ck, const float* raw,
                                                   float* __restrict__ scores,
                                                   const float* raw_out) {
  const int tid = local_tid();
  int i0 = 0;
  if (vector_scores(ck, scores, raw_out)) {
    const int nk4 = ck.nkeys & ~3;
    for (int i = 4 * tid; i < nk4; i += 4 * kFusedThreads)
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t*>(raw + i),
                                  reinterpret_cast<f32x4_t*>(scores + ck.row0 + i));
    i0 = nk4;
  }
  for (int i = i0 + tid; i < ck.nkeys; i += kFusedThreads)
    __builtin_nontemporal_store(raw[i], scores + ck.row0 + i);
}

// Cycle counters of the phase-profiling build of the kernel: per pass, the
// cycles wave 0 of a work-group spends in each phase, summed over passes.
enum FusedPhase {
  kPhStream,    // streaming its blocks of the chunk
  kPhWaves,     // waiting for the work-group's other waves to finish streaming
  kPhNext,      // decoding the next ticket, requesting its first K blocks
  kPhMoments,   // chunk moments: LDS read-back, fp64 sums, publication
  kPhStats,     // waiting for the unit's published statistics, mu and sigma
  kPhZ,         // z-score and group max of the finalized chunk
  kPhTail,      // ticket claim if not ahead, next operands, score stores, barrier
  kPhCount,
};

// STEPS = head_dim / 32.  Persistent: gridDim.x work-groups loop over the
// tickets.  ch = keys per ticket.  With PHASES, wave 0 of every work-group
// adds its per-phase cycle counts (s_memtime) to phases[0 .. kPhCount) and
// its number of passes to phases[kPhCount]; the arithmetic is unchanged.
template <int STEPS, bool HALF, bool PAGED, bool PHASES>
__device__ __forceinline__ void score_fused_body(
    const SeqInfo* __restrict__ seqs, int S, int L, int Hkv, int G, int ch, int total_tickets,
    const uint4* __restrict__ apack, const uint16_t* __restrict__ k, const Pages pg,
    const int32_t* __restrict__ ptab,
    double* __restrict__ chunk_stats, uint32_t* __restrict__ ctrl, uint32_t wait_limit,
    float* __restrict__ scores, float* __restrict__ raw_out, double* __restrict__ head_stats,
    unsigned long long* __restrict__ phases) {
  extern __shared__ float raw_s[];  // 2 buffers of [G][ch + kRawPad]
  __shared__ Shared sh;
  uint32_t* ticket_ctr = ctrl;
  uint32_t* err_flag = ctrl + 1;
  const int rs = ch + kRawPad;

  auto claim = [&]() {
    return __hip_atomic_fetch_add(ticket_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // One vector-memory counter covers loads and stores, so a wait for a load
  // also waits for every store issued before it.  The next chunk's K ring and
  // operands are therefore requested before this chunk's stores (scores,
  // published moments) and the streaming loop never waits on a store.
  uint4 ring[kPrefetch][STEPS];
  int pid[kPrefetch] = {};  // paged: table entries of the blocks the ring loads next
  UnitOperands<STEPS> op;
  Chunk prev, ck;
  int prev_last = 0;  // last ticket of prev's unit
  bool have_prev = false;
  int cur = 0;
  uint64_t ph[kPhCount] = {};
  uint64_t passes = 0, t_prev = 0, t_stats = 0;
  auto mark = [&](int phase) {
    if constexpr (PHASES) {
      const uint64_t now = __builtin_amdgcn_s_memtime();
      ph[phase] += now - t_prev;
      t_prev = now;
    }
  };
  if (threadIdx.x == 0) sh.ticket = (int)claim();
  __syncthreads();
  int t = __builtin_amdgcn_readfirstlane(sh.ticket);  // uniform: chunk fields in SGPRs
  if (t < total_tickets) {
    ck = decode_chunk(seqs, S, L, Hkv, ch, t, 0);
    ring_prime<STEPS, PAGED>(ck, k, pg, ptab, ring, pid);
    load_operands<STEPS>(ck, apack, op);
  }
  // Each pass streams chunk ck (if any) and finalizes prev (if any).  Every
  // step below has one call site, so their per-lane constants exist once.
  for (;;) {
    const bool have = t < total_tickets;
    if (!have && !have_prev) break;
    float* buf_cur = raw_s + cur * G * rs;
    float* buf_prev = raw_s + (cur ^ 1) * G * rs;
    // Claim the next ticket now (its result is read after streaming) when it
    // is bound to lie in a later unit than prev.  Then prev's finalize runs
    // under the next chunk's first loads with the next chunk held
    // unclaimed-by-others and unpublished, of a later unit than the one
    // waited on.  Otherwise the next ticket is claimed after prev's
    // finalize.  This chunk is published before prev's finalize either way.
    const bool ahead = have && (!have_prev || prev_last < t);
    uint32_t next = 0;  // thread 0
    if (ahead && threadIdx.x == 0) next = claim();
    // The stream runs at the lowest wave priority and the chunk boundary
    // (moments, finalize, score stores, next operands) at a higher one, so
    // that a wave at its boundary takes the SIMD's issue slots ahead of the
    // other work-groups' streaming waves, which mostly wait on memory.
    __builtin_amdgcn_s_setprio(0);
    if constexpr (PHASES) {
      t_prev = __builtin_amdgcn_s_memtime();
      ++passes;
    }
    if (have)
      chunk_raw<STEPS, HALF, PAGED>(ck, G, rs, op, k, pg, ptab, buf_cur, ring, pid,
                                    sh.tile[threadIdx.x >> 6]);
    __builtin_amdgcn_s_setprio(2);
    mark(kPhStream);
    if (ahead && threadIdx.x == 0) sh.next_ticket = (int)next;
    __syncthreads();
    mark(kPhWaves);
    // nk: the next chunk, or (past the last ticket) a valid chunk whose loads
    // go unused.  The ring and operands are reloaded on every path so their
    // old contents are dead from here on.
    Chunk nk = ck;
    if (ahead) {
      t = __builtin_amdgcn_readfirstlane(sh.next_ticket);
      if (t < total_tickets) nk = decode_chunk(seqs, S, L, Hkv, ch, t, ck.s);
    }
    if (ahead || !have) ring_prime<STEPS, PAGED>(nk, k, pg, ptab, ring, pid);
    mark(kPhNext);
    if (have) chunk_moments_publish(ck, G, rs, buf_cur, chunk_stats);
    mark(kPhMoments);
    if (have_prev) {
      chunk_finalize<PHASES>(prev, G, rs, buf_prev, sh, chunk_stats, err_flag, wait_limit, scores,
                             raw_out, head_stats, prev.nkeys_unit, t_stats);
      if constexpr (PHASES) {
        ph[kPhStats] += t_stats - t_prev;
        t_prev = t_stats;
      }
    }
    mark(kPhZ);
    if (have && !ahead) {
      if (threadIdx.x == 0) sh.ticket = (int)claim();
      __syncthreads();
      t = __builtin_amdgcn_readfirstlane(sh.ticket);
      if (t < total_tickets) nk = decode_chunk(seqs, S, L, Hkv, ch, t, ck.s);
      ring_prime<STEPS, PAGED>(nk, k, pg, ptab, ring, pid);
    }
    load_operands<STEPS>(nk, apack, op);
    if (have_prev) chunk_store_scores(prev, buf_prev, scores, raw_out);
    __syncthreads();
    mark(kPhTail);
    if (!have) break;
    prev = ck;
    prev_last = ck.t - ck.c + ck.nch - 1;
    have_prev = true;
    ck = nk;
    cur ^= 1;
  }
  if constexpr (PHASES) {
    if (threadIdx.x == 0) {
      for (int i = 0; i < kPhCount; ++i) atomicAdd(phases + i, (unsigned long long)ph[i]);
      atomicAdd(phases + kPhCount, (unsigned long long)passes);
    }
  }
}

template <int STEPS, bool HALF, bool PAGED>
__global__ __launch_bounds__(kFusedThreads) void score_fused_kernel(
    const SeqInfo* __restrict__ seqs, int S, int L, int Hkv, int G, int ch, int total_tickets,
    const uint4* __restrict__ apack, const uint16_t* __restrict__ k, const Pages pg,
    const int32_t* __restrict__ ptab,
    double* __restrict__ chunk_stats, uint32_t* __restrict__ ctrl, uint32_t wait_limit,
    float* __restrict__ scores, float* __restrict__ raw_out, double* __restrict__ head_stats) {
  score_fused_body<STEPS, HALF, PAGED, false>(seqs, S, L, Hkv, G, ch, total_tickets, apack, k, pg,
                                              ptab, chunk_stats, ctrl, wait_limit, scores, raw_out,
                                              head_stats, nullptr);
}

// The same kernel with per-phase cycle counters (interleaved layout, packed
// cache); launched only while a phase buffer is set.
template <int STEPS>
__global__ __launch_bounds__(kFusedThreads) void score_phase_kernel(
    const SeqInfo* __restrict__ seqs, int S, int L, int Hkv, int G, int ch, int total_tickets,
    const uint4* __restrict__ apack, const uint16_t* __restrict__ k, const Pages pg,
    const int32_t* __restrict__ ptab,
    double* __restrict__ chunk_stats, uint32_t* __restrict__ ctrl, uint32_t wait_limit,
    float* __restrict__ scores, float* __restrict__ raw_out, double* __restrict__ head_stats,
    unsigned long long* __restrict__ phases) {
  score_fused_body<STEPS, false, false, true>(seqs, S, L, Hkv, G, ch, total_tickets, apack, k, pg,
                                              ptab, chunk_stats, ctrl, wait_limit, scores, raw_out,
                                              head_stats, phases);
}

// The fused path's preparation of a call, one launch: block 0 writes the
// plan carried in the arguments (plan_words > 0); every thread resets its
// share of the control words and the published-statistics slots; the blocks
// that pack operands first form, in LDS, C_f for every band (built-in
// offsets by repeated squaring; a given set dealt over the block's threads,
// the partial sums added in a fixed order) and E for the sequences their
// units belong to.  Then thread (unit, st, lane) forms A_f = P * E (fp64,
// P = E[q_f] * C_f) for the lane's head h = g*G + lane%16 and the bands of
// its eight elements of step st, splits each element's part (Re or Im, by
// the RoPE layout) into bf16 hi and mid terms and stores them with the fp32 norm
// weights W = (1 - R) E|q| of the step's four norm slots (zeros for lanes
// beyond G).
template <int STEPS>
__global__ __launch_bounds__(256) void prep_fused_kernel(
    int S, int L, int Hkv, int G, int Hq, bool half, double theta, SeqInfo* __restrict__ seqs,
    const ArgWords plan, int plan_words, const float* __restrict__ q_centre,
    const float* __restrict__ q_absmean, const float* __restrict__ q_R,
    const double* __restrict__ offsets, int nD, uint32_t* __restrict__ ctrl, int64_t n_ctrl,
    double* __restrict__ stat_slots, int64_t n_stat_slots, uint4* __restrict__ apack) {
  constexpr int F = STEPS * 16, D = STEPS * 32;
  constexpr int R = 256 / F;  // threads per band for C_f (F <= 128)
  const int tid = threadIdx.x;
  const int64_t idx = (int64_t)blockIdx.x * 256 + tid;
  if (blockIdx.x == 0)
    for (int i = tid; i < plan_words; i += 256) reinterpret_cast<uint32_t*>(seqs)[i] = plan.w[i];
  if (idx < n_ctrl) ctrl[idx] = 0u;
  if (idx < n_stat_slots)
    reinterpret_cast<unsigned long long*>(stat_slots)[idx] = kStatSentinel;
  const int64_t units = (int64_t)S * L * Hkv;
  const int64_t pack_threads = units * STEPS * 64;
  if ((int64_t)blockIdx.x * 256 >= pack_threads) return;  // block-uniform

  __shared__ double2 part[R][F];
  __shared__ double2 cf[F];
  __shared__ double2 es[256];  // E of the block's sequences: at most 256 (sequence, band)
  if (!offsets) {
    // the built-in set {2^0..2^16}: e^{i w 2^(j+1)} = (e^{i w 2^j})^2, one
    // sincos and 16 squarings per band (each squaring doubles the rounding
    // error: at most ~2^16 ulp, 1e-11, far below the operands' bf16 split)
    if (tid < F) {
      const double omega = pow(theta, -2.0 * (double)tid / (double)D);
      double sn, cs;
      sincos(omega, &sn, &cs);
      double cr = cs, ci = sn;
      for (int j = 1; j < nD; ++j) {
        const double c2 = cs * cs - sn * sn, s2 = 2.0 * sn * cs;
        cs = c2;
        sn = s2;
        cr += cs;
        ci += sn;
      }
      part[0][tid] = make_double2(cr, ci);
    }
  } else {
    const int f = tid % F, r = tid / F;
    if (r < R) {
      const double omega = pow(theta, -2.0 * (double)f / (double)D);
      double cr = 0.0, ci = 0.0;
      for (int j = r; j < nD; j += R) {
        double sn, cs;
        sincos(omega * offsets[j], &sn, &cs);
        cr += cs;
        ci += sn;
      }
      part[r][f] = make_double2(cr, ci);
    }
  }
  const int LH = L * Hkv;
  const int64_t u_lo = (int64_t)blockIdx.x * 256 / (64 * STEPS);
  const int64_t u_hi = ((int64_t)blockIdx.x * 256 + 255) / (64 * STEPS);
  const int s_lo = (int)(u_lo / LH);
  const int s_hi = (int)((u_hi < units ? u_hi : units - 1) / LH);
  const int ns = s_hi - s_lo + 1;
  for (int e = tid; e < ns * F; e += 256) {
    const int s = s_lo + e / F, f = e % F;
    const int32_t p_q =
        plan_words ? reinterpret_cast<const SeqInfo*>(plan.w)[s].p_q : seqs[s].p_q;
    const double omega = pow(theta, -2.0 * (double)f / (double)D);
    double sn, cs;
    sincos(omega * (double)p_q, &sn, &cs);
    es[e] = make_double2(cs, sn);
  }
  __syncthreads();
  if (tid < F) {
    double cr = 0.0, ci = 0.0;
    const int parts = offsets ? R : 1;
    for (int r = 0; r < parts; ++r) {
      cr += part[r][tid].x;
      ci += part[r][tid].y;
    }
    const double inv = 1.0 / (double)nD;
    cf[tid] = make_double2(cr * inv, ci * inv);
  }
  __syncthreads();
  if (idx >= pack_threads) return;

  const int lane = (int)(idx & 63);
  const int st = (int)((idx >> 6) % STEPS);
  const int64_t unit = idx / (64 * STEPS);
  const int lg = (int)(unit % LH);
  const int s = (int)(unit / LH);
  const int l = lg / Hkv, g = lg % Hkv;
  const int m = lane & 15, q = lane >> 4;
  uint32_t h2[8], m2[8];
  float wv[4];
  const bool live = m < G;
  const int64_t pbase = ((int64_t)l * Hq + g * G + (live ? m : 0)) * F;
  const double2* ev_s = es + (s - s_lo) * F;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = 32 * st + 8 * q + j;
    const int f = elem_band(e, D, half);
    double x = 0.0;
    if (live) {
      const double qr = (double)q_centre[2 * (pbase + f)];
      const double qi = (double)q_centre[2 * (pbase + f) + 1];
      const double2 c = cf[f];
      const double2 pv = make_double2(qr * c.x - qi * c.y, qr * c.y + qi * c.x);
      const double2 ev = ev_s[f];
      x = elem_part(e, D, half) ? pv.x * ev.y + pv.y * ev.x : pv.x * ev.x - pv.y * ev.y;
    }
    split2(x, h2[j], m2[j]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t wi = pbase + slot_band(st, q, u, STEPS, half);
    wv[u] = live ? (float)((1.0 - (double)q_R[wi]) * (double)q_absmean[wi]) : 0.f;
  }
  auto pack8 = [](const uint32_t (&v)[8]) {
    return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                      v[6] | (v[7] << 16));
  };
  uint4* op = apack + unit * (kOpVecs * STEPS) * 64 + lane;
  op[(kOpVecs * st + 0) * 64] = pack8(h2);
  op[(kOpVecs * st + 1) * 64] = pack8(m2);
  op[(kOpVecs * st + kOpNorm) * 64] = make_uint4(__float_as_uint(wv[0]), __float_as_uint(wv[1]),
                                     __float_as_uint(wv[2]), __float_as_uint(wv[3]));
}

// Polls of a chunk-statistics slot before a finalizing work-group gives up
// on it (the wait ends by construction; this only bounds a broken one).
static std::atomic<uint32_t> g_wait_limit{1u << 22};

uint32_t set_fused_wait_limit(uint32_t polls) { return g_wait_limit.exchange(polls); }

// Device buffer of kPhCount + 1 counters for the phase-profiling kernel;
// null (the default) runs the plain kernel.
static std::atomic<unsigned long long*> g_phase_buf{nullptr};

unsigned long long* set_fused_phase_buffer(unsigned long long* buf) {
  return g_phase_buf.exchange(buf);
}

template <int STEPS, bool HALF, bool PAGED>
static hipError_t launch_fused_t(int total_tickets, int ch, size_t lds, hipStream_t st,
                                 const SeqInfo* seqs, int S, int L, int Hkv, int G, uint4* apack,
                                 const uint16_t* k, const Pages& pg, double* cs, uint32_t* ctrl,
                                 float* scores, float* raw, double* hs, const PrepArgs& prep) {
  const int64_t pack_threads = (int64_t)S * L * Hkv * STEPS * 64;
  ArgWords plan;
  int plan_words = 0;
  if (prep.plan_host) {
    const size_t bytes = (size_t)S * sizeof(SeqInfo);
    if (bytes > sizeof(plan.w)) return hipErrorInvalidValue;
    std::memcpy(plan.w, prep.plan_host, bytes);
    plan_words = (int)(bytes / 4);
  }
  int64_t total = pack_threads;
  if (prep.n_stat_slots > total) total = prep.n_stat_slots;
  if (prep.n_ctrl > total) total = prep.n_ctrl;
  if (total < 1) total = 1;  // block 0 writes the plan
  const int nD = prep.offsets ? prep.n_offsets : 17;
  hipLaunchKernelGGL(prep_fused_kernel<STEPS>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     st, S, L, Hkv, G, prep.Hq, HALF, prep.theta, const_cast<SeqInfo*>(seqs),
                     plan, plan_words, prep.q_centre, prep.q_absmean, prep.q_R, prep.offsets, nD,
                     ctrl, prep.n_ctrl, cs, prep.n_stat_slots, apack);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || total_tickets == 0) return e;
  const void* kern = reinterpret_cast<const void*>(&score_fused_kernel<STEPS, HALF, PAGED>);
  static const hipError_t attr = hipFuncSetAttribute(
      kern, hipFuncAttributeMaxDynamicSharedMemorySize, kFusedMaxLds);
  if (attr != hipSuccess) return attr;
  int dev = 0, cus = 0, per_cu = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kFusedThreads, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) per_cu = 1;
  int grid = cus * per_cu;
  if (grid > total_tickets) grid = total_tickets;
  if constexpr (STEPS == 4 && !HALF && !PAGED) {
    unsigned long long* phases = g_phase_buf.load(std::memory_order_relaxed);
    if (phases) {
      // same grid as the plain kernel; refused if the counters cost occupancy
      const void* pk = reinterpret_cast<const void*>(&score_phase_kernel<STEPS>);
      static const hipError_t pattr = hipFuncSetAttribute(
          pk, hipFuncAttributeMaxDynamicSharedMemorySize, kFusedMaxLds);
      if (pattr != hipSuccess) return pattr;
      int pcu = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&pcu, pk, kFusedThreads, lds);
      if (e != hipSuccess) return e;
      if (pcu < per_cu) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL((score_phase_kernel<STEPS>), dim3(grid), dim3(kFusedThreads), lds, st,
                         seqs, S, L, Hkv, G, ch, total_tickets, apack, k, pg, pg.table, cs, ctrl,
                         g_wait_limit.load(std::memory_order_relaxed), scores, raw, hs, phases);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((score_fused_kernel<STEPS, HALF, PAGED>), dim3(grid), dim3(kFusedThreads),
                     lds, st, seqs, S, L, Hkv, G, ch, total_tickets, apack, k, pg, pg.table, cs, ctrl,
                     g_wait_limit.load(std::memory_order_relaxed), scores, raw, hs);
  return hipGetLastError();
}

// Work-groups of the fused kernel the current device holds at once for a
// shape (occupancy at the shape's LDS size x CUs), cached per device and
// shape; -1 when no device answers.  A test hook may override the value.
static std::atomic<int> g_resident_override{0};

int set_fused_resident_override(int groups) { return g_resident_override.exchange(groups); }

template <int STEPS, bool HALF, bool PAGED>
static int resident_t(size_t lds) {
  const void* kern = reinterpret_cast<const void*>(&score_fused_kernel<STEPS, HALF, PAGED>);
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kFusedMaxLds) !=
      hipSuccess)
    return -1;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kFusedThreads, lds) !=
          hipSuccess)
    return -1;
  return cus * (per_cu < 1 ? 1 : per_cu);
}

int fused_resident_groups(int d, bool half, bool paged, int G) {
  const int forced = g_resident_override.load();
  if (forced > 0) return forced;
  int count = 0, dev = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1 || hipGetDevice(&dev) != hipSuccess)
    return -1;
  static std::mutex mu;
  static std::map<std::tuple<int, int, bool, bool, int>, int> cache;
  const auto key = std::make_tuple(dev, d, half, paged, G);
  {
    std::lock_guard<std::mutex> lk(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  const size_t lds = 2 * (size_t)G * (fused_chunk_keys(G, d) + kRawPad) * sizeof(float);
  int r = -1;
#define TRI_RES(n, h, pgd) \
  case n:                  \
    r = resident_t<n, h, pgd>(lds); \
    break;
#define TRI_RES_ALL(pgd)                                                                  \
  if (half) {                                                                             \
    switch (d / 32) { TRI_RES(2, true, pgd) TRI_RES(4, true, pgd) TRI_RES(6, true, pgd)   \
                      TRI_RES(8, true, pgd) default: break; }                             \
  } else {                                                                                \
    switch (d / 32) { TRI_RES(1, false, pgd) TRI_RES(2, false, pgd) TRI_RES(3, false, pgd) \
                      TRI_RES(4, false, pgd) TRI_RES(5, false, pgd) TRI_RES(6, false, pgd) \
                      TRI_RES(7, false, pgd) TRI_RES(8, false, pgd) default: break; }     \
  }
  if (paged) {
    TRI_RES_ALL(true)
  } else {
    TRI_RES_ALL(false)
  }
#undef TRI_RES_ALL
#undef TRI_RES
  if (r > 0) {
    std::lock_guard<std::mutex> lk(mu);
    cache[key] = r;
  }
  return r;
}

// Half split needs an even number of 32-wide steps (both parts of a band
// in one lane's words).
bool fused_supported(int d, bool half) {
  return d % 32 == 0 && d >= 32 && d <= kMaxHeadDim && (!half || d % 64 == 0);
}

// Keys per ticket: as many as let the work-groups a CU holds (two raw
// buffers of G heads each) share its LDS, in multiples of 64, at most 1024.
// Up to d = 160 the kernel's registers allow three work-groups per CU; from
// d = 192 (six or more 32-wide steps) only two fit, and chunks sized for
// two cut the chunk boundaries by a third (3% on a d = 256 cache).
int fused_chunk_keys(int G, int d) {
  const int wgs = d / 32 >= 6 ? 2 : 3;
  // leave room for the static LDS (Shared)
  const int per_wg = kFusedLdsPerCu / wgs - (int)((sizeof(Shared) + 255) / 256 * 256);
  int ch = (per_wg / (2 * G * (int)sizeof(float)) - kRawPad) / 64 * 64;
  if (ch > 1024) ch = 1024;
  if (ch < 64) ch = 64;
  return ch;
}

size_t fused_operand_bytes(int d, int64_t units) {
  return fused_supported(d, false) ? (size_t)units * (kOpVecs * (d / 32)) * 64 * sizeof(uint4) : 0;
}

hipError_t launch_score_fused(const SeqInfo* seqs, int S, int L, int Hkv, int G, int d, int ch,
                              int total_tickets, void* apack, const uint16_t* k,
                              double* chunk_stats, uint32_t* ctrl, float* scores, float* raw,
                              double* head_stats, bool half, const Pages& pg,
                              const PrepArgs& prep, hipStream_t st) {
  const size_t lds = 2 * (size_t)G * (ch + kRawPad) * sizeof(float);
  if (lds > (size_t)kFusedMaxLds || !fused_supported(d, half)) return hipErrorInvalidValue;
  if (pg.table && pg.page_shift < 4) return hipErrorInvalidValue;  // pages of >= 16 tokens
  uint4* ap = reinterpret_cast<uint4*>(apack);
#define TRI_CASE(n, h, pgd)                                                                   \
  case n:                                                                                     \
    return launch_fused_t<n, h, pgd>(total_tickets, ch, lds, st, seqs, S, L, Hkv, G, ap, k, pg, \
                                     chunk_stats, ctrl, scores, raw, head_stats, prep);
#define TRI_LAYOUTS(pgd)                                                                      \
  if (half) {                                                                                 \
    switch (d / 32) {                                                                         \
      TRI_CASE(2, true, pgd) TRI_CASE(4, true, pgd) TRI_CASE(6, true, pgd)                    \
      TRI_CASE(8, true, pgd)                                                                  \
      default:                                                                                \
        return hipErrorInvalidValue;                                                          \
    }                                                                                         \
  }                                                                                           \
  switch (d / 32) {                                                                           \
    TRI_CASE(1, false, pgd) TRI_CASE(2, false, pgd) TRI_CASE(3, false, pgd)                   \
    TRI_CASE(4, false, pgd) TRI_CASE(5, false, pgd) TRI_CASE(6, false, pgd)                   \
    TRI_CASE(7, false, pgd) TRI_CASE(8, false, pgd)                                           \
    default:                                                                                  \
      return hipErrorInvalidValue;                                                            \
  }
  if (pg.table) {
    TRI_LAYOUTS(true)
  }
  TRI_LAYOUTS(false)
#undef TRI_LAYOUTS
#undef TRI_CASE
}

}  // namespace tri
