// Top-B selection per unit with the lowest-index tie-break, emitting the
// kept indices in ascending (time) order.
//
// Semantics: talk page "聊聊 TriAttention", closing step (rank keys by the
// averaged score, keep the top B); jaedaily.cn tutorial, eviction step (the
// kept indices are sorted so the time order survives).  Equal scores go to
// the lower index, -0.0 == +0.0, NaN ranks below -inf.
//
// Method: scores map to order-preserving 32-bit keys.  A most-significant-
// digit radix select finds the b-th largest key T and how many keys equal
// to T are kept (the quota).  A final ordered pass keeps every key > T and
// the first `quota` keys == T, writing their indices in index order.  By
// unit length: up to 4096 keys, one work-group of 256 threads with the
// keys in LDS; up to 32768, one work-group of 1024 threads with the keys
// in registers (and, when rows are gathered, the gathers in the same
// kernel); up to 35840, one work-group of 512 threads reading the scores
// three times; longer units are split over work-groups of 4096 keys.
#include <cstring>

#include "tri_internal.hpp"

namespace tri {

// Order-preserving key of a score: non-negative floats map to their bits
// with the top bit set, negative ones to their complemented bits; -0 keys
// as +0 and NaN as 0, below every number.  x + 0.0f turns -0 into +0 and
// leaves every other value's bits as they are (these kernels keep fp32
// denormals, and the sum is exact), so one add replaces a compare and a
// select.
__device__ __forceinline__ uint32_t order_key(float x) {
  const float y = x + 0.0f;
  const uint32_t u = __float_as_uint(y);
  const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return y != y ? 0u : k;
}

// ---------------------------------------------------------------------------
// LDS-staged select: the unit's order keys are loaded once (coalesced) into
// LDS; the radix passes and the ordered scan then run on LDS.  Digits are
// 12, 12 and 8 bits wide: z-scores crowd a few exponent values, and 12-bit
// first digits (sign, exponent, 3 mantissa bits) spread them over enough
// bins that LDS atomics rarely collide.  256 threads per unit (units of up
// to 4096 keys), so that many short units share a CU.
// ---------------------------------------------------------------------------
constexpr int kHistBins = 4096;
constexpr int kScanItems = 8;  // consecutive keys per thread in the ordered scan

// Exclusive prefix sum over a block of NT threads; *total gets the sum.
// The wave totals are scanned across the lanes of every wave (one total
// per lane) and read back with readlane, so the scan holds few registers.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  constexpr int NW = NT / 64;
  static_assert(NW <= 64, "one wave total per lane");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t ws = lane < NW ? wsum[lane] : 0u;
#pragma unroll
  for (int o = 1; o < NW; o <<= 1) {
    const uint32_t y = __shfl_up(ws, o, 64);
    if (lane >= o) ws += y;
  }
  const uint32_t before = wave > 0 ? __builtin_amdgcn_readlane(ws, wave - 1) : 0u;
  const uint32_t all = __builtin_amdgcn_readlane(ws, NW - 1);
  __syncthreads();
  *total = all;
  return before + x - v;
}

template <int NT>
__global__ __launch_bounds__(NT) void select_lds_kernel(
    const SeqInfo* __restrict__ seqs, int LH, const float* __restrict__ scores,
    int32_t* __restrict__ kept) {
  constexpr int NW = NT / 64;
  constexpr int BPT = kHistBins / NT;  // histogram bins per thread
  extern __shared__ uint32_t keys_s[];
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t sel[2];
  __shared__ uint32_t wsum[NW];

  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int s = unit / LH, lg = unit % LH;
  const SeqInfo si = seqs[s];
  const int n = si.n, b = si.b;
  if (b <= 0) return;
  const float* in = scores + si.row_base + (int64_t)lg * si.in_stride;
  int32_t* out = kept + si.out_base + (int64_t)lg * si.out_stride;
  if (b >= n) {
    for (int i = tid; i < n; i += NT) out[i] = i;
    return;
  }
#pragma unroll 8
  for (int i = tid; i < n; i += NT) keys_s[i] = order_key(in[i]);
  __syncthreads();

  uint32_t prefix = 0u, mask = 0u, kk = (uint32_t)b;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const uint32_t dmask = pass == 2 ? 0xffu : 0xfffu;
#pragma unroll
    for (int j = 0; j < BPT; ++j) hist[tid * BPT + j] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const uint32_t key = keys_s[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    // Thread t owns bins [t*BPT, (t+1)*BPT); find the bin holding rank kk
    // counted from the top.
    uint32_t c[BPT], mine = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      c[j] = hist[tid * BPT + j];
      mine += c[j];
    }
    uint32_t all = 0;
    const uint32_t below = block_excl_scan<NT>(mine, wsum, &all);
    uint32_t above = all - below - mine;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (above < kk && kk <= above + c[j]) {
        sel[0] = (uint32_t)(tid * BPT + j);
        sel[1] = above;
      }
      above += c[j];
    }
    __syncthreads();
    kk -= sel[1];
    prefix |= sel[0] << shift;
    mask |= dmask << shift;
    __syncthreads();
  }
  const uint32_t T = prefix, quota = kk;

  // Ordered emission: each thread owns kScanItems consecutive keys of a tile.
  uint32_t base_out = 0, base_eq = 0;
  constexpr int kTile = NT * kScanItems;
  for (int tile = 0; tile < n && base_out < (uint32_t)b; tile += kTile) {
    const int i0 = tile + tid * kScanItems;
    uint32_t kv[kScanItems];
    uint32_t neq = 0;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
      kv[j] = (i0 + j < n) ? keys_s[i0 + j] : 0u;
      neq += (i0 + j < n && kv[j] == T) ? 1u : 0u;
    }
    uint32_t eq_tile = 0;
    const uint32_t eq_before = base_eq + block_excl_scan<NT>(neq, wsum, &eq_tile);
    uint32_t nkeep = 0;
    uint32_t e = eq_before;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
      const bool valid = i0 + j < n;
      const bool gt = valid && kv[j] > T;
      const bool eq = valid && kv[j] == T;
      nkeep += (gt || (eq && e < quota)) ? 1u : 0u;
      e += eq ? 1u : 0u;
    }
    uint32_t keep_tile = 0;
    uint32_t pos = base_out + block_excl_scan<NT>(nkeep, wsum, &keep_tile);
    e = eq_before;
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
      const bool valid = i0 + j < n;
      const bool gt = valid && kv[j] > T;
      const bool eq = valid && kv[j] == T;
      if (gt || (eq && e < quota)) {
        if (pos < (uint32_t)b) out[pos] = i0 + j;
        ++pos;
      }
      e += eq ? 1u : 0u;
    }
    base_out += keep_tile;
    base_eq += eq_tile;
  }
}

// Find the bin of hist (kHistBins bins, counts) that holds rank kk counted
// from the top: thread t owns bins [t*BPT, (t+1)*BPT).  Returns the bin and
// sets *above_out to the count in higher bins (all threads get both).
template <int NT>
__device__ __forceinline__ uint32_t pick_bin(const uint32_t* hist, uint32_t kk, uint32_t* sel,
                                             uint32_t* wsum, uint32_t* above_out) {
  constexpr int BPT = kHistBins / NT;
  const int tid = threadIdx.x;
  uint32_t c[BPT], mine = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    c[j] = hist[tid * BPT + j];
    mine += c[j];
  }
  uint32_t all = 0;
  const uint32_t below = block_excl_scan<NT>(mine, wsum, &all);
  uint32_t above = all - below - mine;
#pragma unroll
  for (int j = BPT - 1; j >= 0; --j) {
    if (above < kk && kk <= above + c[j]) {
      sel[0] = (uint32_t)(tid * BPT + j);
      sel[1] = above;
    }
    above += c[j];
  }
  __syncthreads();
  const uint32_t bin = sel[0];
  *above_out = sel[1];
  __syncthreads();
  return bin;
}

// Longest unit one work-group selects (the streaming select); longer units
// take the split select.
constexpr int kSelLdsMaxKeys = 35840;

// ---------------------------------------------------------------------------
// Streaming select for units of 4096 < n <= kSelLdsMaxKeys.  The keys stay
// in neither registers nor LDS (32 KB per work-group), so four work-groups
// share a CU and one group's reads overlap another's arithmetic.  Wave w
// owns the contiguous index segment [w*seg, w*seg + seg) and reads it 64
// consecutive keys at a time: counts per wave are counts per segment, and
// the ordered emission needs one scan over the NW wave totals.
//   sweep 1: histogram of the top 12 key bits; pick that digit (bin0).
//   sweep 2: keys above bin0 are counted per wave, the indices of keys in
//            bin0 go to an LDS list; the 12- and 8-bit lower digits are
//            found over the listed keys alone.  If the list overflows
//            (heavy ties), two more sweeps find them over the whole unit.
//   sweep 3: each wave writes its kept indices in index order; ballots
//            give each lane its rank among the wave's equal and kept keys.
// Sweeps 2 and 3 compare the scores as floats against thresholds derived
// from key bounds (key_floor), which costs one compare per bound instead of
// a key conversion.  Sweep 1 reads HBM; sweeps 2 and 3 mostly hit the
// caches.
// ---------------------------------------------------------------------------
constexpr int kStreamThreads = 512;
constexpr int kStreamCand = 4096;  // candidate indices (16 KB)
constexpr int kStreamBatch = 8;    // loads in flight per lane

// For K in [1, 2^32): order_key(x) >= K  <=>  x >= key_floor(K) (float
// compare, false for NaN).  Keys at or above 2^31 are the non-negative
// floats (and -0) in bit order; keys below it the negative floats in
// reverse bit order, so the bound is the float whose key is K.  Keys in
// [1, 0x007fffff) belong to NaN bit patterns, which key to 0, so such K
// are raised to the key of -inf; K above the key of +inf give a NaN bound,
// which nothing reaches.  K == 0 (every key, NaN included) is the caller's.
__device__ __forceinline__ float key_floor(uint32_t K) {
  K = K < 0x007fffffu ? 0x007fffffu : K;
  return __uint_as_float((K & 0x80000000u) ? (K & 0x7fffffffu) : ~K);
}

// number of set bits of mask held by lanes below this one
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// sum over the wave's 64 lanes, in every lane
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// a[0] + ... + a[w - 1] for a wave-uniform w <= 64, one entry per lane
__device__ __forceinline__ uint32_t sum_below(const uint32_t* a, int w) {
  const int lane = threadIdx.x & 63;
  return __builtin_amdgcn_readfirstlane(wave_sum(lane < w ? a[lane] : 0u));
}

// Calls f(i, valid, x) for each score of the wave's segment [s0, s0 + seg)
// (seg a multiple of 64; scores at i >= s1 invalid), kStreamBatch loads in
// flight per lane.  Every lane of the wave makes every call.
template <class F>
__device__ __forceinline__ void sweep_segment(const float* __restrict__ in, int s0, int seg, int s1,
                                              F&& f) {
  const int lane = threadIdx.x & 63;
  int base = s0;
  for (; base + 64 * kStreamBatch <= s1; base += 64 * kStreamBatch) {
    float v[kStreamBatch];
#pragma unroll
    for (int u = 0; u < kStreamBatch; ++u) v[u] = in[base + u * 64 + lane];
#pragma unroll
    for (int u = 0; u < kStreamBatch; ++u) f(base + u * 64 + lane, true, v[u]);
  }
  for (; base < s1; base += 64 * kStreamBatch) {
    float v[kStreamBatch];
#pragma unroll
    for (int u = 0; u < kStreamBatch; ++u) {
      const int i = base + u * 64 + lane;
      v[u] = i < s1 ? in[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kStreamBatch; ++u) {
      const int i = base + u * 64 + lane;
      f(i, i < s1, v[u]);
    }
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void select_stream_kernel(
    const SeqInfo* __restrict__ seqs, int LH, const float* __restrict__ scores,
    int32_t* __restrict__ kept) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t cand[kStreamCand];
  __shared__ uint32_t sel[2];
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t wgt[NW], weq[NW];
  __shared__ uint32_t ncand;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x;
  const int s = unit / LH, lg = unit % LH;
  const SeqInfo si = seqs[s];
  const int n = si.n, b = si.b;
  if (b <= 0) return;
  const float* in = scores + si.row_base + (int64_t)lg * si.in_stride;
  int32_t* out = kept + si.out_base + (int64_t)lg * si.out_stride;
  if (b >= n) {
    for (int i = tid; i < n; i += NT) out[i] = i;
    return;
  }
  const int seg = (n + NW * 64 - 1) / (NW * 64) * 64;
  const int s0 = wave * seg, s1 = min(n, s0 + seg);

  // sweep 1: top digit
  for (int i = tid; i < kHistBins; i += NT) hist[i] = 0u;
  if (tid < NW) {
    wgt[tid] = 0u;
    weq[tid] = 0u;
  }
  if (tid == 0) ncand = 0u;
  __syncthreads();
  sweep_segment(in, s0, seg, s1, [&](int, bool valid, float x) {
    if (valid) atomicAdd(&hist[order_key(x) >> 20], 1u);
  });
  __syncthreads();
  uint32_t above = 0;
  const uint32_t bin0 = pick_bin<NT>(hist, (uint32_t)b, sel, wsum, &above);
  uint32_t kk = (uint32_t)b - above;

  // sweep 2: keys above bin0 counted, keys in bin0 listed.  bin0 holds the
  // b-th largest key, so bin0 << 20 > 0 unless that key is a NaN's.
  const float lo_f = key_floor(bin0 << 20), hi_f = key_floor((bin0 + 1u) << 20);
  const bool lo_all = bin0 == 0u;
  uint32_t hi = 0;  // wave-uniform
  sweep_segment(in, s0, seg, s1, [&](int i, bool valid, float x) {
    const bool up = valid && x >= hi_f;
    hi += (uint32_t)__popcll(__ballot(up));
    const bool c = valid && !up && (lo_all || x >= lo_f);
    const uint64_t cm = __ballot(c);
    if (cm != 0) {
      uint32_t first = 0;
      if (lane == 0) first = atomicAdd(&ncand, (uint32_t)__popcll(cm));
      const uint32_t slot = (uint32_t)__shfl(first, 0, 64) + lanes_below(cm);
      if (c && slot < (uint32_t)kStreamCand) cand[slot] = (uint32_t)i;
    }
  });
  __syncthreads();
  const uint32_t nc = ncand;
  const bool listed = nc <= (uint32_t)kStreamCand;
  uint32_t prefix = bin0 << 20, mask = 0xfff00000u;
#pragma unroll 1
  for (int pass = 1; pass < 3; ++pass) {
    const int shift = pass == 1 ? 8 : 0;
    const uint32_t dmask = pass == 1 ? 0xfffu : 0xffu;
    for (int i = tid; i < kHistBins; i += NT) hist[i] = 0u;
    __syncthreads();
    if (listed) {
      for (uint32_t c = tid; c < nc; c += NT) {
        const uint32_t key = order_key(in[cand[c]]);
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
      }
    } else {
      sweep_segment(in, s0, seg, s1, [&](int, bool valid, float x) {
        const uint32_t key = order_key(x);
        if (valid && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
      });
    }
    __syncthreads();
    const uint32_t bin = pick_bin<NT>(hist, kk, sel, wsum, &above);
    kk -= above;
    prefix |= bin << shift;
    mask |= dmask << shift;
  }
  const uint32_t T = prefix, quota = kk;
  // key > T <=> x >= gt_f (T is a present key, at most that of +inf, so
  // T + 1 does not wrap); key == T <=> eq_all or x >= eq_f, and not above
  const float gt_f = key_floor(T + 1u), eq_f = key_floor(T);
  const bool eq_all = T == 0u;

  // keys > T and == T per segment
  if (listed) {
    if (lane == 0) atomicAdd(&wgt[wave], hi);
    for (uint32_t c = tid; c < nc; c += NT) {
      const uint32_t i = cand[c];
      const float x = in[i];
      if (x >= gt_f) atomicAdd(&wgt[i / (uint32_t)seg], 1u);
      else if (eq_all || x >= eq_f) atomicAdd(&weq[i / (uint32_t)seg], 1u);
    }
  } else {
    uint32_t gt = 0, eq = 0;
    sweep_segment(in, s0, seg, s1, [&](int, bool valid, float x) {
      const bool up = valid && x >= gt_f;
      gt += (uint32_t)__popcll(__ballot(up));
      eq += (uint32_t)__popcll(__ballot(valid && !up && (eq_all || x >= eq_f)));
    });
    if (lane == 0) {
      wgt[wave] = gt;
      weq[wave] = eq;
    }
  }
  __syncthreads();
  uint32_t gt_before = 0, eq_before = 0;
  for (int w = 0; w < wave; ++w) {  // wave-uniform trip count
    gt_before += wgt[w];
    eq_before += weq[w];
  }
  const uint32_t eq_left = quota > eq_before ? quota - eq_before : 0u;
  if (wgt[wave] + min(eq_left, weq[wave]) == 0u) return;  // nothing kept in this segment

  // sweep 3: ordered emission
  uint32_t pos0 = gt_before + min(quota, eq_before), eq_run = eq_before;
  sweep_segment(in, s0, seg, s1, [&](int i, bool valid, float x) {
    const bool up = valid && x >= gt_f;
    const uint64_t em = __ballot(valid && !up && (eq_all || x >= eq_f));
    bool keep = up;
    if (em != 0) {  // keys equal to T: the first `quota` of the unit are kept
      const bool eq = (em >> lane) & 1u;
      keep = up || (eq && eq_run + lanes_below(em) < quota);
      eq_run += (uint32_t)__popcll(em);
    }
    const uint64_t km = __ballot(keep);
    const uint32_t pos = pos0 + lanes_below(km);
    if (keep && pos < (uint32_t)b) out[pos] = i;
    pos0 += (uint32_t)__popcll(km);
  });
}

// ---------------------------------------------------------------------------
// Register-held select for units of 4096 < n <= NT*KPT: the streaming
// select's steps with the unit's order keys read once into registers (KPT
// per lane; lane l of wave w holds indices w*64*KPT + 64*j + l), so no
// score is read twice and every bound is an integer compare.  Keys in the
// top-digit bin are listed with their index, so the lower digits cost one
// pass over the list; if the list overflows, over the held keys.  At most
// 64 VGPRs, so that two work-groups of 1024 threads share a CU.
// ---------------------------------------------------------------------------
constexpr int kHeldCand = 4096;  // listed keys and their indices (32 KB), split over the waves

// A copy of x the compiler cannot see through: per-lane values derived from
// it in a later phase are recomputed there instead of being kept live from
// an earlier one.
__device__ __forceinline__ int fresh(int x) {
  int r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// One unit's selection by one work-group of NT threads, 0 < b < n; writes
// the b kept indices to out.  Every thread calls it (it holds barriers).
template <int NT, int KPT>
__device__ __forceinline__ void held_select(const float* __restrict__ in, int32_t* __restrict__ out,
                                            int n, int b, uint32_t* __restrict__ buf,
                                            bool keep_in_lds) {
  constexpr int NW = NT / 64, SEG = 64 * KPT;
  uint32_t* const hist = buf;                            // kHistBins
  uint32_t* const cand_key = buf + kHistBins;            // kHeldCand
  uint32_t* const cand_idx = buf + kHistBins + kHeldCand;  // kHeldCand
  __shared__ uint32_t sel[2];
  __shared__ uint32_t wsum[NW];
  __shared__ uint32_t wgt[NW], weq[NW], wcnt[NW];
  constexpr int kHeldWaveCand = kHeldCand / NW;  // list entries per wave

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Places past n hold key 0 (a NaN's): they join the histograms and the
  // list as NaNs whose indices follow every real key, so they rank after
  // every real NaN, and the b < n real keys fill the budget before them.
  const int s0 = wave * SEG + lane;
  uint32_t key[KPT];
  if (wave * SEG + SEG <= n) {  // the whole range real: unconditional loads, all in flight
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = order_key(in[s0 + 64 * j]);
  } else {  // the wave holding the unit's end: per 64-key step, whole, partial or past n
    const int w0 = wave * SEG;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (w0 + 64 * j + 64 <= n)
        key[j] = order_key(in[s0 + 64 * j]);
      else if (w0 + 64 * j < n)
        key[j] = s0 + 64 * j < n ? order_key(in[s0 + 64 * j]) : 0u;
      else
        key[j] = 0u;
    }
  }

  for (int i = tid; i < kHistBins; i += NT) hist[i] = 0u;
  __syncthreads();
  // top digit
#pragma unroll
  for (int j = 0; j < KPT; ++j) atomicAdd(&hist[key[j] >> 20], 1u);
  __syncthreads();
  uint32_t above = 0;
  const uint32_t bin0 = pick_bin<NT>(hist, (uint32_t)b, sel, wsum, &above);
  uint32_t kk = (uint32_t)b - above;

  // keys above bin0 counted per wave; keys in bin0 listed, each wave in its
  // own part of the list (no atomics: the wave keeps its count in a scalar)
  const uint32_t lo = bin0 << 20, hi_k = (bin0 + 1u) << 20;  // bin0 <= 0xff8: no wrap
  uint32_t hi = 0, cnt = 0;  // wave-uniform
  const int s0c = fresh(s0);
  uint32_t* const my_key = cand_key + wave * kHeldWaveCand;
  uint32_t* const my_idx = cand_idx + wave * kHeldWaveCand;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    hi += (uint32_t)__popcll(__ballot(key[j] >= hi_k));
    asm volatile("" : "+s"(hi));  // count now: a deferred count holds its mask in SGPRs
    const bool c = key[j] >= lo && key[j] < hi_k;
    const uint64_t cm = __ballot(c);
    if (cm != 0) {
      const uint32_t slot = cnt + lanes_below(cm);
      if (c && slot < (uint32_t)kHeldWaveCand) {
        my_key[slot] = key[j];
        my_idx[slot] = (uint32_t)(s0c + 64 * j);
      }
      cnt += (uint32_t)__popcll(cm);
    }
  }
  if (lane == 0) wcnt[wave] = cnt;
  __syncthreads();
  const bool listed =
      __ballot(lane < NW && wcnt[lane < NW ? lane : 0] > (uint32_t)kHeldWaveCand) == 0;
  uint32_t prefix = lo, mask = 0xfff00000u;
#pragma unroll 1
  for (int pass = 1; pass < 3; ++pass) {
    const int shift = pass == 1 ? 8 : 0;
    const uint32_t dmask = pass == 1 ? 0xfffu : 0xffu;
    for (int i = tid; i < kHistBins; i += NT) hist[i] = 0u;
    __syncthreads();
    if (listed) {
      for (int c = tid; c < kHeldCand; c += NT) {
        if ((uint32_t)(c % kHeldWaveCand) < wcnt[c / kHeldWaveCand]) {
          const uint32_t k = cand_key[c];
          if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if ((key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
    }
    __syncthreads();
    const uint32_t bin = pick_bin<NT>(hist, kk, sel, wsum, &above);
    kk -= above;
    prefix |= bin << shift;
    mask |= dmask << shift;
  }
  const uint32_t T = prefix, quota = kk;

  // keys > T and == T per wave: from the wave's own list, or its held keys
  uint32_t gt = 0, eq = 0;
  if (listed) {
    for (uint32_t c = lane; c < cnt; c += 64) {
      const uint32_t k = my_key[c];
      gt += k > T ? 1u : 0u;
      eq += k == T ? 1u : 0u;
    }
    gt = hi + __builtin_amdgcn_readfirstlane(wave_sum(gt));  // listed keys above T, and above bin0
    eq = __builtin_amdgcn_readfirstlane(wave_sum(eq));
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      gt += (uint32_t)__popcll(__ballot(key[j] > T));
      eq += (uint32_t)__popcll(__ballot(key[j] == T));
    }
  }
  if (lane == 0) {
    wgt[wave] = gt;
    weq[wave] = eq;
  }
  __syncthreads();
  const uint32_t gt_before = sum_below(wgt, wave), eq_before = sum_below(weq, wave);
  const uint32_t eq_left = quota > eq_before ? quota - eq_before : 0u;
  if (gt + min(eq_left, eq) == 0u) return;  // nothing kept in this wave's range

  // ordered emission
  uint32_t pos0 = gt_before + min(quota, eq_before), eq_run = eq_before;
  const int s0e = fresh(s0);
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const uint64_t em = __ballot(key[j] == T);
    bool keep = key[j] > T;
    if (em != 0) {  // keys equal to T: the first `quota` of the unit are kept
      keep = keep || (key[j] == T && eq_run + lanes_below(em) < quota);
      eq_run += (uint32_t)__popcll(em);
    }
    const uint64_t km = __ballot(keep);
    const uint32_t pos = pos0 + lanes_below(km);
    if (keep && pos < (uint32_t)b) {
      out[pos] = s0e + 64 * j;
      if (keep_in_lds) buf[pos] = s0e + 64 * j;  // the lists are dead by now
    }
    pos0 += (uint32_t)__popcll(km);
  }
}

// Rows of the gathers (K, V, positions), packed or through page tables.
struct CompactArgs {
  int d;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* k_pos;
  uint16_t* k_out;
  uint16_t* v_out;
  int32_t* pos_out;
  Pages in_pg, out_pg;
};

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Moves part `part` (16 bytes) of kept row r (input row idx of unit
// (s, lg)) of K and V, and its position from part 0.  Rows move whole,
// read once and written once: non-temporal on both sides.
__device__ __forceinline__ void copy_row_part(const CompactArgs& ca, int s, int lg, int64_t in0,
                                              int64_t out0, int idx, int r, int part) {
  const int64_t src = ca.in_pg.table ? paged_row_lg(ca.in_pg, s, lg, idx) : in0 + idx;
  const int64_t dst = ca.out_pg.table ? paged_row_lg(ca.out_pg, s, lg, r) : out0 + r;
  if (ca.k_out)
    __builtin_nontemporal_store(
        __builtin_nontemporal_load(reinterpret_cast<const v4u*>(ca.k + src * ca.d) + part),
        reinterpret_cast<v4u*>(ca.k_out + dst * ca.d) + part);
  if (ca.v_out)
    __builtin_nontemporal_store(
        __builtin_nontemporal_load(reinterpret_cast<const v4u*>(ca.v + src * ca.d) + part),
        reinterpret_cast<v4u*>(ca.v_out + dst * ca.d) + part);
  if (ca.pos_out && part == 0) ca.pos_out[dst] = ca.k_pos[src];
}

// Register-held select of one unit per work-group; with COPY the same
// work-group then gathers the unit's kept rows (the kept indices it just
// wrote, read back after a barrier), so that one work-group's selection
// overlaps another's copy on the same CU.  Units below `presel` were
// selected by an earlier launch: their work-groups only gather, so the
// kernel starts with copies under way instead of every resident
// work-group selecting at once.
template <int NT, int KPT, bool COPY>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void select_held_kernel(
    const SeqInfo* __restrict__ seqs, int LH, const float* __restrict__ scores,
    int32_t* __restrict__ kept, const CompactArgs ca, int presel) {
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const int s = unit / LH, lg = unit % LH;
  const SeqInfo si = seqs[s];
  const int n = si.n, b = si.b;
  if (b <= 0) return;
  const int64_t in0 = si.row_base + (int64_t)lg * si.in_stride;
  const int64_t out0 = si.out_base + (int64_t)lg * si.out_stride;
  int32_t* out = kept + out0;
  // histogram and lists of the selection; afterwards, when the gathers
  // follow and b fits, the kept indices
  __shared__ uint32_t buf[kHistBins + 2 * kHeldCand];
  const bool in_lds = COPY && unit >= presel && b <= kHistBins + 2 * kHeldCand;
  if (unit < presel) {
    // kept indices already written
  } else if (b >= n) {
    for (int i = tid; i < n; i += NT) {
      out[i] = i;
      if (in_lds) buf[i] = i;
    }
  } else {
    held_select<NT, KPT>(scores + in0, out, n, b, buf, in_lds);
  }
  if constexpr (COPY) {
    // The unit's kept indices, written by this work-group: from LDS when
    // they fit, else from L2 after the barrier (agent-scope loads skip the
    // CU's L1, which may hold a line shared with a neighbouring unit's
    // indices from before they were written).
    __syncthreads();
    const int lpr = ca.d >> 3;  // lanes per row, 16 bytes each
    const int rows_per_pass = NT / lpr;
    const int sub = tid / lpr, part = tid - sub * lpr;
#pragma unroll 2
    for (int r = sub < rows_per_pass ? sub : b; r < b; r += rows_per_pass) {
      const int idx = in_lds ? (int)buf[r]
                             : __hip_atomic_load(out + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((uint32_t)idx < (uint32_t)n) copy_row_part(ca, s, lg, in0, out0, idx, r, part);
    }
  }
}

// The selection of the first units of a call whose plan travels in the
// launch's arguments: block 0 also writes the plan to seqs, where the
// gathering kernel that follows reads it.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8))) void select_first_kernel(
    SeqInfo* __restrict__ seqs, const ArgWords plan, int plan_words, int LH,
    const float* __restrict__ scores, int32_t* __restrict__ kept) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < plan_words; i += NT)
      reinterpret_cast<uint32_t*>(seqs)[i] = plan.w[i];
  const int unit = blockIdx.x;
  const int s = unit / LH, lg = unit % LH;
  const SeqInfo si = reinterpret_cast<const SeqInfo*>(plan.w)[s];
  const int n = si.n, b = si.b;
  if (b <= 0) return;
  const int64_t in0 = si.row_base + (int64_t)lg * si.in_stride;
  int32_t* out = kept + si.out_base + (int64_t)lg * si.out_stride;
  __shared__ uint32_t buf[kHistBins + 2 * kHeldCand];
  if (b >= n) {
    for (int i = threadIdx.x; i < n; i += NT) out[i] = i;
  } else {
    held_select<NT, KPT>(scores + in0, out, n, b, buf, false);
  }
}

// ---------------------------------------------------------------------------
// Split select for units longer than the LDS-staged select holds: the unit
// is cut into tiles of kSplitTile keys, one work-group each, so that a few
// long units still spread over the chip.  Digits are 8 bits wide (4
// passes).  In each pass every tile stores its histogram of the keys that
// match the digits found so far, and a one-work-group-per-unit pick kernel
// adds the tiles' histograms and picks the digit.  Then a count pass
// records per tile the keys above the threshold T and equal to it, and a
// write pass places each tile's kept indices after those of the tiles
// before it: ahead of tile t sit every key > T of tiles < t and
// min(quota, keys == T in tiles < t).  Kernel boundaries order the steps;
// there are no atomics and no fences (a device-wide fence writes back the
// L2 on this chip, which cost more than the passes themselves).
// ---------------------------------------------------------------------------
constexpr int kSplitThreads = 256;
constexpr int kSplitWaves = kSplitThreads / 64;
constexpr int kSplitItems = 16;
constexpr int kSplitTile = kSplitThreads * kSplitItems;  // 4096 keys

// per unit: digits found (prefix, mask) and the rank still to place (kk)
struct SplitState {
  uint32_t prefix, mask, kk, pad;
};

struct SplitBuffers {
  SplitState* state;  // [units]
  uint32_t* hist;     // [units][tiles][256], the current pass
  uint2* counts;      // [units][tiles]: (keys > T, keys == T)
};

static size_t split_up(int64_t x) { return (size_t)((x + 255) / 256 * 256); }

static SplitBuffers split_buffers(void* ws, int64_t units, int64_t tiles) {
  char* p = (char*)ws;
  SplitBuffers sb;
  sb.state = (SplitState*)p;
  p += split_up(units * (int64_t)sizeof(SplitState));
  sb.hist = (uint32_t*)p;
  p += split_up(units * tiles * 256 * 4);
  sb.counts = (uint2*)p;
  return sb;
}

size_t split_select_bytes(int64_t units, int max_n) {
  if (max_n <= kSelLdsMaxKeys || units <= 0) return 0;
  const int64_t tiles = (max_n + kSplitTile - 1) / kSplitTile;
  return split_up(units * (int64_t)sizeof(SplitState)) + split_up(units * tiles * 256 * 4) +
         split_up(units * tiles * (int64_t)sizeof(uint2));
}

// Work-group's tile of one unit (grid units*tiles); false: nothing to do.
struct SplitTile {
  int unit, tile, n, b;
  int64_t t0;
  const float* in;
  int32_t* out;
};

__device__ __forceinline__ SplitTile split_tile(const SeqInfo* seqs, int LH, int tiles,
                                                const float* scores, int32_t* kept) {
  SplitTile t;
  t.unit = blockIdx.x / tiles;
  t.tile = blockIdx.x % tiles;
  const SeqInfo si = seqs[t.unit / LH];
  const int lg = t.unit % LH;
  t.n = si.n;
  t.b = si.b;
  t.t0 = (int64_t)t.tile * kSplitTile;
  t.in = scores + si.row_base + (int64_t)lg * si.in_stride;
  t.out = kept ? kept + si.out_base + (int64_t)lg * si.out_stride : nullptr;
  return t;
}

// One radix pass (digit bits [24 - 8*pass, 32 - 8*pass)): the tile's
// histogram of the keys that match the digits found so far.
__global__ __launch_bounds__(kSplitThreads) void split_hist_kernel(
    const SeqInfo* __restrict__ seqs, int LH, int tiles, const float* __restrict__ scores,
    int pass, SplitBuffers sb) {
  __shared__ uint32_t h[kSplitWaves][256];
  const int tid = threadIdx.x, wave = tid >> 6;
  const SplitTile t = split_tile(seqs, LH, tiles, scores, nullptr);
  if (t.b <= 0 || t.b >= t.n || t.t0 >= t.n) return;
  uint32_t prefix = 0u, mask = 0u;
  if (pass > 0) {
    const SplitState st = sb.state[t.unit];
    prefix = st.prefix;
    mask = st.mask;
  }
  const int shift = 24 - 8 * pass;
  for (int i = tid; i < kSplitWaves * 256; i += kSplitThreads) (&h[0][0])[i] = 0u;
  __syncthreads();
  float v[kSplitItems];  // all loads in flight before the first LDS atomic
#pragma unroll
  for (int j = 0; j < kSplitItems; ++j) {
    const int64_t i = t.t0 + j * kSplitThreads + tid;
    v[j] = t.in[i < t.n ? i : t.n - 1];
  }
#pragma unroll
  for (int j = 0; j < kSplitItems; ++j) {
    const uint32_t key = order_key(v[j]);
    if (t.t0 + j * kSplitThreads + tid < t.n && (key & mask) == prefix)
      atomicAdd(&h[wave][(key >> shift) & 255u], 1u);
  }
  __syncthreads();
  uint32_t c = 0;
#pragma unroll
  for (int w = 0; w < kSplitWaves; ++w) c += h[w][tid];
  sb.hist[((int64_t)t.unit * tiles + t.tile) * 256 + tid] = c;
}

// The digit of one pass per unit: the bin holding rank kk (from the top) of
// the sum of the tiles' histograms.  Grid units, thread = bin.
__global__ __launch_bounds__(kSplitThreads) void split_pick_kernel(
    const SeqInfo* __restrict__ seqs, int LH, int tiles, int pass, SplitBuffers sb) {
  __shared__ uint32_t wsum[kSplitWaves];
  const int tid = threadIdx.x;
  const int unit = blockIdx.x;
  const SeqInfo si = seqs[unit / LH];
  const int n = si.n, b = si.b;
  if (b <= 0 || b >= n) return;
  const int unit_tiles = (n + kSplitTile - 1) / kSplitTile;
  SplitState st = {0u, 0u, (uint32_t)b, 0u};
  if (pass > 0) st = sb.state[unit];
  const uint32_t* hh = sb.hist + (int64_t)unit * tiles * 256 + tid;
  uint32_t c = 0;
#pragma unroll 8
  for (int t = 0; t < unit_tiles; ++t) c += hh[(int64_t)t * 256];
  uint32_t all = 0;
  const uint32_t below = block_excl_scan<kSplitThreads>(c, wsum, &all);
  const uint32_t above = all - below - c;  // keys in higher bins
  const int shift = 24 - 8 * pass;
  if (above < st.kk && st.kk <= above + c)
    sb.state[unit] = SplitState{st.prefix | ((uint32_t)tid << shift), st.mask | (255u << shift),
                                st.kk - above, 0u};
}

// Keys above the threshold and equal to it, per tile.
__global__ __launch_bounds__(kSplitThreads) void split_count_kernel(
    const SeqInfo* __restrict__ seqs, int LH, int tiles, const float* __restrict__ scores,
    SplitBuffers sb) {
  __shared__ uint32_t wgt[kSplitWaves], weq[kSplitWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const SplitTile t = split_tile(seqs, LH, tiles, scores, nullptr);
  if (t.b <= 0 || t.b >= t.n || t.t0 >= t.n) return;
  const uint32_t T = sb.state[t.unit].prefix;
  float v[kSplitItems];
#pragma unroll
  for (int j = 0; j < kSplitItems; ++j) {
    const int64_t i = t.t0 + j * kSplitThreads + tid;
    v[j] = t.in[i < t.n ? i : t.n - 1];
  }
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kSplitItems; ++j) {
    const uint32_t key = order_key(v[j]);
    const bool valid = t.t0 + j * kSplitThreads + tid < t.n;
    gt += (valid && key > T) ? 1u : 0u;
    eq += (valid && key == T) ? 1u : 0u;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    gt += __shfl_xor(gt, o, 64);
    eq += __shfl_xor(eq, o, 64);
  }
  if (lane == 0) {
    wgt[wave] = gt;
    weq[wave] = eq;
  }
  __syncthreads();
  if (tid == 0) {
    uint2 r = make_uint2(0u, 0u);
    for (int w = 0; w < kSplitWaves; ++w) {
      r.x += wgt[w];
      r.y += weq[w];
    }
    sb.counts[(int64_t)t.unit * tiles + t.tile] = r;
  }
}

// Kept indices of each tile in index order; thread i takes the tile's keys
// [i*kSplitItems, (i+1)*kSplitItems).
__global__ __launch_bounds__(kSplitThreads) void split_write_kernel(
    const SeqInfo* __restrict__ seqs, int LH, int tiles, const float* __restrict__ scores,
    SplitBuffers sb, int32_t* __restrict__ kept) {
  __shared__ uint32_t wsum[kSplitWaves];
  __shared__ uint32_t wa[kSplitWaves], wb[kSplitWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const SplitTile t = split_tile(seqs, LH, tiles, scores, kept);
  const int n = t.n, b = t.b;
  if (b <= 0 || t.t0 >= n) return;
  const int i0 = (int)t.t0 + tid * kSplitItems;
  if (b >= n) {
#pragma unroll
    for (int j = 0; j < kSplitItems; ++j)
      if (i0 + j < n) t.out[i0 + j] = i0 + j;
    return;
  }
  const SplitState st = sb.state[t.unit];
  const uint32_t T = st.prefix, quota = st.kk;
  // keys > T and == T in the tiles before this one
  uint32_t gt_before = 0, eq_before_tiles = 0;
  for (int p = tid; p < t.tile; p += kSplitThreads) {
    const uint2 c = sb.counts[(int64_t)t.unit * tiles + p];
    gt_before += c.x;
    eq_before_tiles += c.y;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    gt_before += __shfl_xor(gt_before, o, 64);
    eq_before_tiles += __shfl_xor(eq_before_tiles, o, 64);
  }
  if (lane == 0) {
    wa[wave] = gt_before;
    wb[wave] = eq_before_tiles;
  }
  __syncthreads();
  gt_before = 0;
  eq_before_tiles = 0;
#pragma unroll
  for (int w = 0; w < kSplitWaves; ++w) {
    gt_before += wa[w];
    eq_before_tiles += wb[w];
  }
  uint32_t key[kSplitItems];
  const int mine = max(0, min(kSplitItems, n - i0));
#pragma unroll
  for (int j = 0; j < kSplitItems; ++j) key[j] = order_key(t.in[min(i0 + j, n - 1)]);
  uint32_t neq = 0;
#pragma unroll
  for (int j = 0; j < kSplitItems; ++j) neq += (j < mine && key[j] == T) ? 1u : 0u;
  uint32_t eq_tile = 0;
  const uint32_t eq_before =
      eq_before_tiles + block_excl_scan<kSplitThreads>(neq, wsum, &eq_tile);
  uint32_t nkeep = 0;
  {
    uint32_t e = eq_before;
#pragma unroll
    for (int j = 0; j < kSplitItems; ++j) {
      const bool valid = j < mine;
      const bool eq = valid && key[j] == T;
      nkeep += ((valid && key[j] > T) || (eq && e < quota)) ? 1u : 0u;
      e += eq ? 1u : 0u;
    }
  }
  uint32_t keep_tile = 0;
  uint32_t pos = gt_before + min(quota, eq_before_tiles) +
                 block_excl_scan<kSplitThreads>(nkeep, wsum, &keep_tile);
  uint32_t e = eq_before;
#pragma unroll
  for (int j = 0; j < kSplitItems; ++j) {
    const bool valid = j < mine;
    const bool eq = valid && key[j] == T;
    if ((valid && key[j] > T) || (eq && e < quota)) {
      if (pos < (uint32_t)b) t.out[pos] = i0 + j;
      ++pos;
    }
    e += eq ? 1u : 0u;
  }
}

constexpr int kSelSmallUnit = 4096;  // up to here 256 threads per unit

template <int NT>
static hipError_t launch_select_lds(int64_t units, int max_n, hipStream_t st, const SeqInfo* seqs,
                                    int LH, const float* scores, int32_t* kept_idx) {
  // at most kSelSmallUnit keys (16 KB) beside the 16 KB histogram: within
  // the default dynamic LDS limit
  const size_t lds = (size_t)(max_n > 0 ? max_n : 1) * sizeof(uint32_t);
  hipLaunchKernelGGL(select_lds_kernel<NT>, dim3((unsigned)units), dim3(NT), lds, st, seqs, LH,
                     scores, kept_idx);
  return hipGetLastError();
}

hipError_t launch_select(const SeqInfo* seqs, int S, int LH, int max_n, const float* scores,
                         int32_t* kept_idx, void* split_ws, hipStream_t st) {
  const int64_t units = (int64_t)S * LH;
  if (units == 0) return hipSuccess;
  if (max_n <= kSelSmallUnit)
    return launch_select_lds<256>(units, max_n, st, seqs, LH, scores, kept_idx);
  if (max_n <= 1024 * 16) {
    hipLaunchKernelGGL((select_held_kernel<1024, 16, false>), dim3((unsigned)units), dim3(1024), 0,
                       st, seqs, LH, scores, kept_idx, CompactArgs{}, 0);
    return hipGetLastError();
  }
  if (max_n <= 1024 * 32) {
    hipLaunchKernelGGL((select_held_kernel<1024, 32, false>), dim3((unsigned)units), dim3(1024), 0,
                       st, seqs, LH, scores, kept_idx, CompactArgs{}, 0);
    return hipGetLastError();
  }
  if (max_n <= kSelLdsMaxKeys) {
    hipLaunchKernelGGL(select_stream_kernel<kStreamThreads>, dim3((unsigned)units),
                       dim3(kStreamThreads), 0, st, seqs, LH, scores, kept_idx);
    return hipGetLastError();
  }
  if (!split_ws) return hipErrorInvalidValue;
  const int tiles = (max_n + kSplitTile - 1) / kSplitTile;
  if (units * tiles > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const SplitBuffers sb = split_buffers(split_ws, units, tiles);
  const dim3 grid((unsigned)(units * tiles)), block(kSplitThreads);
  hipError_t e = hipSuccess;
  for (int pass = 0; pass < 4 && e == hipSuccess; ++pass) {
    hipLaunchKernelGGL(split_hist_kernel, grid, block, 0, st, seqs, LH, tiles, scores, pass, sb);
    e = hipGetLastError();
    if (e != hipSuccess) break;
    hipLaunchKernelGGL(split_pick_kernel, dim3((unsigned)units), block, 0, st, seqs, LH, tiles,
                       pass, sb);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(split_count_kernel, grid, block, 0, st, seqs, LH, tiles, scores, sb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(split_write_kernel, grid, block, 0, st, seqs, LH, tiles, scores, sb,
                     kept_idx);
  return hipGetLastError();
}

// Gather kept rows.  Work-group (unit, tile) copies kCompactRows output rows;
// a group of d/8 lanes moves one row (16 bytes per lane) of K and of V, the
// first lane of the group the position.  Kept indices are always packed.
constexpr int kCompactRows = 64;

__global__ __launch_bounds__(256) void compact_kernel(const SeqInfo* __restrict__ seqs, int LH,
                                                      const int32_t* __restrict__ kept,
                                                      const CompactArgs ca) {
  const int unit = blockIdx.x;
  const int s = unit / LH, lg = unit % LH;
  const SeqInfo si = seqs[s];
  const int b = si.b;
  const int r0 = blockIdx.y * kCompactRows;
  if (r0 >= b) return;
  const int r1 = min(b, r0 + kCompactRows);
  const int lpr = ca.d >> 3;
  const int rows_per_pass = 256 / lpr;
  const int tid = threadIdx.x;
  const int sub = tid / lpr, part = tid - sub * lpr;
  if (sub >= rows_per_pass) return;
  const int64_t out0 = si.out_base + (int64_t)lg * si.out_stride;
  const int64_t in0 = si.row_base + (int64_t)lg * si.in_stride;
#pragma unroll 4
  for (int r = r0 + sub; r < r1; r += rows_per_pass) {
    const int32_t idx = kept[out0 + r];
    if ((uint32_t)idx >= (uint32_t)si.n) continue;  // never read outside the unit
    copy_row_part(ca, s, lg, in0, out0, idx, r, part);
  }
}

hipError_t launch_compact(const SeqInfo* seqs, int S, int LH, int d, int max_b,
                          const int32_t* kept_idx, const uint16_t* k, const uint16_t* v,
                          const int32_t* k_pos, uint16_t* k_out, uint16_t* v_out,
                          int32_t* pos_out, const Pages& in_pg, const Pages& out_pg,
                          hipStream_t st) {
  const int64_t units = (int64_t)S * LH;
  if (units == 0 || max_b <= 0) return hipSuccess;
  const dim3 grid((unsigned)units, (unsigned)((max_b + kCompactRows - 1) / kCompactRows));
  const CompactArgs ca{d, k, v, k_pos, k_out, v_out, pos_out, in_pg, out_pg};
  hipLaunchKernelGGL(compact_kernel, grid, dim3(256), 0, st, seqs, LH, kept_idx, ca);
  return hipGetLastError();
}

hipError_t launch_select_compact(SeqInfo* seqs, const SeqInfo* plan_host, int S, int LH, int d,
                                 int max_n, int max_b, const float* scores, int32_t* kept_idx,
                                 void* split_ws, const uint16_t* k, const uint16_t* v,
                                 const int32_t* k_pos, uint16_t* k_out, uint16_t* v_out,
                                 int32_t* pos_out, const Pages& in_pg, const Pages& out_pg,
                                 hipStream_t st) {
  const int64_t units = (int64_t)S * LH;
  const bool copy = k_out || v_out || pos_out;
  const size_t plan_bytes = (size_t)S * sizeof(SeqInfo);
  // the plan goes to the workspace by a copy kernel unless a first launch
  // below carries it
  auto write_plan = [&]() -> hipError_t {
    return plan_host && plan_bytes ? launch_write_args(seqs, plan_host, plan_bytes, st)
                                   : hipSuccess;
  };
  if (units > 0 && copy && max_n > kSelSmallUnit && max_n <= 1024 * 32) {
    // register-held select and the gathers in one kernel.  With more units
    // than two rounds of resident work-groups, one unit per CU is selected
    // first by a select-only launch (a fraction of the gathers' time), so
    // the gathering kernel starts with one work-group per CU copying while
    // the other selects.
    const CompactArgs ca{d, k, v, k_pos, k_out, v_out, pos_out, in_pg, out_pg};
    int presel = 0;
    {
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) == hipSuccess &&
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
          cus > 0 && units > 2 * (int64_t)cus)
        presel = cus;
    }
    const bool wide = max_n > 1024 * 16;
    ArgWords plan;
    const bool carry = presel > 0 && plan_host && plan_bytes <= sizeof(plan.w);
    if (!carry) {
      const hipError_t e = write_plan();
      if (e != hipSuccess) return e;
    }
    if (carry) {
      std::memcpy(plan.w, plan_host, plan_bytes);
      const int words = (int)(plan_bytes / 4);
      if (wide)
        hipLaunchKernelGGL((select_first_kernel<1024, 32>), dim3((unsigned)presel), dim3(1024), 0,
                           st, seqs, plan, words, LH, scores, kept_idx);
      else
        hipLaunchKernelGGL((select_first_kernel<1024, 16>), dim3((unsigned)presel), dim3(1024), 0,
                           st, seqs, plan, words, LH, scores, kept_idx);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    } else if (presel > 0) {
      if (wide)
        hipLaunchKernelGGL((select_held_kernel<1024, 32, false>), dim3((unsigned)presel),
                           dim3(1024), 0, st, seqs, LH, scores, kept_idx, CompactArgs{}, 0);
      else
        hipLaunchKernelGGL((select_held_kernel<1024, 16, false>), dim3((unsigned)presel),
                           dim3(1024), 0, st, seqs, LH, scores, kept_idx, CompactArgs{}, 0);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    if (wide)
      hipLaunchKernelGGL((select_held_kernel<1024, 32, true>), dim3((unsigned)units), dim3(1024),
                         0, st, seqs, LH, scores, kept_idx, ca, presel);
    else
      hipLaunchKernelGGL((select_held_kernel<1024, 16, true>), dim3((unsigned)units), dim3(1024),
                         0, st, seqs, LH, scores, kept_idx, ca, presel);
    return hipGetLastError();
  }
  hipError_t e = write_plan();
  if (e == hipSuccess) e = launch_select(seqs, S, LH, max_n, scores, kept_idx, split_ws, st);
  if (e != hipSuccess || !copy) return e;
  return launch_compact(seqs, S, LH, d, max_b, kept_idx, k, v, k_pos, k_out, v_out, pos_out, in_pg,
                        out_pg, st);
}

}  // namespace tri
