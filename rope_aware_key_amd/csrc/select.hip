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
// to T are kept (the quota).  A final ordered scan keeps every key > T and
// the first `quota` keys == T, writing their indices through block-wide
// prefix sums.  Units up to 35840 keys take one work-group (keys in
// registers or LDS); longer ones are split over work-groups of 4096 keys.
#include "tri_internal.hpp"

namespace tri {

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below every number
  if (u == 0x80000000u) u = 0u;                      // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// LDS-staged select: the unit's order keys are loaded once (coalesced) into
// LDS; the radix passes and the ordered scan then run on LDS.  Digits are
// 12, 12 and 8 bits wide: z-scores crowd a few exponent values, and 12-bit
// first digits (sign, exponent, 3 mantissa bits) spread them over enough
// bins that LDS atomics rarely collide.  NT threads per unit: 1024 for long
// units, 256 so that many short units share a CU.
// ---------------------------------------------------------------------------
constexpr int kHistBins = 4096;
constexpr int kScanItems = 8;  // consecutive keys per thread in the ordered scan

// Exclusive prefix sum over a block of NT threads; *total gets the sum.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = wsum[w];
    if (w < wave) before += t;
    all += t;
  }
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

// ---------------------------------------------------------------------------
// Register-resident select for units of up to NT*KPT keys: thread t holds
// keys [t*KPT, (t+1)*KPT) in registers, so LDS holds only the histogram and
// two work-groups share a CU.  Same digits and passes as select_lds_kernel;
// since each thread's keys are one contiguous index range, the ordered
// emission needs a single pair of block scans over per-thread counts.
// ---------------------------------------------------------------------------
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void select_reg_kernel(
    const SeqInfo* __restrict__ seqs, int LH, const float* __restrict__ scores,
    int32_t* __restrict__ kept) {
  constexpr int NW = NT / 64;
  static_assert(KPT % 4 == 0, "keys load as float4");
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
  const int i0 = tid * KPT;
  uint32_t key[KPT];
  if ((reinterpret_cast<uintptr_t>(in) & 15u) == 0 && i0 + KPT <= n) {
#pragma unroll
    for (int j = 0; j < KPT; j += 4) {
      const float4 f = *reinterpret_cast<const float4*>(in + i0 + j);
      key[j] = order_key(f.x);
      key[j + 1] = order_key(f.y);
      key[j + 2] = order_key(f.z);
      key[j + 3] = order_key(f.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < KPT; ++j) key[j] = i0 + j < n ? order_key(in[i0 + j]) : 0u;
  }
  // keys past n are 0 (the NaN key) and are excluded by index below
  const int mine = max(0, min(KPT, n - i0));

  uint32_t prefix = 0u, mask = 0u, kk = (uint32_t)b;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const uint32_t dmask = pass == 2 ? 0xffu : 0xfffu;
    for (int i = tid; i < kHistBins; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (j < mine && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
    __syncthreads();
    uint32_t above = 0;
    const uint32_t bin = pick_bin<NT>(hist, kk, sel, wsum, &above);
    kk -= above;
    prefix |= bin << shift;
    mask |= dmask << shift;
  }
  const uint32_t T = prefix, quota = kk;

  // Keys are blocked per thread, so a thread's counts cover a contiguous
  // index range: one scan of the per-thread totals orders the whole unit.
  uint32_t neq = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) neq += (j < mine && key[j] == T) ? 1u : 0u;
  uint32_t eq_all = 0;
  const uint32_t eq_before = block_excl_scan<NT>(neq, wsum, &eq_all);
  uint32_t nkeep = 0;
  {
    uint32_t e = eq_before;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool valid = j < mine;
      const bool gt = valid && key[j] > T;
      const bool eq = valid && key[j] == T;
      nkeep += (gt || (eq && e < quota)) ? 1u : 0u;
      e += eq ? 1u : 0u;
    }
  }
  uint32_t keep_all = 0;
  uint32_t pos = block_excl_scan<NT>(nkeep, wsum, &keep_all);
  uint32_t e = eq_before;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const bool valid = j < mine;
    const bool gt = valid && key[j] > T;
    const bool eq = valid && key[j] == T;
    if (gt || (eq && e < quota)) {
      if (pos < (uint32_t)b) out[pos] = i0 + j;
      ++pos;
    }
    e += eq ? 1u : 0u;
  }
}

// Longest unit whose keys the LDS-staged select holds (140 KB of keys next
// to the 16 KB histogram).
constexpr int kSelLdsMaxKeys = 35840;

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
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&select_lds_kernel<NT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, kSelLdsMaxKeys * (int)sizeof(uint32_t));
  if (attr != hipSuccess) return attr;
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
    hipLaunchKernelGGL((select_reg_kernel<1024, 16>), dim3((unsigned)units), dim3(1024), 0, st,
                       seqs, LH, scores, kept_idx);
    return hipGetLastError();
  }
  if (max_n <= 1024 * 32) {
    hipLaunchKernelGGL((select_reg_kernel<1024, 32>), dim3((unsigned)units), dim3(1024), 0, st,
                       seqs, LH, scores, kept_idx);
    return hipGetLastError();
  }
  if (max_n <= kSelLdsMaxKeys)
    return launch_select_lds<1024>(units, max_n, st, seqs, LH, scores, kept_idx);
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
// first lane of the group the position.
constexpr int kCompactRows = 64;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Rows of K, V and positions: packed, or through the input / output page
// tables (in_pg, out_pg); kept indices are always packed.
__global__ __launch_bounds__(256) void compact_kernel(
    const SeqInfo* __restrict__ seqs, int LH, int d, const int32_t* __restrict__ kept,
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ k_pos, uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out,
    int32_t* __restrict__ pos_out, const Pages in_pg, const Pages out_pg) {
  const int unit = blockIdx.x;
  const int s = unit / LH, lg = unit % LH;
  const SeqInfo si = seqs[s];
  const int b = si.b;
  const int r0 = blockIdx.y * kCompactRows;
  if (r0 >= b) return;
  const int r1 = min(b, r0 + kCompactRows);
  const int lpr = d >> 3;
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
    const int64_t src = in_pg.table ? paged_row_lg(in_pg, s, lg, idx) : in0 + idx;
    const int64_t dst = out_pg.table ? paged_row_lg(out_pg, s, lg, r) : out0 + r;
    // rows move whole (d/8 lanes x 16 bytes), read once and written once:
    // non-temporal on both sides
    if (k_out)
      __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const v4u*>(k + src * d) + part),
                                  reinterpret_cast<v4u*>(k_out + dst * d) + part);
    if (v_out)
      __builtin_nontemporal_store(__builtin_nontemporal_load(reinterpret_cast<const v4u*>(v + src * d) + part),
                                  reinterpret_cast<v4u*>(v_out + dst * d) + part);
    if (pos_out && part == 0) pos_out[dst] = k_pos[src];
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
  hipLaunchKernelGGL(compact_kernel, grid, dim3(256), 0, st, seqs, LH, d, kept_idx, k, v, k_pos,
                     k_out, v_out, pos_out, in_pg, out_pg);
  return hipGetLastError();
}

}  // namespace tri
