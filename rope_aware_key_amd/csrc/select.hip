// Top-B selection per unit with the lowest-index tie-break, emitting the
// kept indices in ascending (time) order.
//
// Semantics: talk page "聊聊 TriAttention", closing step (rank keys by the
// averaged score, keep the top B); jaedaily.cn tutorial, eviction step (the
// kept indices are sorted so the time order survives).  Equal scores go to
// the lower index, -0.0 == +0.0, NaN ranks below -inf.
//
// Method: scores map to order-preserving 32-bit keys.  A most-significant-
// digit radix select (4 passes of 8 bits, per-wave LDS histograms) finds the
// b-th largest key T and how many keys equal to T are kept (the quota).  A
// final ordered scan keeps every key > T and the first `quota` keys == T,
// writing their indices by a block-wide ballot prefix sum.
#include "tri_internal.hpp"

namespace tri {

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN: below every number
  if (u == 0x80000000u) u = 0u;                      // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__global__ __launch_bounds__(kSelThreads) void select_global_kernel(
    const SeqInfo* __restrict__ seqs, int LH, const float* __restrict__ scores,
    int32_t* __restrict__ kept) {
  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ uint32_t sel[2];
  __shared__ uint32_t wcnt_a[kSelWaves], wcnt_b[kSelWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int unit = blockIdx.x;
  const int s = unit / LH, lg = unit % LH;
  const SeqInfo si = seqs[s];
  const int n = si.n, b = si.b;
  if (b <= 0) return;
  const float* in = scores + si.row_base + (int64_t)lg * si.in_stride;
  int32_t* out = kept + si.out_base + (int64_t)lg * si.out_stride;
  if (b >= n) {
    for (int i = tid; i < n; i += kSelThreads) out[i] = i;
    return;
  }

  uint32_t prefix = 0u, mask = 0u;
  uint32_t kk = (uint32_t)b;  // rank of the target within the keys matching prefix
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
      const uint32_t key = order_key(in[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t c[4];
      uint32_t lane_tot = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t v = 0;
        for (int w = 0; w < kSelWaves; ++w) v += hist[w][4 * lane + u];
        c[u] = v;
        lane_tot += v;
      }
      // inclusive suffix sum over lanes (bins above belong to higher lanes)
      uint32_t suf = lane_tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += y;
      }
      uint32_t above = suf - lane_tot;
#pragma unroll
      for (int u = 3; u >= 0; --u) {
        if (above < kk && kk <= above + c[u]) {
          sel[0] = (uint32_t)(4 * lane + u);
          sel[1] = above;
        }
        above += c[u];
      }
    }
    __syncthreads();
    const uint32_t digit = sel[0];
    kk -= sel[1];
    prefix |= digit << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t T = prefix;
  const uint32_t quota = kk;  // keys equal to T that are kept (>= 1)

  uint32_t base_out = 0, base_eq = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int tile = 0; tile < n && base_out < (uint32_t)b; tile += kSelThreads) {
    const int i = tile + tid;
    const uint32_t key = i < n ? order_key(in[i]) : 0u;
    const bool gt = i < n && key > T;
    const bool eq = i < n && key == T;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) wcnt_a[wave] = (uint32_t)__popcll(beq);
    __syncthreads();
    uint32_t eq_before = base_eq + (uint32_t)__popcll(beq & lt_mask);
    uint32_t eq_tile = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      const uint32_t v = wcnt_a[w];
      if (w < wave) eq_before += v;
      eq_tile += v;
    }
    const bool keep = gt || (eq && eq_before < quota);
    const uint64_t bk = __ballot(keep);
    if (lane == 0) wcnt_b[wave] = (uint32_t)__popcll(bk);
    __syncthreads();
    uint32_t pos = base_out + (uint32_t)__popcll(bk & lt_mask);
    uint32_t keep_tile = 0;
    for (int w = 0; w < kSelWaves; ++w) {
      const uint32_t v = wcnt_b[w];
      if (w < wave) pos += v;
      keep_tile += v;
    }
    if (keep && pos < (uint32_t)b) out[pos] = i;
    base_out += keep_tile;
    base_eq += eq_tile;
    __syncthreads();
  }
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
                         int32_t* kept_idx, hipStream_t st) {
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
  hipLaunchKernelGGL(select_global_kernel, dim3((unsigned)units), dim3(kSelThreads), 0, st, seqs,
                     LH, scores, kept_idx);
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
