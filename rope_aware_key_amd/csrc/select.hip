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

__global__ __launch_bounds__(kSelThreads) void select_kernel(
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
  const float* in = scores + si.row_base + (int64_t)lg * n;
  int32_t* out = kept + si.out_base + (int64_t)lg * b;
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

hipError_t launch_select(const SeqInfo* seqs, int S, int LH, const float* scores,
                         int32_t* kept_idx, hipStream_t st) {
  const int64_t units = (int64_t)S * LH;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)units), dim3(kSelThreads), 0, st, seqs, LH,
                     scores, kept_idx);
  return hipGetLastError();
}

// Gather kept rows.  One group of d/8 lanes copies one 16-byte slice each of
// a K row and a V row; the first lane of the group copies the position.
__global__ __launch_bounds__(256) void compact_kernel(
    const SeqInfo* __restrict__ seqs, int S, int LH, int d, int64_t total_out,
    const int32_t* __restrict__ kept, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ k_pos,
    uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out, int32_t* __restrict__ pos_out) {
  const int lpr = d >> 3;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = gid / lpr;
  const int part = (int)(gid - r * lpr);
  if (r >= total_out) return;
  const int s = find_seq_by_out_row(seqs, S, r);
  const SeqInfo si = seqs[s];
  const int64_t local = r - si.out_base;
  const int64_t lg = local / si.b;
  const int32_t idx = kept[r];
  if ((uint32_t)idx >= (uint32_t)si.n) return;  // never read outside the unit
  const int64_t src = si.row_base + lg * si.n + idx;
  if (k_out)
    reinterpret_cast<uint4*>(k_out + r * d)[part] = reinterpret_cast<const uint4*>(k + src * d)[part];
  if (v_out)
    reinterpret_cast<uint4*>(v_out + r * d)[part] = reinterpret_cast<const uint4*>(v + src * d)[part];
  if (pos_out && part == 0) pos_out[r] = k_pos[src];
}

hipError_t launch_compact(const SeqInfo* seqs, int S, int LH, int d, int64_t total_out,
                          const int32_t* kept_idx, const uint16_t* k, const uint16_t* v,
                          const int32_t* k_pos, uint16_t* k_out, uint16_t* v_out,
                          int32_t* pos_out, hipStream_t st) {
  (void)LH;
  if (total_out == 0) return hipSuccess;
  const int64_t threads = total_out * (d >> 3);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(256), 0, st, seqs, S, LH, d,
                     total_out, kept_idx, k, v, k_pos, k_out, v_out, pos_out);
  return hipGetLastError();
}

}  // namespace tri
