// Per-key TriAttention score: raw offset-averaged scores per query head,
// per-head z-score over the unit, max over the GQA group.
//
// Math (talk page "聊聊 TriAttention", S_trig / S_norm / averaged-score
// equations; hyper.ai summary, section "方法" for the z-score and the max):
// with the per-(sequence, head, band) coefficient A_f = E[q_f] C_f
// exp(i omega_f p_q) prepared by the prologue,
//   S~_h(i) = sum_f [ Re(A_f) x_f + Im(A_f) y_f ] + sum_f w_f sqrt(x_f^2 + y_f^2)
// where (x_f, y_f) is band f of the stored post-RoPE key, (k[2f], k[2f+1])
// or, half split, (k[f], k[f + d/2]), and w_f = (1 - R_f) E|q_f|.  One read
// of a key serves all G query heads.
//
// Work split: a "ticket" is one chunk of kScoreChunk keys of one unit.
// Tickets of a unit are consecutive; each records (count, mean, M2) per head
// in fp64, and the z pass merges them in ticket order (Chan's update), so
// the result is deterministic.
#include "tri_internal.hpp"

namespace tri {

__device__ __forceinline__ float bf16_lo_s(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_s(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over the 256 threads of a block; every thread gets the total.
__device__ __forceinline__ double block_sum256(double v, double* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const double t = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return t;
}

struct Ticket {
  int s, lg, c, nch, nkeys, key0;
  int64_t row0;
};

__device__ __forceinline__ Ticket decode_ticket(const SeqInfo* seqs, int S, int t) {
  Ticket k;
  k.s = find_seq_by_ticket(seqs, S, t);
  const SeqInfo si = seqs[k.s];
  k.nch = (si.n + kScoreChunk - 1) / kScoreChunk;
  const int local = t - si.chunk_base;
  k.lg = local / k.nch;
  k.c = local % k.nch;
  k.key0 = k.c * kScoreChunk;
  k.nkeys = min(kScoreChunk, si.n - k.key0);
  k.row0 = si.row_base + (int64_t)k.lg * si.in_stride;
  return k;
}

template <int GT>
__global__ __launch_bounds__(256) void score_raw_kernel(
    const SeqInfo* __restrict__ seqs, int S, int Hkv, int Hq, int G, int d, bool half,
    const Pages pg, const double2* __restrict__ P, const float* __restrict__ W, const double2* __restrict__ E,
    const uint16_t* __restrict__ k, float* __restrict__ raw, double* __restrict__ chunk_stats) {
  constexpr int KPT = kScoreChunk / 256;
  __shared__ float a_s[GT * kMaxHeadDim];
  __shared__ float w_s[GT * (kMaxHeadDim / 2)];
  __shared__ double red[4];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const Ticket tk = decode_ticket(seqs, S, t);
  const int l = tk.lg / Hkv, g = tk.lg % Hkv;
  const int F = d >> 1;

  for (int idx = tid; idx < GT * F; idx += 256) {
    const int h = idx / F, f = idx % F;
    float ar = 0.f, ai = 0.f, wv = 0.f;
    if (h < G) {
      const int64_t o = ((int64_t)l * Hq + g * G + h) * F + f;
      const double2 pv = P[o];
      const double2 ev = E[(int64_t)tk.s * F + f];
      ar = (float)(pv.x * ev.x - pv.y * ev.y);
      ai = (float)(pv.x * ev.y + pv.y * ev.x);
      wv = W[o];
    }
    a_s[h * d + 2 * f] = ar;
    a_s[h * d + 2 * f + 1] = ai;
    w_s[h * F + f] = wv;
  }
  __syncthreads();

  float vals[KPT][GT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int key = tid + j * 256;
    float acc[GT];
#pragma unroll
    for (int h = 0; h < GT; ++h) acc[h] = 0.f;
    auto band = [&](int f, float x, float y) {
      const float r = __builtin_amdgcn_sqrtf(fmaf(x, x, y * y));
#pragma unroll
      for (int h = 0; h < GT; ++h) {
        float a = acc[h];
        a = fmaf(a_s[h * d + 2 * f], x, a);
        a = fmaf(a_s[h * d + 2 * f + 1], y, a);
        a = fmaf(w_s[h * F + f], r, a);
        acc[h] = a;
      }
    };
    // the key's row: packed, or through the page table
    const int64_t krow = key >= tk.nkeys ? 0
                         : pg.table  ? paged_row(pg, tk.s, l, g, tk.key0 + key)
                                     : tk.row0 + tk.key0 + key;
    if (key < tk.nkeys && !half) {
      const uint4* rp = reinterpret_cast<const uint4*>(k + krow * d);
      for (int c8 = 0; c8 < (d >> 3); ++c8) {
        const uint4 q = rp[c8];
        const uint32_t wd[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) band(c8 * 4 + u, bf16_lo_s(wd[u]), bf16_hi_s(wd[u]));
      }
    } else if (key < tk.nkeys) {
      // half split: four bands per step, real parts from the first half of
      // the row, imaginary parts from the second (8-byte loads: d/2 is a
      // multiple of 4, not always of 8)
      const uint2* rp = reinterpret_cast<const uint2*>(k + krow * d);
      for (int c4 = 0; c4 < (F >> 2); ++c4) {
        const uint2 re = rp[c4], im = rp[(F >> 2) + c4];
        band(4 * c4 + 0, bf16_lo_s(re.x), bf16_lo_s(im.x));
        band(4 * c4 + 1, bf16_hi_s(re.x), bf16_hi_s(im.x));
        band(4 * c4 + 2, bf16_lo_s(re.y), bf16_lo_s(im.y));
        band(4 * c4 + 3, bf16_hi_s(re.y), bf16_hi_s(im.y));
      }
    }
#pragma unroll
    for (int h = 0; h < GT; ++h) vals[j][h] = acc[h];
  }

  // Chunk statistics per head: count, mean, sum of squared deviations.
#pragma unroll
  for (int h = 0; h < GT; ++h) {
    if (h >= G) break;
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (tid + j * 256 < tk.nkeys) sum += (double)vals[j][h];
    sum = block_sum256(sum, red);
    const double mean = sum / (double)tk.nkeys;
    double m2 = 0.0;
#pragma unroll
    for (int j = 0; j < KPT; ++j)
      if (tid + j * 256 < tk.nkeys) {
        const double dv = (double)vals[j][h] - mean;
        m2 += dv * dv;
      }
    m2 = block_sum256(m2, red);
    if (tid == 0) {
      double* cs = chunk_stats + ((int64_t)t * kMaxGroup + h) * 3;
      cs[0] = (double)tk.nkeys;
      cs[1] = mean;
      cs[2] = m2;
    }
  }

#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int key = tid + j * 256;
    if (key < tk.nkeys) {
      float* rp = raw + (tk.row0 + tk.key0 + key) * G;
#pragma unroll
      for (int h = 0; h < GT; ++h)
        if (h < G) rp[h] = vals[j][h];
    }
  }
}

// Per-(unit, head) statistics: the unit's tickets merged in ticket order
// (Chan's update), once per unit.  unit_stats[unit][h] = (mu, 1/sigma), with
// 1/sigma = 0 where sigma = 0; head_stats (optional) gets (mu, sigma).
__global__ __launch_bounds__(256) void unit_stats_kernel(
    const SeqInfo* __restrict__ seqs, int S, int LH, int G, const double* __restrict__ chunk_stats,
    double* __restrict__ unit_stats, double* __restrict__ head_stats) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)S * LH * G) return;
  const int64_t unit = idx / G;
  const int h = (int)(idx % G);
  const SeqInfo si = seqs[unit / LH];
  if (si.n == 0) return;
  const int lg = (int)(unit % LH);
  const int nch = (si.n + kScoreChunk - 1) / kScoreChunk;
  const int t0 = si.chunk_base + lg * nch;
  double cnt = 0.0, mean = 0.0, m2 = 0.0;
#pragma unroll 4
  for (int cc = 0; cc < nch; ++cc) {
    const double* cs = chunk_stats + ((int64_t)(t0 + cc) * kMaxGroup + h) * 3;
    const double nb = cs[0], mb = cs[1], m2b = cs[2];
    if (cc == 0) {
      cnt = nb; mean = mb; m2 = m2b;
    } else {
      const double tot = cnt + nb;
      const double dl = mb - mean;
      mean += dl * (nb / tot);
      m2 += m2b + dl * dl * (cnt * nb / tot);
      cnt = tot;
    }
  }
  const double sigma = sqrt(m2 / cnt);
  unit_stats[(unit * G + h) * 2] = mean;
  unit_stats[(unit * G + h) * 2 + 1] = sigma > 0.0 ? 1.0 / sigma : 0.0;
  if (head_stats) {
    head_stats[(unit * G + h) * 2] = mean;
    head_stats[(unit * G + h) * 2 + 1] = sigma;
  }
}

// scores = max_h (raw_h - mu_h) / sigma_h, one ticket per work-group.  The
// ticket's raw block (nkeys * G contiguous floats) is copied to LDS with
// coalesced loads, into rows of odd stride GT|1 (conflict-free row reads).
template <int GT>
__global__ __launch_bounds__(256) void zmax_kernel(
    const SeqInfo* __restrict__ seqs, int S, int LH, int G, const float* __restrict__ raw,
    const double* __restrict__ unit_stats, float* __restrict__ scores) {
  constexpr int GP = GT | 1;
  __shared__ float blk[kScoreChunk * GP];
  __shared__ double mu_s[GT], inv_s[GT];
  const int tid = threadIdx.x;
  const Ticket tk = decode_ticket(seqs, S, blockIdx.x);
  const int64_t unit = (int64_t)tk.s * LH + tk.lg;
  if (tid < GT) {
    mu_s[tid] = tid < G ? unit_stats[(unit * G + tid) * 2] : 0.0;
    inv_s[tid] = tid < G ? unit_stats[(unit * G + tid) * 2 + 1] : 0.0;
  }
  const float* base = raw + (tk.row0 + tk.key0) * G;
  const int total = tk.nkeys * G;
  const float invG = 1.0f / (float)G;
  // element i of the block is head i % G of key i / G
  auto put = [&](int i, float x) {
    int key = (int)((float)i * invG);  // i < 2^14: off by at most one
    key += (key + 1) * G <= i;
    key -= key * G > i;
    blk[key * GP + (i - key * G)] = x;
  };
  constexpr int kUnroll = 4;
  int done = 0;
  if ((reinterpret_cast<uintptr_t>(base) & 15u) == 0) {
    // 16-byte loads: four times the bytes in flight per thread
    const int total4 = total >> 2;
    const float4* b4 = reinterpret_cast<const float4*>(base);
    for (int i0 = tid; i0 < total4; i0 += 256 * kUnroll) {
      float4 v[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int i = i0 + 256 * j;
        v[j] = i < total4 ? b4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int i = i0 + 256 * j;
        if (i < total4) {
          put(4 * i, v[j].x);
          put(4 * i + 1, v[j].y);
          put(4 * i + 2, v[j].z);
          put(4 * i + 3, v[j].w);
        }
      }
    }
    done = total4 * 4;
  }
  for (int i0 = done + tid; i0 < total; i0 += 256 * kUnroll) {
    float v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int i = i0 + 256 * j;
      v[j] = i < total ? base[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int i = i0 + 256 * j;
      if (i < total) put(i, v[j]);
    }
  }
  __syncthreads();
  for (int key = tid; key < tk.nkeys; key += 256) {
    double best = -__builtin_huge_val();
#pragma unroll
    for (int h = 0; h < GT; ++h)
      if (h < G) best = fmax(best, ((double)blk[key * GP + h] - mu_s[h]) * inv_s[h]);
    // non-temporal: written once here, read once by the select kernel
    __builtin_nontemporal_store((float)best, scores + tk.row0 + tk.key0 + key);
  }
}

template <int GT>
static void launch_raw(int grid, hipStream_t st, const SeqInfo* seqs, int S, int Hkv, int Hq,
                       int G, int d, bool half, const Pages& pg, const double2* P,
                       const float* W, const double2* E, const uint16_t* k, float* raw,
                       double* cs) {
  hipLaunchKernelGGL(score_raw_kernel<GT>, dim3(grid), dim3(256), 0, st, seqs, S, Hkv, Hq, G, d,
                     half, pg, P, W, E, k, raw, cs);
}

hipError_t launch_score(const SeqInfo* seqs, int S, int L, int Hkv, int G, int d,
                        int total_tickets, const double2* P, const float* W, const double2* E,
                        const uint16_t* k, float* raw, double* chunk_stats, double* unit_stats,
                        float* scores, double* head_stats, bool half, const Pages& pg,
                        hipStream_t st) {
  if (total_tickets == 0) return hipSuccess;
  const int Hq = Hkv * G;
  if (G <= 1)
    launch_raw<1>(total_tickets, st, seqs, S, Hkv, Hq, G, d, half, pg, P, W, E, k, raw,
                  chunk_stats);
  else if (G <= 2)
    launch_raw<2>(total_tickets, st, seqs, S, Hkv, Hq, G, d, half, pg, P, W, E, k, raw,
                  chunk_stats);
  else if (G <= 4)
    launch_raw<4>(total_tickets, st, seqs, S, Hkv, Hq, G, d, half, pg, P, W, E, k, raw,
                  chunk_stats);
  else if (G <= 8)
    launch_raw<8>(total_tickets, st, seqs, S, Hkv, Hq, G, d, half, pg, P, W, E, k, raw,
                  chunk_stats);
  else
    launch_raw<16>(total_tickets, st, seqs, S, Hkv, Hq, G, d, half, pg, P, W, E, k, raw,
                  chunk_stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_zmax(seqs, S, L, Hkv, G, total_tickets, raw, chunk_stats, unit_stats, scores,
                     head_stats, st);
}

hipError_t launch_zmax(const SeqInfo* seqs, int S, int L, int Hkv, int G, int total_tickets,
                       const float* raw, const double* chunk_stats, double* unit_stats,
                       float* scores, double* head_stats, hipStream_t st) {
  if (total_tickets == 0) return hipSuccess;
  const int LH = L * Hkv;
  const int64_t n_us = (int64_t)S * LH * G;
  hipLaunchKernelGGL(unit_stats_kernel, dim3((unsigned)((n_us + 255) / 256)), dim3(256), 0, st,
                     seqs, S, LH, G, chunk_stats, unit_stats, head_stats);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
#define TRI_Z(GT)                                                                              \
  hipLaunchKernelGGL(zmax_kernel<GT>, dim3(total_tickets), dim3(256), 0, st, seqs, S, LH, G, raw, \
                     unit_stats, scores)
  if (G <= 1)
    TRI_Z(1);
  else if (G <= 2)
    TRI_Z(2);
  else if (G <= 4)
    TRI_Z(4);
  else if (G <= 8)
    TRI_Z(8);
  else
    TRI_Z(16);
#undef TRI_Z
  return hipGetLastError();
}

}  // namespace tri
