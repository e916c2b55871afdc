// Raw scores with the offsets reduced by their maximum instead of their mean
// (the blog review's reading of the offset step, a maximum over D):
//   S~_h(i) = max_{delta in D} S_trig(k_i, Delta_i + delta) + S_norm(k_i)
//   S_trig(k, Delta + delta) = sum_f Re(E[q_f] exp(i omega_f (p_q + delta)) conj(k'_f))
// (talk page "聊聊 TriAttention", S_trig / S_norm equations; the key position
// cancels exactly as in the averaged score).  A maximum does not fold into
// one coefficient per band: every (query head, offset) pair is a row of its
// own, so per unit the trig term is a (G*|D| x d) by (d x n) product.
//
// Mapping onto CDNA4:
//  * Rows are (head h, offset slot j), row = h*Dp + j with Dp = |D| rounded
//    up to a multiple of 4; slots past |D| repeat the first offset (a repeat
//    leaves the maximum unchanged).  The 4 accumulator rows one lane holds
//    (4q..4q+3 of a 16-row tile) therefore always belong to one head.
//  * v_mfma_f32_16x16x32_bf16 with each fp64 coefficient split into three
//    bf16 terms (hi, mid, lo), the same fp32-accurate scheme as the averaged
//    path.  The split rows live in LDS and each A-operand read serves GB
//    blocks of 16 keys held in registers.
//  * When the rows of all G heads do not fit in LDS, the heads are taken in
//    passes of whole heads (each pass re-reads the keys); a head's maximum
//    is always complete within one pass.
//  * A lane reduces its 4 rows and merges the result into a per-(key, head)
//    maximum in LDS with an integer atomic max on an order-preserving map;
//    the norm term is a v_mfma_f32_16x16x4_f32 product with heads as rows.
//  * Raw scores are spilled in the generic path's layout with per-ticket
//    (count, mean, M2) per head; the generic z pass (zmax_kernel) then merges
//    the tickets of each unit and writes the z-score maxima.
//  * A work-group takes kTicketsPerGroup consecutive tickets and stages the
//    split rows again only when the unit (or pass) changes.
#include "tri_internal.hpp"

namespace tri {

typedef short bf16x8m_t __attribute__((ext_vector_type(8)));
typedef float f32x4m_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2m_t __attribute__((ext_vector_type(2)));

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kTicketsPerGroup = 8;

struct MaxLds {
  uint32_t smax[kWaves][64][kMaxGroup];
  double red_s[kWaves][kMaxGroup], red_q[kWaves][kMaxGroup];
};

__device__ __forceinline__ uint32_t bf16_rne_m(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void split3_m(double x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = bf16_rne_m((float)x);
  const double r1 = x - (double)__uint_as_float(hi << 16);
  mid = bf16_rne_m((float)r1);
  const double r2 = r1 - (double)__uint_as_float(mid << 16);
  lo = bf16_rne_m((float)r2);
}

// Order-preserving map of finite floats to uint32 (0 is below every image).
__device__ __forceinline__ uint32_t ord(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unord(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ float band_sq_m(uint32_t w) {
  bf16x2m_t pr;
  __builtin_memcpy(&pr, &w, 4);
  return __builtin_amdgcn_fdot2_f32_bf16(pr, pr, 0.0f, false);
}

struct MaxTicket {
  int s, lg, nkeys, key0;
  int64_t row0, unit;
};

__device__ __forceinline__ MaxTicket decode_max_ticket(const SeqInfo* seqs, int S, int LH, int t) {
  MaxTicket k;
  k.s = find_seq_by_ticket(seqs, S, t);
  const SeqInfo si = seqs[k.s];
  const int nch = (si.n + kScoreChunk - 1) / kScoreChunk;
  const int local = t - si.chunk_base;
  k.lg = local / nch;
  const int c = local % nch;
  k.key0 = c * kScoreChunk;
  k.nkeys = min(kScoreChunk, si.n - k.key0);
  k.row0 = si.row_base + (int64_t)k.lg * si.n;
  k.unit = (int64_t)k.s * LH + k.lg;
  return k;
}

__device__ __forceinline__ uint4 pack8(const uint32_t (&v)[8]) {
  return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                    v[6] | (v[7] << 16));
}

}  // namespace

// Split coefficient rows: thread (unit, pass, tile, step, lane) forms, for
// row r = 16*tile + lane%16 of the pass (local head r / Dp, slot r % Dp),
// the fp64 coefficients of the lane's four bands of the step,
//   a_f = P[l][h][f] E[s][f] exp(i omega_f delta_slot),
// and stores their bf16 hi/mid/lo splits in MFMA A-operand lane order.
// The norm weights (heads as rows, one set per unit) go to wpack.
template <int STEPS>
__global__ __launch_bounds__(256) void pack_max_operands_kernel(
    int S, int L, int Hkv, int G, int Dp, int nD, int hp, int npass, int ptiles, double theta,
    const double2* __restrict__ P, const float* __restrict__ W, const double2* __restrict__ E,
    const double* __restrict__ offsets, uint4* __restrict__ apack, uint4* __restrict__ wpack) {
  constexpr int F = STEPS * 16;
  constexpr int D = STEPS * 32;
  const int64_t units = (int64_t)S * L * Hkv;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_a = units * npass * ptiles * STEPS * 64;
  const int64_t n_w = units * STEPS * 64;
  if (idx >= n_a + n_w) return;
  const int lane = (int)(idx & 63);
  const int m = lane & 15, q = lane >> 4;
  const int Hq = Hkv * G;
  if (idx < n_a) {
    int64_t r = idx >> 6;
    const int st = (int)(r % STEPS);
    r /= STEPS;
    const int tile = (int)(r % ptiles);
    r /= ptiles;
    const int pass = (int)(r % npass);
    const int64_t unit = r / npass;
    const int lg = (int)(unit % ((int64_t)L * Hkv));
    const int s = (int)(unit / ((int64_t)L * Hkv));
    const int l = lg / Hkv, g = lg % Hkv;
    const int row = tile * 16 + m;
    const int hl = row / Dp, slot = row % Dp;
    const int h = pass * hp + hl;
    const bool live = hl < hp && h < G;
    const double delta = offsets[slot < nD ? slot : 0];
    uint32_t h3[8], m3[8], l3[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int f = 4 * (4 * st + q) + u;
      double re = 0.0, im = 0.0;
      if (live) {
        const double2 pv = P[((int64_t)l * Hq + g * G + h) * F + f];
        const double2 ev = E[(int64_t)s * F + f];
        const double omega = pow(theta, -2.0 * (double)f / (double)D);
        double sn, cs;
        sincos(omega * delta, &sn, &cs);
        const double ar = pv.x * ev.x - pv.y * ev.y, ai = pv.x * ev.y + pv.y * ev.x;
        re = ar * cs - ai * sn;
        im = ar * sn + ai * cs;
      }
      split3_m(re, h3[2 * u], m3[2 * u], l3[2 * u]);
      split3_m(im, h3[2 * u + 1], m3[2 * u + 1], l3[2 * u + 1]);
    }
    uint4* op = apack + (idx >> 6) * 3 * 64 + lane;
    op[0] = pack8(h3);
    op[64] = pack8(m3);
    op[128] = pack8(l3);
  } else {
    const int64_t j = idx - n_a;
    const int st = (int)((j >> 6) % STEPS);
    const int64_t unit = (j >> 6) / STEPS;
    const int lg = (int)(unit % ((int64_t)L * Hkv));
    const int l = lg / Hkv, g = lg % Hkv;
    float wv[4] = {0.f, 0.f, 0.f, 0.f};
    if (m < G) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        wv[u] = W[((int64_t)l * Hq + g * G + m) * F + 4 * (4 * st + q) + u];
    }
    wpack[j] = make_uint4(__float_as_uint(wv[0]), __float_as_uint(wv[1]),
                          __float_as_uint(wv[2]), __float_as_uint(wv[3]));
  }
}

// kTicketsPerGroup consecutive tickets (kScoreChunk keys of one unit each)
// per work-group.  Dynamic LDS: the split rows of one (unit, pass),
// [ptiles][STEPS][3][64] uint4.
template <int STEPS, int GB>
__global__ __launch_bounds__(kThreads) void score_max_kernel(
    const SeqInfo* __restrict__ seqs, int S, int LH, int G, int Dp, int hp, int npass,
    int ptiles, int total_tickets, const uint4* __restrict__ apack,
    const uint4* __restrict__ wpack, const uint16_t* __restrict__ k, float* __restrict__ raw,
    double* __restrict__ chunk_stats) {
  constexpr int D = STEPS * 32;
  constexpr int KG = 16 * GB;  // keys per wave group
  extern __shared__ uint4 a_s[];
  __shared__ MaxLds sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, q = lane >> 4;
  const int rows_per_head = Dp >> 2;  // row groups of 4 per head
  const int n_a = ptiles * STEPS * 3 * 64;
  const int t_begin = blockIdx.x * kTicketsPerGroup;
  const int t_end = min(t_begin + kTicketsPerGroup, total_tickets);
  int64_t staged = -1;
  float wn[STEPS][4];

  for (int t = t_begin; t < t_end; ++t) {
    const MaxTicket tk = decode_max_ticket(seqs, S, LH, t);
    double s1[4] = {0.0, 0.0, 0.0, 0.0}, s2[4] = {0.0, 0.0, 0.0, 0.0};
    const uint16_t* kbase = k + (tk.row0 + tk.key0) * (int64_t)D;
    const int ngroups = (tk.nkeys + KG - 1) / KG;
    for (int pass = 0; pass < npass; ++pass) {
      const int64_t tag = tk.unit * npass + pass;
      if (tag != staged) {
        __syncthreads();  // every wave is done with the previous rows
        const uint4* src = apack + tag * (int64_t)n_a;
        for (int i = tid; i < n_a; i += kThreads) a_s[i] = src[i];
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
          const uint4 w = wpack[(tk.unit * STEPS + st) * 64 + lane];
          wn[st][0] = __uint_as_float(w.x);
          wn[st][1] = __uint_as_float(w.y);
          wn[st][2] = __uint_as_float(w.z);
          wn[st][3] = __uint_as_float(w.w);
        }
        __syncthreads();
        staged = tag;
      }
      const int h0 = pass * hp, h1 = min(G, h0 + hp);
      for (int grp = wave; grp < ngroups; grp += kWaves) {
        const int key_g = grp * KG;
        uint4 kb[GB][STEPS];
#pragma unroll
        for (int bb = 0; bb < GB; ++bb) {
          int key = key_g + bb * 16 + m;
          key = key < tk.nkeys ? key : tk.nkeys - 1;  // padding lanes re-read a valid row
          const uint4* rp = reinterpret_cast<const uint4*>(kbase + (int64_t)key * D);
#pragma unroll
          for (int st = 0; st < STEPS; ++st) kb[bb][st] = rp[4 * st + q];
        }
        // lane (m, q) owns keys m of each block, heads 4q..4q+3
#pragma unroll
        for (int bb = 0; bb < GB; ++bb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sh.smax[wave][bb * 16 + m][4 * q + i] = 0u;
        // Other lanes' atomics below touch these words: keep the three LDS
        // phases (reset, max, read) in program order; one wave's LDS
        // operations complete in issue order.
        __builtin_amdgcn_wave_barrier();
        // norm term, heads as rows: D[head][key] = sum_f w_f |k_f|
        f32x4m_t acc_n[GB];
#pragma unroll
        for (int bb = 0; bb < GB; ++bb) {
          acc_n[bb] = f32x4m_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < STEPS; ++st) {
            const uint32_t wd[4] = {kb[bb][st].x, kb[bb][st].y, kb[bb][st].z, kb[bb][st].w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const float r = __builtin_amdgcn_sqrtf(band_sq_m(wd[u]));
              acc_n[bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(wn[st][u], r, acc_n[bb], 0, 0, 0);
            }
          }
        }
        // trig term per (head, offset) row, reduced to a maximum per head
        for (int tile = 0; tile < ptiles; ++tile) {
          f32x4m_t acc[GB];
#pragma unroll
          for (int bb = 0; bb < GB; ++bb) acc[bb] = f32x4m_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < STEPS; ++st) {
            const uint4* ap = a_s + (tile * STEPS + st) * 3 * 64 + lane;
            const uint4 vh = ap[0], vm = ap[64], vl = ap[128];
            bf16x8m_t ah, am, al;
            __builtin_memcpy(&ah, &vh, 16);
            __builtin_memcpy(&am, &vm, 16);
            __builtin_memcpy(&al, &vl, 16);
#pragma unroll
            for (int bb = 0; bb < GB; ++bb) {
              bf16x8m_t bk;
              __builtin_memcpy(&bk, &kb[bb][st], 16);
              acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bk, acc[bb], 0, 0, 0);
              acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, bk, acc[bb], 0, 0, 0);
              acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bk, acc[bb], 0, 0, 0);
            }
          }
          // accumulator rows 4q..4q+3 of the tile: row group 4*tile + q
          const int hl = (4 * tile + q) / rows_per_head;
          const int h = h0 + hl;
          if (hl < hp && h < h1) {
#pragma unroll
            for (int bb = 0; bb < GB; ++bb) {
              const float v =
                  fmaxf(fmaxf(acc[bb][0], acc[bb][1]), fmaxf(acc[bb][2], acc[bb][3]));
              __hip_atomic_fetch_max(&sh.smax[wave][bb * 16 + m][h], ord(v), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_WORKGROUP);
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
        // raw = max over offsets + norm, for the heads of this pass
#pragma unroll
        for (int bb = 0; bb < GB; ++bb) {
          const int key = key_g + bb * 16 + m;
          if (key < tk.nkeys) {
            float* rp = raw + (tk.row0 + tk.key0 + key) * G;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int h = 4 * q + i;
              if (h >= h0 && h < h1) {
                const float v = unord(__hip_atomic_load(&sh.smax[wave][bb * 16 + m][h],
                                                        __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_WORKGROUP)) +
                                acc_n[bb][i];
                rp[h] = v;
                const double dv = (double)v;
                s1[i] += dv;
                s2[i] = fma(dv, dv, s2[i]);
              }
            }
          }
        }
      }
    }
    // per-ticket statistics per head: count, mean, M2 (from fp64 sums)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        s1[i] += __shfl_xor(s1[i], o, 64);
        s2[i] += __shfl_xor(s2[i], o, 64);
      }
    }
    if (m == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sh.red_s[wave][4 * q + i] = s1[i];
        sh.red_q[wave][4 * q + i] = s2[i];
      }
    }
    __syncthreads();
    if (tid < G) {
      double a = 0.0, b2 = 0.0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        a += sh.red_s[w][tid];
        b2 += sh.red_q[w][tid];
      }
      const double cnt = (double)tk.nkeys;
      const double mean = a / cnt;
      double* cs = chunk_stats + ((int64_t)t * kMaxGroup + tid) * 3;
      cs[0] = cnt;
      cs[1] = mean;
      cs[2] = fmax(b2 - cnt * mean * mean, 0.0);
    }
    __syncthreads();  // red_s / red_q are rewritten by the next ticket
  }
}

MaxOffsetsPlan plan_max_offsets(int d, int G, int n_offsets) {
  MaxOffsetsPlan mp;
  if (d % 32 != 0 || d < 32 || d > kMaxHeadDim || G < 1 || G > kMaxGroup || n_offsets < 1 ||
      n_offsets > kMaxOffsets)
    return mp;
  const int steps = d / 32;
  mp.Dp = (n_offsets + 3) / 4 * 4;
  const size_t tile_bytes = (size_t)steps * 3 * 64 * sizeof(uint4);
  const int max_tiles = (int)(kMaxOffsetsLds / tile_bytes);
  // most heads whose rows fit in LDS, then balanced over the passes
  int hp = 0;
  while (hp < G && ((hp + 1) * mp.Dp + 15) / 16 <= max_tiles) ++hp;
  if (hp == 0) return mp;
  mp.npass = (G + hp - 1) / hp;
  mp.hp = (G + mp.npass - 1) / mp.npass;
  mp.ptiles = (mp.hp * mp.Dp + 15) / 16;
  mp.ok = true;
  return mp;
}

size_t max_offsets_operand_bytes(int d, const MaxOffsetsPlan& mp, int64_t units) {
  if (!mp.ok) return 0;
  const int steps = d / 32;
  return (size_t)units *
         ((size_t)mp.npass * mp.ptiles * steps * 3 * 64 + (size_t)steps * 64) * sizeof(uint4);
}

template <int STEPS>
static hipError_t launch_max_t(const SeqInfo* seqs, int S, int L, int Hkv, int G, int nD,
                               const MaxOffsetsPlan& mp, double theta, int total_tickets,
                               const double2* P, const float* W, const double2* E,
                               const double* offsets, void* operands, const uint16_t* k,
                               float* raw, double* chunk_stats, hipStream_t st) {
  const int64_t units = (int64_t)S * L * Hkv;
  uint4* apack = reinterpret_cast<uint4*>(operands);
  uint4* wpack = apack + units * mp.npass * mp.ptiles * STEPS * 3 * 64;
  const int64_t threads = units * mp.npass * mp.ptiles * STEPS * 64 + units * STEPS * 64;
  hipLaunchKernelGGL(pack_max_operands_kernel<STEPS>, dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, st, S, L, Hkv, G, mp.Dp, nD, mp.hp, mp.npass, mp.ptiles,
                     theta, P, W, E, offsets, apack, wpack);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)mp.ptiles * STEPS * 3 * 64 * sizeof(uint4);
  const int grid = (total_tickets + kTicketsPerGroup - 1) / kTicketsPerGroup;
  if constexpr (STEPS <= 4)
    hipLaunchKernelGGL((score_max_kernel<STEPS, 4>), dim3(grid), dim3(kThreads), lds, st, seqs,
                       S, L * Hkv, G, mp.Dp, mp.hp, mp.npass, mp.ptiles, total_tickets, apack,
                       wpack, k, raw, chunk_stats);
  else
    hipLaunchKernelGGL((score_max_kernel<STEPS, 2>), dim3(grid), dim3(kThreads), lds, st, seqs,
                       S, L * Hkv, G, mp.Dp, mp.hp, mp.npass, mp.ptiles, total_tickets, apack,
                       wpack, k, raw, chunk_stats);
  return hipGetLastError();
}

hipError_t launch_score_max(const SeqInfo* seqs, int S, int L, int Hkv, int G, int d, int nD,
                            const MaxOffsetsPlan& mp, double theta, int total_tickets,
                            const double2* P, const float* W, const double2* E,
                            const double* offsets, void* operands, const uint16_t* k,
                            float* raw, double* chunk_stats, float* scores, double* head_stats,
                            hipStream_t st) {
  if (total_tickets == 0) return hipSuccess;
  if (!mp.ok) return hipErrorInvalidValue;
  hipError_t e = hipErrorInvalidValue;
  switch (d / 32) {
#define TRI_CASE(n)                                                                         \
  case n:                                                                                   \
    e = launch_max_t<n>(seqs, S, L, Hkv, G, nD, mp, theta, total_tickets, P, W, E, offsets, \
                        operands, k, raw, chunk_stats, st);                                 \
    break;
    TRI_CASE(1) TRI_CASE(2) TRI_CASE(3) TRI_CASE(4) TRI_CASE(5) TRI_CASE(6) TRI_CASE(7)
    TRI_CASE(8)
#undef TRI_CASE
    default:
      return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_zmax(seqs, S, L, Hkv, G, total_tickets, raw, chunk_stats, scores, head_stats, st);
}

}  // namespace tri
