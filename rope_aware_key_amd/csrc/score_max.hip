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
//  * v_mfma_f32_16x16x32_bf16 with each fp64 coefficient split into two
//    bf16 terms (hi, mid; kTrigTerms says why two suffice here, where the
//    averaged path keeps three).  The split rows of one unit live in LDS;
//    each A-operand read serves GB blocks of 16 keys held in registers.
//  * Lane (m, q) of an MFMA holds accumulator rows 4q..4q+3 of key m, so the
//    rows are dealt to the four lane slots q.  Normally head h of a pass
//    owns slot h % 4: its Dp rows (|D| rounded up to 4) fill Dp/4
//    consecutive tiles of that slot, every lane takes the running maximum of
//    its own rows in registers and ends holding heads q, q+4, q+8, q+12 of
//    its key.  When one head's rows exceed the LDS budget the head is spread
//    over all four slots and two cross-lane maxima merge them.  No LDS
//    traffic is spent on the reduction.
//  * When the rows of all G heads do not fit in LDS, the heads are taken in
//    passes (each pass re-reads the keys); a head's maximum is always
//    complete within one pass.
//  * The norm term runs on the same bf16 MFMA with heads as rows (weights
//    and band magnitudes split exactly into three bf16 terms each), the rows
//    permuted so that lane q's accumulator entry i is head 4i + q of the
//    pass, the same heads the lane holds maxima for.
//  * Raw scores are spilled in the generic path's layout.  Each wave writes
//    its sums (S1, S2) per (ticket, head); a merge kernel turns them into
//    per-ticket (count, mean, M2) in wave order and the generic z pass
//    (zmax_kernel) merges the tickets of each unit and writes the z-score
//    maxima.
//  * A work-group takes kTicketsPerGroup consecutive tickets and stages the
//    split rows again only when the unit (or pass) changes; otherwise its
//    waves run independently, each loading the keys of its next group while
//    it computes the current one.
#include <algorithm>

#include "tri_internal.hpp"

namespace tri {

typedef short bf16x8m_t __attribute__((ext_vector_type(8)));
typedef float f32x4m_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2m_t __attribute__((ext_vector_type(2)));
typedef float f32x2m_t __attribute__((ext_vector_type(2)));

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kTicketsPerGroup = 8;
// bf16 terms of each trig coefficient (hi + mid, ~17 significant bits).  The
// split error of a coefficient is at most 2^-17 of it, so a raw score moves
// by at most 2^-17 of sum_j |a_j k_j|, a few 2^-17 of the raw scores' own
// spread: on the five workload shapes the z-scores move by at most 2e-5
// (fp64 check of 2 against 3 terms), a fifth of the 1e-4 bar; the third
// term would add a third more MFMAs for 3e-8.
constexpr int kTrigTerms = 2;

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

// Two floats to a bf16 pair (round to nearest even), a in the low half.
__device__ __forceinline__ uint32_t cvt_pair(float a, float b) {
  const bf16x2m_t v = __builtin_convertvector((f32x2m_t){a, b}, bf16x2m_t);
  uint32_t u;
  __builtin_memcpy(&u, &v, 4);
  return u;
}

// Exact three-term bf16 split of two floats: x = t1 + t2 + t3 for each,
// returned as bf16 pairs (x_a in the low half).
__device__ __forceinline__ void split3_pair(float a, float b, uint32_t& t1, uint32_t& t2,
                                            uint32_t& t3) {
  t1 = cvt_pair(a, b);
  a -= __uint_as_float(t1 << 16);
  b -= __uint_as_float(t1 & 0xffff0000u);
  t2 = cvt_pair(a, b);
  a -= __uint_as_float(t2 << 16);
  b -= __uint_as_float(t2 & 0xffff0000u);
  t3 = cvt_pair(a, b);
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
  k.row0 = si.row_base + (int64_t)k.lg * si.in_stride;
  k.unit = (int64_t)k.s * LH + k.lg;
  return k;
}

__device__ __forceinline__ uint4 pack8(const uint32_t (&v)[8]) {
  return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                    v[6] | (v[7] << 16));
}

}  // namespace

// Offset phasors exp(i omega_f delta_j) for every (offset, band), fp64: they
// depend on neither the unit nor the head, so the pack kernel reads them
// instead of evaluating a sincos per operand element.
__global__ __launch_bounds__(256) void max_phasor_kernel(int F, int d, int nD, double theta,
                                                         const double* __restrict__ offsets,
                                                         double2* __restrict__ ph) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= nD * F) return;
  const int j = idx / F, f = idx % F;
  const double omega = pow(theta, -2.0 * (double)f / (double)d);
  double sn, cs;
  sincos(omega * offsets[j], &sn, &cs);
  ph[idx] = make_double2(cs, sn);
}

// Split coefficient rows: thread (unit, pass, tile, step, lane) forms the
// fp64 coefficients of the row the lane feeds at tile position m = lane%16
// (slot m/4, entry m%4; head and offset from the slot layout above),
//   a_f = P[l][h][f] E[s][f] exp(i omega_f delta)  (the last factor from ph),
// for the lane's eight elements of the step (the real or imaginary part of
// each element's band, by the RoPE layout), and stores their bf16
// hi/mid/lo splits in MFMA A-operand lane order.  Rows past |D| repeat the first
// offset; rows of heads outside the pass are zero.
//
// The norm term sum_f w_f |k_f| runs on the same bf16 MFMA: with
// w = w1 + w2 + w3 and r = |k_f| = r1 + r2 + r3 split exactly into bf16
// terms, three products per 16 bands,
//   [w1 w1].[r1 r2] + [w2 w2].[r1 r2] + [w1 w3].[r3 r1],
// keep every term down to 2^-24 of w r.  Lane (m, q) of step st feeds
// the bands of its four norm slots, b_u = slot_band(st, q, u) (16 st + 4q
// + u when interleaved), as k = 8q + {r(b0) r(b1) r'(b0) r'(b1) r(b2)
// r(b3) r'(b2) r'(b3)}, the order in which bf16 pairs come out of the
// split.  wpack holds the three A operands per (unit, pass, step),
// row r = 4q' + i carrying the pass's local head 4i + q'.
template <int STEPS>
__global__ __launch_bounds__(256) void pack_max_operands_kernel(
    int S, int L, int Hkv, int G, bool half, MaxOffsetsPlan mp, int nD,
    const double2* __restrict__ P, const float* __restrict__ W, const double2* __restrict__ E,
    const double2* __restrict__ ph, uint4* __restrict__ apack, uint4* __restrict__ wpack) {
  constexpr int F = STEPS * 16;
  constexpr int D = STEPS * 32;
  const int64_t units = (int64_t)S * L * Hkv;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_a = units * mp.npass * mp.ptiles * STEPS * 64;
  const int64_t n_w = units * mp.npass * STEPS * 64;  // one thread: 3 operands
  if (idx >= n_a + n_w) return;
  const int lane = (int)(idx & 63);
  const int m = lane & 15, q = lane >> 4;
  const int Hq = Hkv * G;
  if (idx < n_a) {
    int64_t r = idx >> 6;
    const int st = (int)(r % STEPS);
    r /= STEPS;
    const int tile = (int)(r % mp.ptiles);
    r /= mp.ptiles;
    const int pass = (int)(r % mp.npass);
    const int64_t unit = r / mp.npass;
    const int lg = (int)(unit % ((int64_t)L * Hkv));
    const int s = (int)(unit / ((int64_t)L * Hkv));
    const int l = lg / Hkv, g = lg % Hkv;
    const int slot = m >> 2, entry = m & 3;
    const int k = tile / mp.tiles_per_head, tt = tile % mp.tiles_per_head;
    int hl, j;
    if (mp.spread == 1) {
      hl = 4 * k + slot;
      j = 4 * tt + entry;
    } else {
      hl = k;
      j = 16 * tt + 4 * slot + entry;
    }
    const int h = pass * mp.hp + hl;
    const bool live = hl < mp.hp && h < G;
    const double2* phj = ph + (int64_t)(j < nD ? j : 0) * F;
    // element j of the lane's eight: the real or imaginary part (by the
    // RoPE layout) of its band's coefficient
    uint32_t h3[8], m3[8], l3[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = 32 * st + 8 * q + j;
      const int f = elem_band(e, D, half);
      double x = 0.0;
      if (live) {
        const double2 pv = P[((int64_t)l * Hq + g * G + h) * F + f];
        const double2 ev = E[(int64_t)s * F + f];
        const double2 pd = phj[f];
        const double cs = pd.x, sn = pd.y;
        const double ar = pv.x * ev.x - pv.y * ev.y, ai = pv.x * ev.y + pv.y * ev.x;
        x = elem_part(e, D, half) ? ar * sn + ai * cs : ar * cs - ai * sn;
      }
      split3_m(x, h3[j], m3[j], l3[j]);
    }
    uint4* op = apack + (idx >> 6) * kTrigTerms * 64 + lane;
    op[0] = pack8(h3);
    op[64] = pack8(m3);
    if (kTrigTerms > 2) op[128] = pack8(l3);
  } else {
    const int64_t j = idx - n_a;
    const int st = (int)((j >> 6) % STEPS);
    const int64_t r = (j >> 6) / STEPS;
    const int pass = (int)(r % mp.npass);
    const int64_t unit = r / mp.npass;
    const int lg = (int)(unit % ((int64_t)L * Hkv));
    const int l = lg / Hkv, g = lg % Hkv;
    // row m = 4q' + i carries local head 4i + q' of the pass
    const int hl = 4 * (m & 3) + (m >> 2);
    const int h = pass * mp.hp + hl;
    float wv[4] = {0.f, 0.f, 0.f, 0.f};
    if (hl < mp.hp && h < G) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        wv[u] = W[((int64_t)l * Hq + g * G + h) * F + slot_band(st, q, u, STEPS, half)];
    }
    uint32_t a1, a2, a3, c1, c2, c3;  // splits of (w_b0, w_b1) and (w_b2, w_b3)
    split3_pair(wv[0], wv[1], a1, a2, a3);
    split3_pair(wv[2], wv[3], c1, c2, c3);
    uint4* op = wpack + (j >> 6) * 3 * 64 + lane;
    op[0] = make_uint4(a1, a1, c1, c1);    // [w1 w1] against [r1 r2]
    op[64] = make_uint4(a2, a2, c2, c2);   // [w2 w2] against [r1 r2]
    op[128] = make_uint4(a1, a3, c1, c3);  // [w1 w3] against [r3 r1]
  }
}

// One work item of a wave: group grp (KG keys) of ticket t in pass `pass`.
// A wave takes the groups grp = wave, wave + kWaves, ... of every ticket of
// its work-group, pass by pass.
struct MaxItem {
  int pass, t, grp;
  bool valid;
};

// First item of the wave at or after (pass, t), or an invalid item.
__device__ __forceinline__ MaxItem first_item(const SeqInfo* seqs, int S, int npass, int t_begin,
                                              int t_end, int pass, int t, int wave, int KG) {
  for (; pass < npass; ++pass, t = t_begin) {
    for (; t < t_end; ++t) {
      const SeqInfo si = seqs[find_seq_by_ticket(seqs, S, t)];
      const int nch = (si.n + kScoreChunk - 1) / kScoreChunk;
      const int c = (t - si.chunk_base) % nch;
      const int nkeys = min(kScoreChunk, si.n - c * kScoreChunk);
      if (wave * KG < nkeys) return MaxItem{pass, t, wave, true};
    }
  }
  return MaxItem{0, 0, 0, false};
}

// Key rows of one item into registers: block bb, key 16*bb + m of the
// group, dims 32*st + 8q .. +7 (the MFMA B-operand layout).  Rows past the
// ticket's keys re-read its last row.  Paged pools: each row through the
// page table.
template <int STEPS, int GB>
__device__ __forceinline__ void load_item_keys(const SeqInfo* seqs, int S, int LH,
                                               const uint16_t* __restrict__ k, const Pages& pg,
                                               const MaxItem& it, int m, int q,
                                               uint4 (&kb)[GB][STEPS]) {
  constexpr int D = STEPS * 32;
  const MaxTicket tk = decode_max_ticket(seqs, S, LH, it.t);
#pragma unroll
  for (int bb = 0; bb < GB; ++bb) {
    int key = it.grp * 16 * GB + bb * 16 + m;
    key = key < tk.nkeys ? key : tk.nkeys - 1;
    const int64_t row = pg.table ? paged_row_lg(pg, tk.s, tk.lg, tk.key0 + key)
                                 : tk.row0 + tk.key0 + key;
    const uint4* rp = reinterpret_cast<const uint4*>(k + row * D);
#pragma unroll
    for (int st = 0; st < STEPS; ++st) kb[bb][st] = rp[4 * st + q];
  }
}

// kTicketsPerGroup consecutive tickets (kScoreChunk keys of one unit each)
// per work-group.  Dynamic LDS: the norm operands of one (unit, pass),
// [STEPS][3][64] uint4, then its split rows, [ptiles][STEPS][3][64] uint4.
// Each wave keeps the keys of its next item loading while it computes the
// current one.  NE = ceil(hp/4) head entries per lane; every lane issues
// the same GB*NE raw stores per group (rows past the ticket or heads past
// the pass go to `sink`), so the load/store counter waits for the
// prefetched keys stay exact.
template <int STEPS, int GB, int NE, bool HALF>
__global__ __launch_bounds__(kThreads) void score_max_kernel(
    const SeqInfo* __restrict__ seqs, int S, int LH, int G, MaxOffsetsPlan mp, int total_tickets,
    const uint4* __restrict__ apack, const uint4* __restrict__ wpack,
    const uint16_t* __restrict__ k, const Pages pg, float* __restrict__ raw,
    double* __restrict__ wsum,
    float* __restrict__ sink) {
  constexpr int KG = 16 * GB;  // keys per wave group
  extern __shared__ uint4 lds[];
  uint4* w_s = lds;
  uint4* a_s = lds + STEPS * 3 * 64;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave index as a scalar: the work list and ticket lookups stay uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, q = lane >> 4;
  const int n_a = mp.ptiles * STEPS * kTrigTerms * 64;
  const int t_begin = blockIdx.x * kTicketsPerGroup;
  const int t_end = min(t_begin + kTicketsPerGroup, total_tickets);
  const bool spread = mp.spread != 1;
  int64_t staged = -1;

  MaxItem cur = first_item(seqs, S, mp.npass, t_begin, t_end, 0, t_begin, wave, KG);
  uint4 kb[GB][STEPS];
  if (cur.valid) load_item_keys<STEPS, GB>(seqs, S, LH, k, pg, cur, m, q, kb);

  // Waves run through the tickets independently; the block meets only
  // where the staged rows change (a new unit or pass).
  for (int pass = 0; pass < mp.npass; ++pass) {
    const int h0 = pass * mp.hp, h1 = min(G, h0 + mp.hp);
    for (int t = t_begin; t < t_end; ++t) {
      const MaxTicket tk = decode_max_ticket(seqs, S, LH, t);
      double s1[NE], s2[NE];
#pragma unroll
      for (int i = 0; i < NE; ++i) s1[i] = s2[i] = 0.0;
      const int ngroups = (tk.nkeys + KG - 1) / KG;
      const int64_t tag = tk.unit * mp.npass + pass;
      if (tag != staged) {
        __syncthreads();  // every wave is done with the previous rows
        const uint4* src = apack + tag * (int64_t)n_a;
        for (int i = tid; i < n_a; i += kThreads) a_s[i] = src[i];
        for (int i = tid; i < STEPS * 3 * 64; i += kThreads)
          w_s[i] = wpack[tag * STEPS * 3 * 64 + i];
        __syncthreads();
        staged = tag;
      }
      for (int grp = wave; grp < ngroups; grp += kWaves) {
        // this item is `cur`, its keys are in kb; start loading the next
        // item's keys (the current item again when there is none)
        const MaxItem nx = grp + kWaves < ngroups
                               ? MaxItem{pass, t, grp + kWaves, true}
                               : first_item(seqs, S, mp.npass, t_begin, t_end, pass, t + 1, wave, KG);
        uint4 kn[GB][STEPS];
        load_item_keys<STEPS, GB>(seqs, S, LH, k, pg, nx.valid ? nx : cur, m, q, kn);
        const int key_g = grp * KG;
        // trig term: running maximum over each head's tiles
        float hm[GB][NE];
#pragma unroll
        for (int bb = 0; bb < GB; ++bb)
#pragma unroll
          for (int i = 0; i < NE; ++i) hm[bb][i] = 0.f;
        // A operands run one MFMA step ahead of their use (tiles in order
        // over all rounds); past the last tile the last step is re-read.
        const uint4* ap = a_s + lane;
        uint4 va[kTrigTerms];
#pragma unroll
        for (int tt = 0; tt < kTrigTerms; ++tt) va[tt] = ap[64 * tt];
        for (int kk = 0; kk < mp.nk; ++kk) {
          float run[GB];
#pragma unroll
          for (int bb = 0; bb < GB; ++bb) run[bb] = -__builtin_huge_valf();
          const int tile0 = kk * mp.tiles_per_head;
          for (int tile = tile0; tile < tile0 + mp.tiles_per_head; ++tile) {
            f32x4m_t acc[GB];
#pragma unroll
            for (int bb = 0; bb < GB; ++bb) acc[bb] = f32x4m_t{0.f, 0.f, 0.f, 0.f};
            const bool more = tile + 1 < mp.ptiles;
#pragma unroll
            for (int st = 0; st < STEPS; ++st) {
              const uint4* np = ap + ((st + 1 < STEPS || more) ? 64 * kTrigTerms : 0);
              uint4 vn[kTrigTerms];
#pragma unroll
              for (int tt = 0; tt < kTrigTerms; ++tt) vn[tt] = np[64 * tt];
              bf16x8m_t at[kTrigTerms];
#pragma unroll
              for (int tt = 0; tt < kTrigTerms; ++tt) __builtin_memcpy(&at[tt], &va[tt], 16);
#pragma unroll
              for (int bb = 0; bb < GB; ++bb) {
                bf16x8m_t bk;
                __builtin_memcpy(&bk, &kb[bb][st], 16);
#pragma unroll
                for (int tt = 0; tt < kTrigTerms; ++tt)
                  acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(at[tt], bk, acc[bb], 0, 0, 0);
              }
              __builtin_amdgcn_sched_group_barrier(0x100, kTrigTerms, 0);       // next operands
              __builtin_amdgcn_sched_group_barrier(0x008, kTrigTerms * GB, 0);  // this step
#pragma unroll
              for (int tt = 0; tt < kTrigTerms; ++tt) va[tt] = vn[tt];
              ap = np;
            }
#pragma unroll
            for (int bb = 0; bb < GB; ++bb)
              run[bb] = fmaxf(run[bb], fmaxf(fmaxf(acc[bb][0], acc[bb][1]),
                                             fmaxf(acc[bb][2], acc[bb][3])));
          }
          // head of this kk step: 4*kk + q (own slot), or kk spread over all
          // slots (merge the four, lane kk % 4 keeps it as entry kk / 4)
          int ent = kk;
          bool own = true;
          if (spread) {
#pragma unroll
            for (int bb = 0; bb < GB; ++bb) {
              run[bb] = fmaxf(run[bb], __shfl_xor(run[bb], 16, 64));
              run[bb] = fmaxf(run[bb], __shfl_xor(run[bb], 32, 64));
            }
            ent = kk >> 2;
            own = q == (kk & 3);
          }
#pragma unroll
          for (int i = 0; i < NE; ++i) {
            if (own && i == ent) {
#pragma unroll
              for (int bb = 0; bb < GB; ++bb) hm[bb][i] = run[bb];
            }
          }
        }
        // norm term, heads as (permuted) rows: entry i of lane q is local
        // head 4i + q of the pass
        f32x4m_t acc_n[GB];
#pragma unroll
        for (int bb = 0; bb < GB; ++bb) acc_n[bb] = f32x4m_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
          const uint4* wp = w_s + st * 3 * 64 + lane;
          const uint4 w1 = wp[0], w2 = wp[64], w3 = wp[128];
          bf16x8m_t aw1, aw2, aw3;
          __builtin_memcpy(&aw1, &w1, 16);
          __builtin_memcpy(&aw2, &w2, 16);
          __builtin_memcpy(&aw3, &w3, 16);
#pragma unroll
          for (int bb = 0; bb < GB; ++bb) {
            // magnitudes of the bands of the step's four norm slots
            uint32_t r1a, r2a, r3a, r1b, r2b, r3b;
            split3_pair(__builtin_amdgcn_sqrtf(band_sq_m(slot_pair<STEPS, HALF>(kb[bb], st, 0))),
                        __builtin_amdgcn_sqrtf(band_sq_m(slot_pair<STEPS, HALF>(kb[bb], st, 1))),
                        r1a, r2a, r3a);
            split3_pair(__builtin_amdgcn_sqrtf(band_sq_m(slot_pair<STEPS, HALF>(kb[bb], st, 2))),
                        __builtin_amdgcn_sqrtf(band_sq_m(slot_pair<STEPS, HALF>(kb[bb], st, 3))),
                        r1b, r2b, r3b);
            const uint4 b12 = make_uint4(r1a, r2a, r1b, r2b);
            const uint4 b31 = make_uint4(r3a, r1a, r3b, r1b);
            bf16x8m_t bx, by;
            __builtin_memcpy(&bx, &b12, 16);
            __builtin_memcpy(&by, &b31, 16);
            acc_n[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw1, bx, acc_n[bb], 0, 0, 0);
            acc_n[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw2, bx, acc_n[bb], 0, 0, 0);
            acc_n[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw3, by, acc_n[bb], 0, 0, 0);
          }
        }
        // raw = max over offsets + norm, for the lane's heads 4i + q of this pass
#pragma unroll
        for (int bb = 0; bb < GB; ++bb) {
          const int key = key_g + bb * 16 + m;
          float* rp = raw + (tk.row0 + tk.key0 + key) * G;
#pragma unroll
          for (int i = 0; i < NE; ++i) {
            const int h = h0 + 4 * i + q;
            const bool ok = key < tk.nkeys && h < h1;
            const float v = hm[bb][i] + acc_n[bb][i];
            *(ok ? rp + h : sink + lane) = v;
            const double dv = ok ? (double)v : 0.0;
            s1[i] += dv;
            s2[i] = fma(dv, dv, s2[i]);
          }
        }
#pragma unroll
        for (int bb = 0; bb < GB; ++bb)
#pragma unroll
          for (int st = 0; st < STEPS; ++st) kb[bb][st] = kn[bb][st];
        cur = nx;
      }
      // this wave's sums over its keys of ticket t for the pass's heads
      // (entry i of lane q is head h0 + 4i + q): wsum[t][wave][h] = (S1, S2)
#pragma unroll
      for (int i = 0; i < NE; ++i) {
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
          s1[i] += __shfl_xor(s1[i], o, 64);
          s2[i] += __shfl_xor(s2[i], o, 64);
        }
      }
      if (m == 0) {
#pragma unroll
        for (int i = 0; i < NE; ++i) {
          const int h = h0 + 4 * i + q;
          if (h < h1) {
            double* ws = wsum + (((int64_t)t * kWaves + wave) * G + h) * 2;
            ws[0] = s1[i];
            ws[1] = s2[i];
          }
        }
      }
    }
  }
}

// Per-ticket statistics from the per-wave sums, in wave order:
// chunk_stats[t][h] = (count, mean, M2) as the z pass reads them.
__global__ __launch_bounds__(256) void max_stats_merge_kernel(
    const SeqInfo* __restrict__ seqs, int S, int G, int total_tickets,
    const double* __restrict__ wsum, double* __restrict__ chunk_stats) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)total_tickets * G) return;
  const int t = (int)(idx / G), h = (int)(idx % G);
  const SeqInfo si = seqs[find_seq_by_ticket(seqs, S, t)];
  const int nch = (si.n + kScoreChunk - 1) / kScoreChunk;
  const int c = (t - si.chunk_base) % nch;
  const double cnt = (double)min(kScoreChunk, si.n - c * kScoreChunk);
  double a = 0.0, b2 = 0.0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const double* ws = wsum + (((int64_t)t * kWaves + w) * G + h) * 2;
    a += ws[0];
    b2 += ws[1];
  }
  const double mean = a / cnt;
  double* cs = chunk_stats + ((int64_t)t * kMaxGroup + h) * 3;
  cs[0] = cnt;
  cs[1] = mean;
  cs[2] = fmax(b2 - cnt * mean * mean, 0.0);
}

MaxOffsetsPlan plan_max_offsets(int d, int G, int n_offsets) {
  MaxOffsetsPlan mp;
  if (d % 32 != 0 || d < 32 || d > kMaxHeadDim || G < 1 || G > kMaxGroup || n_offsets < 1 ||
      n_offsets > kMaxOffsets)
    return mp;
  const int steps = d / 32;
  const size_t tile_bytes = (size_t)steps * kTrigTerms * 64 * sizeof(uint4);
  // the norm operands (three terms per step) take their share of the budget
  const size_t norm_bytes = (size_t)steps * 3 * 64 * sizeof(uint4);
  const int max_tiles = (int)((kMaxOffsetsLds - norm_bytes) / tile_bytes);
  // one slot per head: Dp/4 tiles per head, four heads per round of tiles
  int tph = (n_offsets + 3) / 4;
  if (tph <= max_tiles) {
    mp.spread = 1;
    mp.Dp = 4 * tph;
    const int hp_max = std::min(G, 4 * (max_tiles / tph));
    mp.npass = (G + hp_max - 1) / hp_max;
    mp.hp = (G + mp.npass - 1) / mp.npass;
    mp.nk = (mp.hp + 3) / 4;
  } else {
    // one head over all four slots: Dp/16 tiles per head, one head per round
    tph = (n_offsets + 15) / 16;
    if (tph > max_tiles) return mp;
    mp.spread = 4;
    mp.Dp = 16 * tph;
    const int hp_max = std::min(G, max_tiles / tph);
    mp.npass = (G + hp_max - 1) / hp_max;
    mp.hp = (G + mp.npass - 1) / mp.npass;
    mp.nk = mp.hp;
  }
  mp.tiles_per_head = tph;
  mp.ptiles = mp.nk * tph;
  mp.ok = true;
  return mp;
}

size_t max_offsets_operand_bytes(int d, int G, int nD, const MaxOffsetsPlan& mp, int64_t units,
                                 int64_t tickets) {
  if (!mp.ok) return 0;
  const int steps = d / 32;
  const size_t ops = (size_t)units * mp.npass *
                     ((size_t)mp.ptiles * steps * kTrigTerms * 64 + (size_t)steps * 3 * 64) *
                     sizeof(uint4);
  return ops + (size_t)tickets * kWaves * G * 2 * sizeof(double) + 64 * sizeof(float) +
         (size_t)nD * (d / 2) * sizeof(double2);
}

template <int STEPS, bool HALF>
static hipError_t launch_max_t(const SeqInfo* seqs, int S, int L, int Hkv, int G, int nD,
                               const MaxOffsetsPlan& mp, double theta, int total_tickets,
                               const double2* P, const float* W, const double2* E,
                               const double* offsets, void* operands, const uint16_t* k,
                               const Pages& pg, float* raw, double* chunk_stats,
                               hipStream_t st) {
  const int64_t units = (int64_t)S * L * Hkv;
  uint4* apack = reinterpret_cast<uint4*>(operands);
  uint4* wpack = apack + units * mp.npass * mp.ptiles * STEPS * kTrigTerms * 64;
  double* wsum = reinterpret_cast<double*>(wpack + units * mp.npass * STEPS * 3 * 64);
  float* sink = reinterpret_cast<float*>(wsum + (int64_t)total_tickets * kWaves * G * 2);
  double2* ph = reinterpret_cast<double2*>(sink + 64);
  constexpr int F = STEPS * 16;
  hipLaunchKernelGGL(max_phasor_kernel, dim3((unsigned)((nD * F + 255) / 256)), dim3(256), 0, st,
                     F, STEPS * 32, nD, theta, offsets, ph);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = units * mp.npass * mp.ptiles * STEPS * 64 + units * mp.npass * STEPS * 64;
  hipLaunchKernelGGL(pack_max_operands_kernel<STEPS>, dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, st, S, L, Hkv, G, HALF, mp, nD, P, W, E, ph, apack, wpack);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = ((size_t)mp.ptiles * kTrigTerms + 3) * STEPS * 64 * sizeof(uint4);
  const int grid = (total_tickets + kTicketsPerGroup - 1) / kTicketsPerGroup;
  constexpr int GB = STEPS <= 4 ? 4 : 2;
  const int ne = (mp.hp + 3) / 4;
#define TRI_LAUNCH(NE)                                                                         \
  hipLaunchKernelGGL((score_max_kernel<STEPS, GB, NE, HALF>), dim3(grid), dim3(kThreads), lds, \
                     st,                                                                       \
                     seqs, S, L * Hkv, G, mp, total_tickets, apack, wpack, k, pg, raw, wsum, sink)
  if (ne == 1)
    TRI_LAUNCH(1);
  else if (ne == 2)
    TRI_LAUNCH(2);
  else
    TRI_LAUNCH(4);
#undef TRI_LAUNCH
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t merge = (int64_t)total_tickets * G;
  hipLaunchKernelGGL(max_stats_merge_kernel, dim3((unsigned)((merge + 255) / 256)), dim3(256), 0,
                     st, seqs, S, G, total_tickets, wsum, chunk_stats);
  return hipGetLastError();
}

hipError_t launch_score_max(const SeqInfo* seqs, int S, int L, int Hkv, int G, int d, int nD,
                            const MaxOffsetsPlan& mp, double theta, int total_tickets,
                            const double2* P, const float* W, const double2* E,
                            const double* offsets, void* operands, const uint16_t* k,
                            float* raw, double* chunk_stats, double* unit_stats, float* scores,
                            double* head_stats, bool half, const Pages& pg, hipStream_t st) {
  if (total_tickets == 0) return hipSuccess;
  if (!mp.ok) return hipErrorInvalidValue;
  hipError_t e = hipErrorInvalidValue;
#define TRI_CASE(n, h)                                                                         \
  case n:                                                                                      \
    e = launch_max_t<n, h>(seqs, S, L, Hkv, G, nD, mp, theta, total_tickets, P, W, E, offsets, \
                           operands, k, pg, raw, chunk_stats, st);                             \
    break;
  // half split keeps both parts of a band in one lane only with an even
  // number of 32-wide steps
  if (half) {
    switch (d / 32) {
      TRI_CASE(2, true) TRI_CASE(4, true) TRI_CASE(6, true) TRI_CASE(8, true)
      default:
        return hipErrorInvalidValue;
    }
  } else {
    switch (d / 32) {
      TRI_CASE(1, false) TRI_CASE(2, false) TRI_CASE(3, false) TRI_CASE(4, false)
      TRI_CASE(5, false) TRI_CASE(6, false) TRI_CASE(7, false) TRI_CASE(8, false)
      default:
        return hipErrorInvalidValue;
    }
  }
#undef TRI_CASE
  if (e != hipSuccess) return e;
  return launch_zmax(seqs, S, L, Hkv, G, total_tickets, raw, chunk_stats, unit_stats, scores,
                     head_stats, st);
}

}  // namespace tri
