// Offline calibration of per-band query statistics, and the per-call
// prologue that folds the statistics, the offset mean and the current
// position into per-band complex coefficients.
//
// Calibration follows the talk page "聊聊 TriAttention" (S_norm paragraph:
// R_f = |E[q_f]| / E[|q_f|], statistics of pre-RoPE queries) and the hyper.ai
// summary, section "方法".  The prologue rests on the same page's S_trig
// equation and the averaged-score equation over D = {1, 2, ..., 2^16}:
// band f of a query at p_q + delta contributes
//   Re(E[q_f] conj(k_f) exp(i omega_f (Delta + delta)))
// and with the stored key k'_f = k_f exp(i omega_f p_k) this is
//   Re(E[q_f] C_f exp(i omega_f p_q) conj(k'_f)),  C_f = mean_delta exp(i omega_f delta),
// so one complex coefficient per (sequence, query head, band) carries the
// whole offset mean and the key position drops out.
#include <cstring>

#include "tri_internal.hpp"

namespace tri {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Calibration runs in three steps, all deterministic:
//  1. a phasor table e^{-i omega_f p_t} per (sample, band), formed in fp64
//     and stored as fp32 (relative error ~6e-8): the de-rotation angle
//     depends on the band and the sample only, so one sincos serves every
//     layer and head;
//  2. partial sums per (layer, chunk of kCalibChunk samples, band): the
//     de-rotated band (fp32 rotation) and its magnitude (x^2 + y^2 of bf16
//     values is exact in fp32), summed in fp64 over the chunk's samples in
//     order;
//  3. a merge per (layer, head, band) over the chunks in order.
constexpr int kCalibChunk = 256;
constexpr int kCalibWaves = 4;   // waves per work-group, one chunk each
constexpr int kCalibBatch = 4;  // samples per register batch (two batches in flight)
constexpr int kXcds = 8;        // XCDs of the chip, each with its own L2

__global__ __launch_bounds__(256) void calib_phasor_kernel(int F, int d, double theta,
                                                           const int32_t* __restrict__ q_pos,
                                                           int64_t N, float2* __restrict__ ph) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= N * F) return;
  const int f = (int)(idx % F);
  const int64_t t = idx / F;
  const double omega = pow(theta, -2.0 * (double)f / (double)d);
  double sn, cs;
  sincos(omega * (double)q_pos[t], &sn, &cs);
  ph[idx] = make_float2((float)cs, (float)-sn);  // exp(-i omega p)
}

namespace {

// Bands 4j .. 4j+3 of head h in one sample row of W words (one word is two
// bf16 elements), as (x, y) pairs.  Interleaved: the four words
// h*F + 4j .. +3, one band each.  Half split: words h*F + 2j, +1 hold the
// real parts and words h*F + F/2 + 2j, +1 the imaginary parts.
template <bool HALF>
struct QuadLoad {
  uint4 a;
  __device__ __forceinline__ void load(const uint32_t* row, int h, int F, int j) {
    if constexpr (!HALF) {
      a = *reinterpret_cast<const uint4*>(row + h * F + 4 * j);
    } else {
      const uint2 re = *reinterpret_cast<const uint2*>(row + h * F + 2 * j);
      const uint2 im = *reinterpret_cast<const uint2*>(row + h * F + (F >> 1) + 2 * j);
      a = make_uint4(re.x, re.y, im.x, im.y);
    }
  }
  __device__ __forceinline__ void band(int b, float& x, float& y) const {
    if constexpr (!HALF) {
      const uint32_t w = b == 0 ? a.x : b == 1 ? a.y : b == 2 ? a.z : a.w;
      x = bf16_lo(w);
      y = bf16_hi(w);
    } else {
      const uint32_t wr = b < 2 ? a.x : a.y, wi = b < 2 ? a.z : a.w;
      x = (b & 1) ? bf16_hi(wr) : bf16_lo(wr);
      y = (b & 1) ? bf16_hi(wi) : bf16_lo(wi);
    }
  }
};

}  // namespace

// Work item (chunk group cg, layer l, slab zq), zq fastest; 64 * kCalibWaves
// threads.  Wave w takes chunk kCalibWaves*cg + w; lane i takes band quad
// zq*64 + i (head h = quad / (F/4), bands 4j .. 4j+3 with j = quad mod F/4),
// so a wave reads one contiguous stretch of each sample row.  Work-groups
// are dealt to the chip's 8 XCDs in turn (block b on XCD b mod 8, each XCD
// with its own L2); block b takes item (b mod 8)*per + b/8, so an XCD walks
// a contiguous run of items and the phasors of its few chunk groups stay in
// its L2 (1.4% faster than the plain 3-D grid at 10240 samples, 28 x 28).  Loads are double-buffered: the queries and phasors of the next
// kCalibBatch samples are in flight while the current ones are summed.
// partial[((l*chunks + c)*W + h*F + f)*3 + {0,1,2}] = sums of Re, Im, |q_f|.
template <bool HALF, bool ROTATE>
__global__ __launch_bounds__(64 * kCalibWaves) void calib_partial_kernel(
    int Hq, int F, int64_t N, int chunks, const uint16_t* __restrict__ q,
    const float2* __restrict__ ph, double* __restrict__ partial, int L, int nz, int64_t items,
    int64_t per) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (item >= items) return;
  const int zq = (int)(item % nz);
  const int64_t rr = item / nz;
  const int l = (int)(rr % L);
  const int c = (int)(rr / L) * kCalibWaves + (threadIdx.x >> 6);
  const int quads = F >> 2;
  const int quad = zq * 64 + lane;
  if (c >= chunks || quad >= Hq * quads) return;
  const int h = quad / quads, j = quad % quads;
  const int64_t W = (int64_t)Hq * F;
  const uint32_t* rows = reinterpret_cast<const uint32_t*>(q) + (int64_t)l * N * W;
  const int64_t t0 = (int64_t)c * kCalibChunk;
  const int64_t t1 = min(N, t0 + kCalibChunk);
  double sr[4] = {0.0, 0.0, 0.0, 0.0}, si[4] = {0.0, 0.0, 0.0, 0.0}, sa[4] = {0.0, 0.0, 0.0, 0.0};
  auto add = [&](const QuadLoad<HALF>& v, const float4* p) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      float x, y;
      v.band(b, x, y);
      float re = x, im = y;
      if constexpr (ROTATE) {  // (x + i y) * exp(-i omega p)
        const float4 pp = p[b >> 1];
        const float px = (b & 1) ? pp.z : pp.x, py = (b & 1) ? pp.w : pp.y;
        re = fmaf(x, px, -y * py);
        im = fmaf(x, py, y * px);
      }
      sr[b] += (double)re;
      si[b] += (double)im;
      sa[b] += (double)__builtin_amdgcn_sqrtf(fmaf(x, x, y * y));  // |q_f|: unchanged by the rotation
    }
  };
  // two batches of NB samples in registers: the loads of batch i+1 are in
  // flight while batch i is summed (sample indexes past the chunk are
  // clamped to its last sample and their values dropped)
  constexpr int NB = kCalibBatch;
  struct Batch {
    QuadLoad<HALF> v[NB];
    float4 p[NB][2];
  };
  auto fetch = [&](Batch& bt, int64_t tb) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int64_t tt = min(tb + u, t1 - 1);
      bt.v[u].load(rows + tt * W, h, F, j);
      if constexpr (ROTATE) {
        const float4* pq = reinterpret_cast<const float4*>(ph + tt * F + 4 * j);
        bt.p[u][0] = pq[0];
        bt.p[u][1] = pq[1];
      }
    }
  };
  auto sum = [&](const Batch& bt, int64_t tb) {
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (tb + u < t1) add(bt.v[u], bt.p[u]);
  };
  Batch A, B;
  fetch(A, t0);
  for (int64_t t = t0; t < t1; t += 2 * NB) {
    fetch(B, t + NB);
    sum(A, t);
    fetch(A, t + 2 * NB);
    sum(B, t + NB);
  }
  double* out = partial + (((int64_t)l * chunks + c) * W + (int64_t)h * F + 4 * j) * 3;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    out[3 * b] = sr[b];
    out[3 * b + 1] = si[b];
    out[3 * b + 2] = sa[b];
  }
}

__global__ __launch_bounds__(256) void calib_merge_kernel(
    int L, int W, int64_t N, int chunks, const double* __restrict__ partial,
    float* __restrict__ centre, float* __restrict__ absmean, float* __restrict__ R) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)L * W) return;
  const int l = (int)(idx / W), w = (int)(idx % W);
  double sr = 0.0, si = 0.0, sa = 0.0;
  for (int c = 0; c < chunks; ++c) {
    const double* p = partial + (((int64_t)l * chunks + c) * W + w) * 3;
    sr += p[0];
    si += p[1];
    sa += p[2];
  }
  const double inv = 1.0 / (double)N;
  const double cr = sr * inv, ci = si * inv, am = sa * inv;
  centre[2 * idx] = (float)cr;
  centre[2 * idx + 1] = (float)ci;
  absmean[idx] = (float)am;
  R[idx] = am > 0.0 ? (float)(sqrt(cr * cr + ci * ci) / am) : 1.0f;
}

size_t calibrate_workspace_bytes(int L, int Hq, int d, int64_t n_samples) {
  const int64_t F = d / 2;
  const int64_t chunks = (n_samples + kCalibChunk - 1) / kCalibChunk;
  return (size_t)(n_samples * F * 8) + (size_t)(L * chunks * Hq * F * 3 * 8) + 256;
}

hipError_t launch_calibrate(int L, int Hq, int d, double theta, bool half, const uint16_t* q,
                            const int32_t* q_pos, int64_t n_samples, float* centre,
                            float* absmean, float* R, void* workspace, hipStream_t st) {
  const int F = d / 2, W = Hq * F;
  const int chunks = (int)((n_samples + kCalibChunk - 1) / kCalibChunk);
  float2* ph = nullptr;
  char* ws = (char*)workspace;
  double* partial = (double*)(ws + ((n_samples * F * 8 + 255) / 256) * 256);
  if (q_pos) {
    ph = (float2*)ws;
    const int64_t n = n_samples * F;
    hipLaunchKernelGGL(calib_phasor_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, F,
                       d, theta, q_pos, n_samples, ph);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nz = (Hq * (F / 4) + 63) / 64;
  const int64_t items = (int64_t)((chunks + kCalibWaves - 1) / kCalibWaves) * L * nz;
  const int64_t per = (items + kXcds - 1) / kXcds;
  if (per * kXcds > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)(per * kXcds));
  const dim3 block(64 * kCalibWaves);
  if (half && ph)
    hipLaunchKernelGGL((calib_partial_kernel<true, true>), grid, block, 0, st, Hq, F, n_samples,
                       chunks, q, ph, partial, L, nz, items, per);
  else if (half)
    hipLaunchKernelGGL((calib_partial_kernel<true, false>), grid, block, 0, st, Hq, F, n_samples,
                       chunks, q, ph, partial, L, nz, items, per);
  else if (ph)
    hipLaunchKernelGGL((calib_partial_kernel<false, true>), grid, block, 0, st, Hq, F, n_samples,
                       chunks, q, ph, partial, L, nz, items, per);
  else
    hipLaunchKernelGGL((calib_partial_kernel<false, false>), grid, block, 0, st, Hq, F, n_samples,
                       chunks, q, ph, partial, L, nz, items, per);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t m = (int64_t)L * W;
  hipLaunchKernelGGL(calib_merge_kernel, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, st, L, W,
                     n_samples, chunks, partial, centre, absmean, R);
  return hipGetLastError();
}

// P[l][h][f] = E[q_f] * C_f and W[l][h][f] = (1 - R_f) E|q_f| for every
// (layer, query head, band); E[s][f] = exp(i omega_f p_q(s)) per sequence.
// C_f is the mean of exp(i omega_f delta) over the offsets, summed in their
// order (the default set is {2^0, ..., 2^16}); without folding C_f = 1.
// All in fp64 (W is stored as fp32: it multiplies fp32 magnitudes).
// With plan_words > 0 the call's sequence plan arrives in the arguments:
// block 0 writes it to seqs (for the kernels after this one) and the
// query positions are read from the arguments.
__global__ __launch_bounds__(256) void prologue_kernel(
    int L, int Hq, int d, double theta, int S, SeqInfo* __restrict__ seqs, const ArgWords plan,
    int plan_words, const float* __restrict__ q_centre, const float* __restrict__ q_absmean,
    const float* __restrict__ q_R, const double* __restrict__ offsets, int nD, int fold,
    double2* __restrict__ P, float* __restrict__ W, double2* __restrict__ E,
    uint32_t* __restrict__ ctrl, int64_t n_ctrl, double* __restrict__ stat_slots,
    int64_t n_stat_slots) {
  const int F = d >> 1;
  const int64_t n_stat = (int64_t)L * Hq * F;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < plan_words; i += blockDim.x)
      reinterpret_cast<uint32_t*>(seqs)[i] = plan.w[i];
  // score control words and published-statistics slots of this call
  if (idx < n_ctrl) ctrl[idx] = 0u;
  if (idx < n_stat_slots)
    reinterpret_cast<unsigned long long*>(stat_slots)[idx] = kStatSentinel;
  // C_f = mean over the offsets of exp(i omega_f delta), once per band per
  // block (F <= 128), in the blocks that form P (the others only reset the
  // statistics slots)
  __shared__ double2 cf[kMaxHeadDim / 2];
  const bool forms_p = (int64_t)blockIdx.x * blockDim.x < n_stat;
  for (int f = threadIdx.x; forms_p && f < F; f += blockDim.x) {
    const double omega = pow(theta, -2.0 * (double)f / (double)d);
    double cr = 1.0, ci = 0.0;
    if (fold) {
      cr = 0.0;
      for (int j = 0; j < nD; ++j) {
        const double delta = offsets ? offsets[j] : ldexp(1.0, j);
        double sn, cs;
        sincos(omega * delta, &sn, &cs);
        cr += cs;
        ci += sn;
      }
      const double inv = 1.0 / (double)nD;
      cr *= inv;
      ci *= inv;
    }
    cf[f] = make_double2(cr, ci);
  }
  if (forms_p) __syncthreads();  // block-uniform
  if (idx < n_stat) {
    const int f = (int)(idx % F);
    const double cr = cf[f].x, ci = cf[f].y;
    const double qr = (double)q_centre[2 * idx], qi = (double)q_centre[2 * idx + 1];
    P[idx] = make_double2(qr * cr - qi * ci, qr * ci + qi * cr);
    W[idx] = (float)((1.0 - (double)q_R[idx]) * (double)q_absmean[idx]);
  } else if (idx < n_stat + (int64_t)S * F) {
    const int64_t j = idx - n_stat;
    const int s = (int)(j / F), f = (int)(j % F);
    const double omega = pow(theta, -2.0 * (double)f / (double)d);
    double sn, cs;
    const int32_t p_q =
        plan_words ? reinterpret_cast<const SeqInfo*>(plan.w)[s].p_q : seqs[s].p_q;
    sincos(omega * (double)p_q, &sn, &cs);
    E[j] = make_double2(cs, sn);
  }
}

hipError_t launch_prologue(int L, int Hq, int d, double theta, int S, const SeqInfo* seqs,
                           const SeqInfo* plan_host, const float* q_centre,
                           const float* q_absmean, const float* q_R, const double* offsets,
                           int n_offsets, bool fold, double2* P, float* W, double2* E,
                           uint32_t* ctrl, int64_t n_ctrl, double* stat_slots,
                           int64_t n_stat_slots, hipStream_t st) {
  int64_t total = (int64_t)L * Hq * (d / 2) + (int64_t)S * (d / 2);
  if (n_stat_slots > total) total = n_stat_slots;
  if (n_ctrl > total) total = n_ctrl;
  const int nD = offsets ? n_offsets : 17;
  const int blocks = (int)((total + 255) / 256);
  ArgWords plan;
  int plan_words = 0;
  if (plan_host) {
    const size_t bytes = (size_t)S * sizeof(SeqInfo);
    if (bytes > sizeof(plan.w)) return hipErrorInvalidValue;
    std::memcpy(plan.w, plan_host, bytes);
    plan_words = (int)(bytes / 4);
  }
  hipLaunchKernelGGL(prologue_kernel, dim3(blocks), dim3(256), 0, st, L, Hq, d, theta, S,
                     const_cast<SeqInfo*>(seqs), plan, plan_words, q_centre, q_absmean, q_R,
                     offsets, nD, fold ? 1 : 0, P, W, E, ctrl, n_ctrl, stat_slots, n_stat_slots);
  return hipGetLastError();
}

// Host tables of a call (the sequence plan, an offset set, decode items)
// written to device memory from kernel arguments, 2560 bytes per launch:
// the data travels with the launch, so nothing on the host has to outlive
// the call, no staging memory is held, and the copy is an ordinary kernel
// node under stream capture.

__global__ __launch_bounds__(256) void write_args_kernel(ArgWords a, int n,
                                                         uint32_t* __restrict__ dst) {
  for (int i = threadIdx.x; i < n; i += 256) dst[i] = a.w[i];
}

hipError_t launch_write_args(void* dst, const void* host, size_t bytes, hipStream_t st) {
  if (bytes % 4 != 0) return hipErrorInvalidValue;
  const size_t words = bytes / 4;
  const uint32_t* src = static_cast<const uint32_t*>(host);
  uint32_t* out = static_cast<uint32_t*>(dst);
  for (size_t w0 = 0; w0 < words; w0 += kArgWords) {
    const int n = (int)(words - w0 < (size_t)kArgWords ? words - w0 : kArgWords);
    ArgWords a;
    std::memcpy(a.w, src + w0, (size_t)n * 4);
    hipLaunchKernelGGL(write_args_kernel, dim3(1), dim3(256), 0, st, a, n, out + w0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tri
