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
#include "tri_internal.hpp"

namespace tri {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One thread per (layer, query head, band); samples are summed in order in
// fp64, so the result does not depend on the launch shape.
__global__ __launch_bounds__(256) void calibrate_kernel(
    int L, int Hq, int d, double theta, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ q_pos, int64_t N, float* __restrict__ centre,
    float* __restrict__ absmean, float* __restrict__ R) {
  const int F = d >> 1;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)L * Hq * F) return;
  const int f = (int)(idx % F);
  const int h = (int)((idx / F) % Hq);
  const int l = (int)(idx / ((int64_t)F * Hq));
  const double omega = pow(theta, -2.0 * (double)f / (double)d);
  const uint32_t* words = reinterpret_cast<const uint32_t*>(q);
  const int64_t words_per_sample = (int64_t)Hq * F;
  int64_t off = ((int64_t)l * N * Hq + h) * F + f;
  double sr = 0.0, si = 0.0, sa = 0.0;
  for (int64_t t = 0; t < N; ++t, off += words_per_sample) {
    const uint32_t w = words[off];
    const double x = (double)bf16_lo(w), y = (double)bf16_hi(w);
    double re = x, im = y;
    if (q_pos) {
      double sn, cs;
      sincos(omega * (double)q_pos[t], &sn, &cs);
      re = x * cs + y * sn;   // (x + i y) * exp(-i omega p)
      im = y * cs - x * sn;
    }
    sr += re;
    si += im;
    sa += sqrt(x * x + y * y);  // |q_f| is unchanged by the rotation
  }
  const double inv = 1.0 / (double)N;
  const double cr = sr * inv, ci = si * inv, am = sa * inv;
  const int64_t o = ((int64_t)l * Hq + h) * F + f;
  centre[2 * o] = (float)cr;
  centre[2 * o + 1] = (float)ci;
  absmean[o] = (float)am;
  R[o] = am > 0.0 ? (float)(sqrt(cr * cr + ci * ci) / am) : 1.0f;
}

hipError_t launch_calibrate(int L, int Hq, int d, double theta, const uint16_t* q,
                            const int32_t* q_pos, int64_t n_samples, float* centre,
                            float* absmean, float* R, hipStream_t st) {
  const int64_t total = (int64_t)L * Hq * (d / 2);
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(calibrate_kernel, dim3(blocks), dim3(256), 0, st, L, Hq, d, theta, q,
                     q_pos, n_samples, centre, absmean, R);
  return hipGetLastError();
}

// P[l][h][f] = E[q_f] * C_f and W[l][h][f] = (1 - R_f) E|q_f| for every
// (layer, query head, band); E[s][f] = exp(i omega_f p_q(s)) per sequence.
// C_f is the mean of exp(i omega_f delta) over the offsets, summed in their
// order (the default set is {2^0, ..., 2^16}); without folding C_f = 1.
// All in fp64 (W is stored as fp32: it multiplies fp32 magnitudes).
__global__ __launch_bounds__(256) void prologue_kernel(
    int L, int Hq, int d, double theta, int S, const SeqInfo* __restrict__ seqs,
    const float* __restrict__ q_centre, const float* __restrict__ q_absmean,
    const float* __restrict__ q_R, const double* __restrict__ offsets, int nD, int fold,
    double2* __restrict__ P, float* __restrict__ W, double2* __restrict__ E,
    uint32_t* __restrict__ ctrl, double* __restrict__ stat_slots, int64_t n_stat_slots) {
  const int F = d >> 1;
  const int64_t n_stat = (int64_t)L * Hq * F;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // score control block and published-statistics slots of this call
  if (idx < kCtrlHeader) ctrl[idx] = 0u;
  if (idx < n_stat_slots)
    reinterpret_cast<unsigned long long*>(stat_slots)[idx] = kStatSentinel;
  if (idx < n_stat) {
    const int f = (int)(idx % F);
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
    const double qr = (double)q_centre[2 * idx], qi = (double)q_centre[2 * idx + 1];
    P[idx] = make_double2(qr * cr - qi * ci, qr * ci + qi * cr);
    W[idx] = (float)((1.0 - (double)q_R[idx]) * (double)q_absmean[idx]);
  } else if (idx < n_stat + (int64_t)S * F) {
    const int64_t j = idx - n_stat;
    const int s = (int)(j / F), f = (int)(j % F);
    const double omega = pow(theta, -2.0 * (double)f / (double)d);
    double sn, cs;
    sincos(omega * (double)seqs[s].p_q, &sn, &cs);
    E[j] = make_double2(cs, sn);
  }
}

hipError_t launch_prologue(int L, int Hq, int d, double theta, int S, const SeqInfo* seqs,
                           const float* q_centre, const float* q_absmean, const float* q_R,
                           const double* offsets, int n_offsets, bool fold, double2* P,
                           float* W, double2* E, uint32_t* ctrl, double* stat_slots,
                           int64_t n_stat_slots, hipStream_t st) {
  int64_t total = (int64_t)L * Hq * (d / 2) + (int64_t)S * (d / 2);
  if (n_stat_slots > total) total = n_stat_slots;
  if (kCtrlHeader > total) total = kCtrlHeader;
  const int nD = offsets ? n_offsets : 17;
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(prologue_kernel, dim3(blocks), dim3(256), 0, st, L, Hq, d, theta, S,
                     seqs, q_centre, q_absmean, q_R, offsets, nD, fold ? 1 : 0, P, W, E, ctrl,
                     stat_slots, n_stat_slots);
  return hipGetLastError();
}

}  // namespace tri
