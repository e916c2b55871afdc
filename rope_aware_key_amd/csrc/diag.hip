// Reconstruction diagnostic (shibing624 blog review, Fig. 1(D) and Fig. 7):
// how well the trig series built from the query centres follows the real
// attention logits.  For layer l and query head h (KV head g = h / G), over
// every pair of a sample query j and a key i:
//   x_ji = S_trig(k_i, p_j - p_i) = sum_f Re(E[q_f] exp(i omega_f p_j) conj(k'_{i,f}))
//   y_ji = <q'_j, k'_i>   (the post-RoPE logit, unscaled)
// (talk page "聊聊 TriAttention", logit decomposition and S_trig equation:
// with the stored key k'_f = k_f exp(i omega_f p_k) the x form is
// |E q_f||k_f| cos(omega_f (p_j - p_i) + arg E q_f - arg k_f)), and
// r[l][h] = Pearson(x, y) over all n_q * n_k pairs.
//
// Both are 16 x 16 tiles of (query x key) products on
// v_mfma_f32_16x16x32_bf16: queries and keys are bf16 already, so y is one
// exact MFMA per 32-wide step; the rotated centres are formed per query in
// fp64 and split into three bf16 terms (fp32-accurate; the score kernels
// keep two, which their 1e-4 score bar allows).  A wave owns 16 queries of one (layer, head) and streams the
// KV head's keys in blocks of 16, the next block's loads in flight while
// the current one is multiplied; each lane sums x, y, x^2, y^2, xy over
// its valid pairs in fp64, the wave reduces them and a merge kernel adds
// the waves of a head in order (deterministic).
#include "tri_internal.hpp"

namespace tri {

typedef short bf16x8d_t __attribute__((ext_vector_type(8)));
typedef float f32x4d_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int kDiagWaves = 4;

__device__ __forceinline__ uint32_t bf16_rne_d(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void split3_d(double x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = bf16_rne_d((float)x);
  const double r1 = x - (double)__uint_as_float(hi << 16);
  mid = bf16_rne_d((float)r1);
  const double r2 = r1 - (double)__uint_as_float(mid << 16);
  lo = bf16_rne_d((float)r2);
}

__device__ __forceinline__ uint4 pack8_d(const uint32_t (&v)[8]) {
  return make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16),
                    v[6] | (v[7] << 16));
}

}  // namespace

// Grid: (L*Hq) x ceil(n_q / 64) work-groups of 4 waves; wave w takes query
// tile 4*blockIdx.y + w (16 queries).  partial[(lh*tiles + tile)*5 + k]:
// the tile's sums (x, y, xx, yy, xy).
template <int STEPS, bool HALF>
__global__ __launch_bounds__(64 * kDiagWaves) void trig_corr_kernel(
    int Hq, int Hkv, int64_t n_q, int64_t n_k, double theta, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ q_pos, const uint16_t* __restrict__ k,
    const int32_t* __restrict__ k_pos, const float* __restrict__ q_centre,
    double* __restrict__ partial) {
  constexpr int D = STEPS * 32;
  constexpr int F = STEPS * 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, qd = lane >> 4;
  const int lh = blockIdx.x;
  const int l = lh / Hq, h = lh % Hq;
  const int g = h / (Hq / Hkv);
  const int64_t tiles = (n_q + 15) / 16;
  const int64_t tile = (int64_t)blockIdx.y * kDiagWaves + wave;
  if (tile >= tiles) return;

  // A operands of this lane's query row j = 16*tile + m (clamped; rows past
  // n_q are masked out of the sums)
  const int64_t j = min<int64_t>(tile * 16 + m, n_q - 1);
  const uint4* qrow = reinterpret_cast<const uint4*>(q + (((int64_t)l * n_q + j) * Hq + h) * D);
  const double pj = (double)q_pos[j];
  uint4 ay[STEPS], axh[STEPS], axm[STEPS], axl[STEPS];
  const float* cbase = q_centre + ((int64_t)l * Hq + h) * F * 2;
  // rotated centre of band f at the query's position:
  // E[q_f] exp(i omega_f p_j), omega_f = theta^(-2f/d)
  auto rotated = [&](int f, double& re, double& im) {
    const double omega = pow(theta, -2.0 * (double)f / (double)D);
    double sn, cs;
    sincos(omega * pj, &sn, &cs);
    const double cr = (double)cbase[2 * f], ci = (double)cbase[2 * f + 1];
    re = cr * cs - ci * sn;
    im = cr * sn + ci * cs;
  };
#pragma unroll
  for (int st = 0; st < STEPS; ++st) ay[st] = qrow[4 * st + qd];
  if constexpr (!HALF) {
    // interleaved pairs: the lane's eight elements of a step are bands
    // 16st + 4qd + u, real part then imaginary part
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      uint32_t h3[8], m3[8], l3[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        double re, im;
        rotated(16 * st + 4 * qd + u, re, im);
        split3_d(re, h3[2 * u], m3[2 * u], l3[2 * u]);
        split3_d(im, h3[2 * u + 1], m3[2 * u + 1], l3[2 * u + 1]);
      }
      axh[st] = pack8_d(h3);
      axm[st] = pack8_d(m3);
      axl[st] = pack8_d(l3);
    }
  } else if constexpr (STEPS % 2 == 0) {
    // half-split pairs, d a multiple of 64: element e < d/2 is the real part
    // of band e and element e + d/2, in step st + STEPS/2 of the same lane,
    // its imaginary part
#pragma unroll
    for (int st = 0; st < STEPS / 2; ++st) {
      uint32_t h3[8], m3[8], l3[8], h4[8], m4[8], l4[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        double re, im;
        rotated(32 * st + 8 * qd + j, re, im);
        split3_d(re, h3[j], m3[j], l3[j]);
        split3_d(im, h4[j], m4[j], l4[j]);
      }
      axh[st] = pack8_d(h3);
      axm[st] = pack8_d(m3);
      axl[st] = pack8_d(l3);
      axh[st + STEPS / 2] = pack8_d(h4);
      axm[st + STEPS / 2] = pack8_d(m4);
      axl[st + STEPS / 2] = pack8_d(l4);
    }
  } else {
    // half-split pairs with an odd number of 32-wide steps: a step straddles
    // d/2, so each element takes its own band and part
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      uint32_t h3[8], m3[8], l3[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int e = 32 * st + 8 * qd + j;
        double re, im;
        rotated(elem_band(e, D, true), re, im);
        split3_d(elem_part(e, D, true) ? im : re, h3[j], m3[j], l3[j]);
      }
      axh[st] = pack8_d(h3);
      axm[st] = pack8_d(m3);
      axl[st] = pack8_d(l3);
    }
  }
  (void)k_pos;  // the key position cancels: keys are stored rotated

  double sx = 0.0, sy = 0.0, sxx = 0.0, syy = 0.0, sxy = 0.0;
  const uint16_t* kunit = k + ((int64_t)l * Hkv + g) * n_k * D;
  const int64_t blocks = (n_k + 15) / 16;
  // B operands of block blk (key 16*blk + m, clamped), one block ahead
  auto load_keys = [&](int64_t blk, uint4 (&kb)[STEPS]) {
    const uint4* krow =
        reinterpret_cast<const uint4*>(kunit + min<int64_t>(blk * 16 + m, n_k - 1) * D);
#pragma unroll
    for (int st = 0; st < STEPS; ++st) kb[st] = krow[4 * st + qd];
  };
  uint4 kcur[STEPS];
  load_keys(0, kcur);
  for (int64_t blk = 0; blk < blocks; ++blk) {
    const int64_t key = blk * 16 + m;
    uint4 knext[STEPS];
    load_keys(blk + 1 < blocks ? blk + 1 : blk, knext);
    f32x4d_t accx = {0.f, 0.f, 0.f, 0.f}, accy = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const uint4 kb = kcur[st];
      bf16x8d_t bk, a0, a1, a2, a3;
      __builtin_memcpy(&bk, &kb, 16);
      __builtin_memcpy(&a0, &ay[st], 16);
      __builtin_memcpy(&a1, &axh[st], 16);
      __builtin_memcpy(&a2, &axm[st], 16);
      __builtin_memcpy(&a3, &axl[st], 16);
      accy = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, bk, accy, 0, 0, 0);
      accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, bk, accx, 0, 0, 0);
      accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a2, bk, accx, 0, 0, 0);
      accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a3, bk, accx, 0, 0, 0);
    }
    // lane (m, qd) holds queries 16*tile + 4qd + i against key m of the block
    const bool key_ok = key < n_k;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = key_ok && tile * 16 + 4 * qd + i < n_q;
      const double x = ok ? (double)accx[i] : 0.0, y = ok ? (double)accy[i] : 0.0;
      sx += x;
      sy += y;
      sxx = fma(x, x, sxx);
      syy = fma(y, y, syy);
      sxy = fma(x, y, sxy);
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) kcur[st] = knext[st];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sx += __shfl_xor(sx, o, 64);
    sy += __shfl_xor(sy, o, 64);
    sxx += __shfl_xor(sxx, o, 64);
    syy += __shfl_xor(syy, o, 64);
    sxy += __shfl_xor(sxy, o, 64);
  }
  if (lane == 0) {
    double* out = partial + ((int64_t)lh * tiles + tile) * 5;
    out[0] = sx;
    out[1] = sy;
    out[2] = sxx;
    out[3] = syy;
    out[4] = sxy;
  }
}

// r[lh] from the tiles' sums, added in tile order:
// r = cov(x, y) / sqrt(var x * var y), 0 when either variance is 0.
__global__ __launch_bounds__(256) void trig_corr_merge_kernel(int LHq, int64_t tiles, double n,
                                                              const double* __restrict__ partial,
                                                              double* __restrict__ r) {
  const int lh = blockIdx.x * blockDim.x + threadIdx.x;
  if (lh >= LHq) return;
  double s[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
  for (int64_t t = 0; t < tiles; ++t)
#pragma unroll
    for (int c = 0; c < 5; ++c) s[c] += partial[((int64_t)lh * tiles + t) * 5 + c];
  const double mx = s[0] / n, my = s[1] / n;
  const double vx = s[2] / n - mx * mx, vy = s[3] / n - my * my;
  const double cxy = s[4] / n - mx * my;
  r[lh] = (vx > 0.0 && vy > 0.0) ? cxy / sqrt(vx * vy) : 0.0;
}

size_t trig_corr_workspace_bytes(int L, int Hq, int64_t n_q) {
  return (size_t)L * Hq * ((n_q + 15) / 16) * 5 * sizeof(double);
}

hipError_t launch_trig_corr(int L, int Hq, int Hkv, int d, int64_t n_q, int64_t n_k, double theta,
                            bool half, const uint16_t* q, const int32_t* q_pos, const uint16_t* k,
                            const int32_t* k_pos, const float* q_centre, double* partial,
                            double* r, hipStream_t st) {
  const int64_t tiles = (n_q + 15) / 16;
  const dim3 grid((unsigned)(L * Hq), (unsigned)((tiles + kDiagWaves - 1) / kDiagWaves));
  switch (d / 32) {
#define TRI_CASE(n)                                                                         \
  case n:                                                                                   \
    if (half)                                                                               \
      hipLaunchKernelGGL((trig_corr_kernel<n, true>), grid, dim3(64 * kDiagWaves), 0, st,   \
                         Hq, Hkv, n_q, n_k, theta, q, q_pos, k, k_pos, q_centre, partial);  \
    else                                                                                    \
      hipLaunchKernelGGL((trig_corr_kernel<n, false>), grid, dim3(64 * kDiagWaves), 0, st,  \
                         Hq, Hkv, n_q, n_k, theta, q, q_pos, k, k_pos, q_centre, partial);  \
    break;
    TRI_CASE(1) TRI_CASE(2) TRI_CASE(3) TRI_CASE(4) TRI_CASE(5) TRI_CASE(6) TRI_CASE(7)
    TRI_CASE(8)
#undef TRI_CASE
    default:
      return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(trig_corr_merge_kernel, dim3((L * Hq + 255) / 256), dim3(256), 0, st,
                     L * Hq, tiles, (double)n_q * (double)n_k, partial, r);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Read-bandwidth probe: the rate a plain streaming read reaches on this
// device, the practical ceiling of the score kernel's K stream.  Each
// work-group reads one contiguous span of src (as each of the score
// kernel's work-groups streams one span of K: on this chip contiguous spans
// read 5-7% faster than a grid-strided sweep) with 16-byte non-temporal
// loads, four per lane in flight, and XORs the words; one atomic per wave
// folds them into *sink (so no load can be dropped).
// ---------------------------------------------------------------------------
typedef uint32_t v4u_probe_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_probe_kernel(const v4u_probe_t* __restrict__ src,
                                                           int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;  // 16-byte words per work-group
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < n16 ? beg + per : n16;
  int64_t i = beg + threadIdx.x;
  v4u_probe_t x = {0u, 0u, 0u, 0u};
  for (; i + 3 * 256 < end; i += 4 * 256) {
    const v4u_probe_t a = __builtin_nontemporal_load(src + i);
    const v4u_probe_t b = __builtin_nontemporal_load(src + i + 256);
    const v4u_probe_t c = __builtin_nontemporal_load(src + i + 512);
    const v4u_probe_t d = __builtin_nontemporal_load(src + i + 768);
    x ^= a ^ b ^ c ^ d;
  }
  for (; i < end; i += 256) x ^= __builtin_nontemporal_load(src + i);
  uint32_t w = x.x ^ x.y ^ x.z ^ x.w;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) w ^= __shfl_xor(w, o, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, w);
}

hipError_t launch_stream_probe(const void* src, int64_t bytes, uint32_t* sink, hipStream_t st) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void*>(&stream_probe_kernel), 256, 0);
  if (e != hipSuccess) return e;
  const int64_t n16 = bytes / 16;
  int64_t grid = (int64_t)cus * (per_cu < 1 ? 1 : per_cu);
  if (grid > (n16 + 255) / 256) grid = (n16 + 255) / 256;
  if (grid < 1) return hipSuccess;
  hipLaunchKernelGGL(stream_probe_kernel, dim3((unsigned)grid), dim3(256), 0, st,
                     reinterpret_cast<const v4u_probe_t*>(src), n16, sink);
  return hipGetLastError();
}

}  // namespace tri
