// Kernels of the decode-loop driver (tutorial page, streaming-generation
// paragraph: each decode step appends the new token's K and V to the cache,
// eviction runs when the cache is over budget and the most recent tokens are
// protected; its renormalisation paragraph keeps attention-sink tokens;
// hyper.ai summary, section "方法": prune once every 128 generated tokens).
#include "tri_internal.hpp"

namespace tri {

// One token per sequence: unit u = s*LH + lg of the [S][L][Hkv][d] input
// goes to row items[s].row0 + lg*stride of the cache.  A thread moves 16
// bytes of K and of V; the first thread of a unit writes the position.
__device__ __forceinline__ void append_one(const DecodeItem& it, int64_t unit, int part,
                                           int lg, int d, int64_t stride,
                                           const uint16_t* __restrict__ k_new,
                                           const uint16_t* __restrict__ v_new,
                                           uint16_t* __restrict__ k, uint16_t* __restrict__ v,
                                           int32_t* __restrict__ pos) {
  const int64_t row = it.row0 + (int64_t)lg * stride;
  reinterpret_cast<uint4*>(k + row * d)[part] = reinterpret_cast<const uint4*>(k_new + unit * d)[part];
  reinterpret_cast<uint4*>(v + row * d)[part] = reinterpret_cast<const uint4*>(v_new + unit * d)[part];
  if (part == 0) pos[row] = it.pos;
}

// items in device memory (uploaded by the caller of launch_append)
__global__ __launch_bounds__(256) void append_kernel(
    const DecodeItem* __restrict__ items, int S, int LH, int d, int64_t stride,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k, uint16_t* __restrict__ v, int32_t* __restrict__ pos) {
  const int parts = d >> 3;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)S * LH * parts) return;
  const int part = (int)(idx % parts);
  const int64_t unit = idx / parts;
  append_one(items[unit / LH], unit, part, (int)(unit % LH), d, stride, k_new, v_new, k, v, pos);
}

// Up to kAppendInline sequences: the items ride in the kernel arguments, so
// a decode step queues one launch and no host-to-device copy.
struct AppendItems {
  DecodeItem it[kAppendInline];
};

__global__ __launch_bounds__(256) void append_inline_kernel(
    const AppendItems items, int S, int LH, int d, int64_t stride,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ k, uint16_t* __restrict__ v, int32_t* __restrict__ pos) {
  const int parts = d >> 3;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)S * LH * parts) return;
  const int part = (int)(idx % parts);
  const int64_t unit = idx / parts;
  append_one(items.it[unit / LH], unit, part, (int)(unit % LH), d, stride, k_new, v_new, k, v,
             pos);
}

// For every unit that is pruned (b < n): scores of its first `sink` and last
// `recent` keys become +inf.  Scores from the score kernels are finite
// z-scores, so the top-B then keeps exactly these keys plus the best of the
// rest, ranked as before (lower index on ties).  sink + recent <= b.
__global__ __launch_bounds__(256) void protect_kernel(const SeqInfo* __restrict__ seqs, int LH,
                                                      int sink, int recent,
                                                      float* __restrict__ scores) {
  const int unit = blockIdx.x;
  const SeqInfo si = seqs[unit / LH];
  if (si.b >= si.n) return;
  const int lg = unit % LH;
  float* row = scores + si.row_base + (int64_t)lg * si.in_stride;
  for (int j = threadIdx.x; j < sink + recent; j += blockDim.x) {
    const int i = j < sink ? j : si.n - recent + (j - sink);
    row[i] = __builtin_huge_valf();
  }
}

hipError_t launch_append(const DecodeItem* items, int S, int LH, int d, int64_t stride,
                         const uint16_t* k_new, const uint16_t* v_new, uint16_t* k, uint16_t* v,
                         int32_t* pos, hipStream_t st) {
  const int64_t threads = (int64_t)S * LH * (d / 8);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st,
                     items, S, LH, d, stride, k_new, v_new, k, v, pos);
  return hipGetLastError();
}

hipError_t launch_append_inline(const DecodeItem* host_items, int S, int LH, int d,
                                int64_t stride, const uint16_t* k_new, const uint16_t* v_new,
                                uint16_t* k, uint16_t* v, int32_t* pos, hipStream_t st) {
  if (S > kAppendInline) return hipErrorInvalidValue;
  const int64_t threads = (int64_t)S * LH * (d / 8);
  if (threads == 0) return hipSuccess;
  AppendItems items = {};
  for (int s = 0; s < S; ++s) items.it[s] = host_items[s];
  hipLaunchKernelGGL(append_inline_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     st, items, S, LH, d, stride, k_new, v_new, k, v, pos);
  return hipGetLastError();
}

hipError_t launch_protect(const SeqInfo* seqs, int S, int LH, int sink, int recent,
                          float* scores, hipStream_t st) {
  if (S == 0 || sink + recent == 0) return hipSuccess;
  hipLaunchKernelGGL(protect_kernel, dim3((unsigned)(S * LH)), dim3(64), 0, st, seqs, LH, sink,
                     recent, scores);
  return hipGetLastError();
}

}  // namespace tri
