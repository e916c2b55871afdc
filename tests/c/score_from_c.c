/*
 * tri_score and tri_select_compact called from plain C with the HIP runtime
 * API: no Python, no torch.  The caller owns every buffer (hipMalloc), as
 * the ABI requires.
 *
 *   score_from_c DIR d Hq Hkv L S
 *
 * DIR holds little-endian raw arrays written by the test:
 *   cu_len.bin int64[S+1], cur_pos.bin int32[S], budget.bin int32[S],
 *   k.bin uint16[rows*d] (bf16), k_pos.bin int32[rows],
 *   centre.bin float[L*Hq*d], absmean.bin float[L*Hq*d/2], R.bin float[L*Hq*d/2].
 * Writes DIR/scores.bin float[rows] and DIR/kept.bin int32[kept rows].
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>

#include "triattn.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(2); }
  void* p = malloc(bytes ? bytes : 1);
  if (bytes && fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(2); }
  fclose(f);
  return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(2); }
  fclose(f);
}

#define HIP(x)                                                              \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));               \
      return 3;                                                             \
    }                                                                       \
  } while (0)

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 16) != hipSuccess) { fprintf(stderr, "hipMalloc\n"); exit(3); }
  if (bytes && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "hipMemcpy\n");
    exit(3);
  }
  return d;
}

int main(int argc, char** argv) {
  if (argc != 7) { fprintf(stderr, "usage: %s DIR d Hq Hkv L S\n", argv[0]); return 2; }
  const char* dir = argv[1];
  tri_shape sh = {atoi(argv[2]), atoi(argv[3]), atoi(argv[4]), atoi(argv[5]), 10000.0,
                  TRI_ROPE_INTERLEAVED};
  const int S = atoi(argv[6]);
  const int d = sh.head_dim, F = d / 2, Hkv = sh.num_kv_heads, L = sh.num_layers;
  const size_t stat = (size_t)L * sh.num_q_heads * F;

  int64_t* cu = read_file(dir, "cu_len.bin", (S + 1) * sizeof(int64_t));
  int32_t* cur = read_file(dir, "cur_pos.bin", S * sizeof(int32_t));
  int32_t* budget = read_file(dir, "budget.bin", S * sizeof(int32_t));
  const size_t rows = (size_t)L * Hkv * cu[S];
  size_t out_rows = 0;
  for (int s = 0; s < S; ++s) {
    const int64_t n = cu[s + 1] - cu[s];
    out_rows += (size_t)L * Hkv * (budget[s] < n ? budget[s] : n);
  }
  void* k = to_device(read_file(dir, "k.bin", rows * d * 2), rows * d * 2);
  void* kp = to_device(read_file(dir, "k_pos.bin", rows * 4), rows * 4);
  void* c = to_device(read_file(dir, "centre.bin", stat * 2 * 4), stat * 2 * 4);
  void* a = to_device(read_file(dir, "absmean.bin", stat * 4), stat * 4);
  void* r = to_device(read_file(dir, "R.bin", stat * 4), stat * 4);

  void *scores = NULL, *kept = NULL, *ws = NULL;
  const size_t wsb = tri_workspace_bytes(&sh, S, cu);
  HIP(hipMalloc(&scores, rows * 4 + 16));
  HIP(hipMalloc(&kept, out_rows * 4 + 16));
  HIP(hipMalloc(&ws, wsb ? wsb : 16));
  hipStream_t st;
  HIP(hipStreamCreate(&st));
  tri_status t = tri_score(&sh, S, cu, cur, k, kp, c, a, r, scores, NULL, NULL, ws, wsb, st);
  if (t != TRI_OK) { fprintf(stderr, "tri_score: %s\n", tri_last_error()); return 4; }
  t = tri_select_compact(&sh, S, cu, budget, scores, NULL, NULL, NULL, kept, NULL, NULL, NULL,
                         ws, wsb, st);
  if (t != TRI_OK) { fprintf(stderr, "tri_select_compact: %s\n", tri_last_error()); return 4; }
  HIP(hipStreamSynchronize(st));

  float* hs = malloc(rows * 4 + 4);
  int32_t* hk = malloc(out_rows * 4 + 4);
  HIP(hipMemcpy(hs, scores, rows * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(hk, kept, out_rows * 4, hipMemcpyDeviceToHost));
  write_file(dir, "scores.bin", hs, rows * 4);
  write_file(dir, "kept.bin", hk, out_rows * 4);
  printf("scored %zu rows, kept %zu\n", rows, out_rows);
  return 0;
}
