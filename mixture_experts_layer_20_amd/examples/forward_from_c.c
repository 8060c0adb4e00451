/*
 * forward_from_c.c -- the MoE layer driven from plain C through moe.h and
 * the HIP runtime's C API, with no other library.
 *
 * run_forward_case(in, out) reads a layer from the file `in`, runs
 * moe_forward on it and writes the outputs to the file `out`:
 *   in:  int64 T, d, E, k, F; float64 capacity_factor; then float32 x [T,d],
 *        w_router [d,E], w_in [E,F,d], b_in [E,F], w_out [E,d,F], b_out [E,d]
 *        (a float32 GELU layer, softmax scores, default gate renormalisation)
 *   out: int32 idx [T,k], float32 gates [T,k], int32 slot [T,k],
 *        uint8 dropped [T,k], int32 counts [E], float32 losses [2],
 *        int32 stats [4], float32 y [T,d]
 * Returns 0, or a negative step number with a message on stderr.
 * Built as a shared object (for the tests) and as a program whose main()
 * takes the two file names.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n ? 0 : -1; }

static void* to_device(const void* host, size_t n) {
  void* d = NULL;
  if (hipMalloc(&d, n > 0 ? n : 1) != hipSuccess) return NULL;
  if (n > 0 && hipMemcpy(d, host, n, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int run_forward_case(const char* in_path, const char* out_path) {
  FILE* f = fopen(in_path, "rb");
  if (!f) return -1;
  int64_t hdr[5];
  double cf;
  if (read_all(f, hdr, sizeof hdr) || read_all(f, &cf, sizeof cf)) return -2;
  const int64_t T = hdr[0], d = hdr[1], E = hdr[2], k = hdr[3], F = hdr[4];
  const size_t sz[6] = {(size_t)(T * d), (size_t)(d * E), (size_t)(E * F * d), (size_t)(E * F), (size_t)(E * d * F),
                        (size_t)(E * d)};
  float* host[6];
  void* dev[6];
  for (int i = 0; i < 6; ++i) {
    host[i] = (float*)malloc(sz[i] * sizeof(float) + 1);
    if (!host[i] || read_all(f, host[i], sz[i] * sizeof(float))) return -3;
    dev[i] = to_device(host[i], sz[i] * sizeof(float));
    if (!dev[i]) return -4;
  }
  fclose(f);

  moe_config cfg;
  memset(&cfg, 0, sizeof cfg);
  cfg.T = T;
  cfg.d = (int32_t)d;
  cfg.E = (int32_t)E;
  cfg.k = (int32_t)k;
  cfg.d_ff = (int32_t)F;
  cfg.capacity_factor = cf;
  cfg.renormalize = -1;
  cfg.score = MOE_SOFTMAX;
  cfg.act = MOE_GELU;
  cfg.dtype = MOE_F32;
  cfg.priority = MOE_RANK_MAJOR;
  int64_t C = 0;
  if (moe_validate(&cfg, &C) != MOE_OK) {
    fprintf(stderr, "moe_validate: %s\n", moe_last_error());
    return -5;
  }
  void* ws = NULL;
  if (hipMalloc(&ws, moe_workspace_bytes(&cfg)) != hipSuccess) return -6;

  moe_weights w;
  memset(&w, 0, sizeof w);
  w.w_router = (const float*)dev[1];
  w.w_in = dev[2];
  w.b_in = dev[3];
  w.w_out = dev[4];
  w.b_out = dev[5];
  const size_t tk = (size_t)(T * k);
  const size_t out_sz[8] = {tk * 4, tk * 4, tk * 4, tk, (size_t)E * 4, 2 * 4, 4 * 4, (size_t)(T * d) * 4};
  void* o[8];
  for (int i = 0; i < 8; ++i)
    if (hipMalloc(&o[i], out_sz[i] > 0 ? out_sz[i] : 1) != hipSuccess) return -7;
  moe_outputs out;
  memset(&out, 0, sizeof out);
  out.idx = (int32_t*)o[0];
  out.gates = (float*)o[1];
  out.slot = (int32_t*)o[2];
  out.dropped = (uint8_t*)o[3];
  out.counts = (int32_t*)o[4];
  out.losses = (float*)o[5];
  out.stats = (int32_t*)o[6];
  out.y = o[7];
  hipStream_t s;
  if (hipStreamCreate(&s) != hipSuccess) return -8;
  if (moe_forward(&cfg, &w, dev[0], &out, ws, s) != MOE_OK) {
    fprintf(stderr, "moe_forward: %s\n", moe_last_error());
    return -9;
  }
  if (hipStreamSynchronize(s) != hipSuccess) return -10;

  FILE* g = fopen(out_path, "wb");
  if (!g) return -11;
  for (int i = 0; i < 8; ++i) {
    void* h = malloc(out_sz[i] + 1);
    if (!h || hipMemcpy(h, o[i], out_sz[i], hipMemcpyDeviceToHost) != hipSuccess) return -12;
    if (fwrite(h, 1, out_sz[i], g) != out_sz[i]) return -13;
    free(h);
  }
  fclose(g);
  for (int i = 0; i < 8; ++i) hipFree(o[i]);
  for (int i = 0; i < 6; ++i) {
    hipFree(dev[i]);
    free(host[i]);
  }
  hipFree(ws);
  hipStreamDestroy(s);
  return 0;
}

#ifdef MOE_EXAMPLE_MAIN
int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <layer file> <output file>\n", argv[0]);
    return 2;
  }
  const int r = run_forward_case(argv[1], argv[2]);
  if (r) fprintf(stderr, "failed at step %d\n", -r);
  return r ? 1 : 0;
}
#endif
