/* pa_decode driven from C with the HIP runtime only: reads the problem from raw files, runs
 * the decode through the library's C ABI and writes the output.  Used by
 * tests/test_gpu_c_program.py, which makes the inputs and checks the output against the oracle.
 *
 * usage: decode_from_c DIR S HQ HKV D NB MB MAXLEN SCALE
 *   DIR/q.bin        bf16 [S][HQ][D]          DIR/k.bin, DIR/v.bin  bf16 [NB][HKV][16][D]
 *   DIR/tables.bin   int32 [S][MB]            DIR/lens.bin          int32 [S]
 *   writes DIR/out.bin  bf16 [S][HQ][D]
 * Exit status 0 on success; otherwise a message on stderr. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>
#include "pagedattn.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  if (p && fread(p, 1, bytes, f) != bytes) { free(p); p = NULL; }
  fclose(f);
  return p;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 16) != hipSuccess) return NULL;
  if (bytes && hipMemcpy(d, host, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int main(int argc, char** argv) {
  if (argc != 10) { fprintf(stderr, "usage: %s DIR S HQ HKV D NB MB MAXLEN SCALE\n", argv[0]); return 2; }
  const char* dir = argv[1];
  const int S = atoi(argv[2]), HQ = atoi(argv[3]), HKV = atoi(argv[4]), D = atoi(argv[5]);
  const int NB = atoi(argv[6]), MB = atoi(argv[7]), MAXLEN = atoi(argv[8]);
  const float scale = (float)atof(argv[9]);
  const size_t qb = (size_t)S * HQ * D * 2, kb = (size_t)NB * HKV * 16 * D * 2;
  const size_t tb = (size_t)S * MB * 4, lb = (size_t)S * 4;
  void *hq = read_file(dir, "q.bin", qb), *hk = read_file(dir, "k.bin", kb);
  void *hv = read_file(dir, "v.bin", kb), *ht = read_file(dir, "tables.bin", tb);
  void *hl = read_file(dir, "lens.bin", lb);
  if (!hq || !hk || !hv || !ht || !hl) { fprintf(stderr, "cannot read the inputs\n"); return 3; }
  void *dq = to_device(hq, qb), *dk = to_device(hk, kb), *dv = to_device(hv, kb);
  void *dt = to_device(ht, tb), *dl = to_device(hl, lb), *dout = NULL, *dws = NULL;
  const size_t ws = pa_decode_workspace_size(S, HQ, HKV, D, 16, MAXLEN);
  if (!dq || !dk || !dv || !dt || !dl || hipMalloc(&dout, qb) != hipSuccess ||
      hipMalloc(&dws, ws ? ws : 16) != hipSuccess) {
    fprintf(stderr, "device allocation or copy failed\n");
    return 4;
  }
  const pa_status st = pa_decode(dout, dq, dk, dv, (const int32_t*)dt, (const int32_t*)dl, S, HQ,
                                 HKV, D, 16, NB, MB, MAXLEN, scale, PA_DTYPE_BF16, dws, ws, NULL);
  if (st != PA_OK) { fprintf(stderr, "pa_decode: %s: %s\n", pa_status_string(st), pa_last_error()); return 5; }
  if (hipDeviceSynchronize() != hipSuccess) { fprintf(stderr, "synchronize failed\n"); return 6; }
  void* hout = malloc(qb);
  if (!hout || hipMemcpy(hout, dout, qb, hipMemcpyDeviceToHost) != hipSuccess) { fprintf(stderr, "copy back failed\n"); return 7; }
  char path[4096];
  snprintf(path, sizeof path, "%s/out.bin", dir);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(hout, 1, qb, f) != qb) { fprintf(stderr, "cannot write the output\n"); return 8; }
  fclose(f);
  printf("pa_decode from C: %d sequences, workspace %zu bytes\n", S, ws);
  return 0;
}
