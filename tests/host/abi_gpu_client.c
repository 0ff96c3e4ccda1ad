/*
 * A C client that runs the loss through the C ABI with no Python or torch in
 * the process: device buffers from hipMalloc, the default stream, explicit
 * copies. Usage: abi_gpu_client <dir>. <dir>/dims.txt holds
 *   B T U V HA HL H blank dtype(0 fp32, 1 bf16) mode(0 tiled, 1 untiled) tile_t tile_u
 * and the inputs are raw little-endian files: T_len, U_len, labels (int32),
 * hA, hL, WA, WL, bZ, WO, bO (fp32, or the upper 16 bits of fp32 for bf16).
 * It writes costs, dhA, dhL, dWA, dWL, dbZ, dWO, dbO (fp32) into <dir> and
 * prints "ok" (exit 0), or "FAIL <what>" (exit 1).
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rnnt.h"

static char dir[4096];

static void* read_file(const char* name, size_t bytes) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  size_t got = fread(p, 1, bytes, f);
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char* name, const void* p, size_t bytes) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 0;
  size_t put = fwrite(p, 1, bytes, f);
  fclose(f);
  return put == bytes;
}

/* host file -> new device buffer */
static void* upload(const char* name, size_t bytes) {
  void* h = read_file(name, bytes);
  void* d = NULL;
  if (!h || hipMalloc(&d, bytes ? bytes : 1) != hipSuccess || hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    free(h);
    return NULL;
  }
  free(h);
  return d;
}

#define CHECK(cond, what)            \
  do {                               \
    if (!(cond)) {                   \
      printf("FAIL %s\n", what);     \
      return 1;                      \
    }                                \
  } while (0)

int main(int argc, char** argv) {
  CHECK(argc == 2, "usage: abi_gpu_client <dir>");
  snprintf(dir, sizeof dir, "%s", argv[1]);
  rnnt_desc d;
  memset(&d, 0, sizeof d);
  {
    char path[4200];
    snprintf(path, sizeof path, "%s/dims.txt", dir);
    FILE* f = fopen(path, "r");
    CHECK(f, "dims.txt");
    int n = fscanf(f, "%d %d %d %d %d %d %d %d %d %d %d %d", &d.B, &d.T, &d.U, &d.V, &d.HA, &d.HL, &d.H, &d.blank,
                   &d.dtype, &d.mode, &d.tile_t, &d.tile_u);
    fclose(f);
    CHECK(n == 12, "dims.txt fields");
  }
  const size_t es = d.dtype == RNNT_BF16 ? 2 : 4;
  const size_t B = (size_t)d.B, T = (size_t)d.T, U1 = (size_t)d.U + 1;
  int32_t* T_len = (int32_t*)read_file("T_len", 4 * B);
  int32_t* U_len = (int32_t*)read_file("U_len", 4 * B);
  CHECK(T_len && U_len, "lengths");
  void* labels = upload("labels", 4 * B * U1);
  void* hA = upload("hA", es * B * T * d.HA);
  void* hL = upload("hL", es * B * U1 * d.HL);
  void* WA = upload("WA", es * (size_t)d.H * d.HA);
  void* WL = upload("WL", es * (size_t)d.H * d.HL);
  void* bZ = upload("bZ", es * (size_t)d.H);
  void* WO = upload("WO", es * (size_t)d.V * d.H);
  void* bO = upload("bO", es * (size_t)d.V);
  CHECK(labels && hA && hL && WA && WL && bZ && WO && bO, "inputs");

  size_t s_bytes = 0, w_bytes = 0;
  rnnt_status st = rnnt_loss_query(&d, T_len, U_len, &s_bytes, &w_bytes);
  CHECK(st == RNNT_OK, rnnt_last_error());
  void *saved = NULL, *ws = NULL;
  float *costs = NULL, *g[7] = {NULL};
  const size_t gn[7] = {B * T * d.HA, B * U1 * d.HL, (size_t)d.H * d.HA, (size_t)d.H * d.HL, (size_t)d.H,
                        (size_t)d.V * d.H, (size_t)d.V};
  const char* gname[7] = {"dhA", "dhL", "dWA", "dWL", "dbZ", "dWO", "dbO"};
  CHECK(hipMalloc(&saved, s_bytes ? s_bytes : 1) == hipSuccess, "saved");
  CHECK(hipMalloc(&ws, w_bytes ? w_bytes : 1) == hipSuccess, "workspace");
  CHECK(hipMalloc((void**)&costs, 4 * B) == hipSuccess, "costs");
  for (int k = 0; k < 7; ++k) CHECK(hipMalloc((void**)&g[k], 4 * gn[k]) == hipSuccess, "gradients");

  st = rnnt_loss_fwd(&d, hA, hL, (const int32_t*)labels, T_len, U_len, WA, WL, bZ, WO, bO, costs, saved, s_bytes,
                     ws, w_bytes, NULL);
  CHECK(st == RNNT_OK, rnnt_last_error());
  st = rnnt_loss_bwd(&d, hA, hL, (const int32_t*)labels, T_len, U_len, WA, WL, bZ, WO, bO, NULL, saved, s_bytes, ws,
                     w_bytes, g[0], g[1], g[2], g[3], g[4], g[5], g[6], NULL);
  CHECK(st == RNNT_OK, rnnt_last_error());
  CHECK(hipDeviceSynchronize() == hipSuccess, "synchronize");

  float* h = (float*)malloc(4 * (gn[5] > B ? (gn[5] > gn[0] ? gn[5] : gn[0]) : B));
  CHECK(h, "host buffer");
  CHECK(hipMemcpy(h, costs, 4 * B, hipMemcpyDeviceToHost) == hipSuccess && write_file("costs", h, 4 * B), "costs out");
  for (int k = 0; k < 7; ++k) {
    float* hk = (float*)malloc(4 * gn[k]);
    CHECK(hk && hipMemcpy(hk, g[k], 4 * gn[k], hipMemcpyDeviceToHost) == hipSuccess &&
              write_file(gname[k], hk, 4 * gn[k]),
          gname[k]);
    free(hk);
  }
  printf("ok\n");
  return 0;
}
