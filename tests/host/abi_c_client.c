/*
 * A plain C99 client of the library's C ABI, host-only calls: compiled with
 * gcc -std=c99 -pedantic against include/rnnt.h and linked to the library,
 * it checks that the header is valid C on its own and that the host-only
 * entry points work from C (no GPU work is launched):
 *   - rnnt_loss_query for a tiled and an untiled bf16 descriptor (the
 *     untiled one keeps the scores and z, so it needs more `saved`);
 *   - rnnt_waves_for_budget at the tiled query's own total;
 *   - a refused descriptor (blank outside [0, V)) with its status string and
 *     last-error text.
 * Prints one line "ok ..." or "FAIL ..." and exits with 0 or 1.
 */
#include <stdio.h>
#include <string.h>

#include "rnnt.h"

static rnnt_desc base_desc(void) {
  rnnt_desc d;
  memset(&d, 0, sizeof d);
  d.B = 2;
  d.T = 50;
  d.U = 10;
  d.V = 300;
  d.HA = 64;
  d.HL = 64;
  d.H = 640;
  d.blank = 0;
  d.dtype = RNNT_BF16;
  d.mode = RNNT_TILED;
  d.tile_t = 32;
  d.tile_u = 8;
  d.tiles_per_wave = 0;
  return d;
}

int main(void) {
  const int32_t T_len[2] = {50, 20}, U_len[2] = {10, 3};
  size_t s_tiled = 0, w_tiled = 0, s_untiled = 0, w_untiled = 0;
  int32_t tpw = 0;
  rnnt_desc d = base_desc();
  rnnt_status st = rnnt_loss_query(&d, T_len, U_len, &s_tiled, &w_tiled);
  if (st != RNNT_OK) {
    printf("FAIL tiled query: %s: %s\n", rnnt_status_string(st), rnnt_last_error());
    return 1;
  }
  d.mode = RNNT_UNTILED;
  st = rnnt_loss_query(&d, T_len, U_len, &s_untiled, &w_untiled);
  if (st != RNNT_OK) {
    printf("FAIL untiled query: %s: %s\n", rnnt_status_string(st), rnnt_last_error());
    return 1;
  }
  if (s_untiled <= s_tiled) {
    printf("FAIL untiled saved %zu not above tiled %zu\n", s_untiled, s_tiled);
    return 1;
  }
  d = base_desc();
  st = rnnt_waves_for_budget(&d, T_len, U_len, s_tiled + w_tiled, &tpw);
  if (st != RNNT_OK || tpw < 1) {
    printf("FAIL waves_for_budget: %d %d\n", (int)st, (int)tpw);
    return 1;
  }
  d.blank = d.V;  /* outside [0, V) */
  st = rnnt_loss_query(&d, T_len, U_len, &s_tiled, &w_tiled);
  if (st != RNNT_E_INVALID || strlen(rnnt_last_error()) == 0 || strlen(rnnt_status_string(st)) == 0) {
    printf("FAIL refused descriptor: %d\n", (int)st);
    return 1;
  }
  printf("ok saved %zu / %zu, workspace %zu / %zu, tiles per wave %d\n", s_tiled, s_untiled, w_tiled, w_untiled,
         (int)tpw);
  return 0;
}
