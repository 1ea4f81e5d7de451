/* Plain C99 client of the C ABI (include/rs.h): sizes a Mamba-2 layer and a
 * KDA layer and checks host-side rejections. No device call is made. Prints
 * one line per check and exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "rs.h"

static int check(int ok, const char* what) {
  printf("%s %s\n", ok ? "ok" : "FAIL", what);
  return ok ? 0 : 1;
}

int main(void) {
  rs_config c;
  rs_layer L;
  memset(&c, 0, sizeof c);
  c.kind = RS_MAMBA2;
  c.mode = RS_REPLAY;
  c.batch = 256;
  c.nheads = 128;
  c.headdim = 64;
  c.dstate = 128;
  c.ngroups = 8;
  c.ring = 16;
  c.in_dtype = RS_BF16;
  c.ckpt_dtype = RS_F32;
  if (check(rs_init(&c, &L) == RS_OK, "mamba2 layer")) return 1;
  if (check(L.ckpt_bytes == 256ull * 128 * 64 * 128 * 4, "mamba2 checkpoint bytes")) return 1;
  if (check(L.meta_bytes >= 256ull * sizeof(rs_meta), "meta bytes")) return 1;
  if (check(sizeof(rs_meta) == 32, "rs_meta is 32 bytes")) return 1;

  rs_config k = c;
  k.kind = RS_KDA;
  k.nheads = k.headdim = k.dstate = k.ngroups = 0;
  k.n_qk_heads = 16;
  k.n_v_heads = 32;
  k.head_k_dim = 128;
  k.head_v_dim = 128;
  k.max_draft = 4;
  rs_layer K;
  if (check(rs_init(&k, &K) == RS_OK, "kda layer with drafts")) return 1;
  if (check(K.ring_beta_off - K.ring_g_off >= 256ull * 32 * 16 * 128 * 4, "kda gate ring")) return 1;

  rs_config bad = c;
  bad.ring = 8;
  if (check(rs_init(&bad, &L) == RS_E_ARG, "ring other than 16 refused")) return 1;
  rs_buffers none;
  memset(&none, 0, sizeof none);
  if (check(rs_reset_slots(&K, &none, NULL, 0, NULL) == RS_E_ARG, "reset without meta refused")) return 1;
  if (check(rs_gated_norm(&K, 1, NULL, NULL, NULL, 1, 1e-5f, NULL, NULL) == RS_E_MODE,
            "gated norm refused for a KDA layer")) return 1;
  if (check(strlen(rs_status_string(RS_E_ALIGN)) > 0 && rs_version() >= 100, "status strings, version"))
    return 1;
  return 0;
}
