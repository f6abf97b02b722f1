/* A plain C99 caller of the library's C ABI, built and run by
   tests/test_abi.py on the host: the headers compile as strict C, the
   library links from C, and the host-only entry points (planner, workspace
   size, tree check, error strings, argument validation) behave as the
   header states without a GPU. Exits 0 on success, else the failing check. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mla_verify.h"
#include "mla_verify_probe.h"

#define CHECK(id, cond)                                  \
  do {                                                   \
    if (!(cond)) {                                       \
      fprintf(stderr, "check %d failed: %s\n", id, #cond); \
      return id;                                         \
    }                                                    \
  } while (0)

int main(void) {
  mlav_plan p;
  mlav_options o;
  memset(&o, 0, sizeof o);
  /* the headline shape: 9 tokens x 64 heads = 9 row blocks over 16393 keys */
  CHECK(1, mla_verify_plan(9, 64, 1, 16393, 16393, 256, &o, &p) == MLAV_OK);
  CHECK(2, p.tile == 32 && p.chunk % p.tile == 0 && p.nsplit == (int32_t)((16393 + p.chunk - 1) / p.chunk));
  CHECK(3, p.grid >= 9 * p.nsplit && p.combine == 1);
  CHECK(4, mla_verify_workspace_size(9, 64, 1, 16393, 16393, 256, NULL) > 0);
  /* one split: no workspace, no combine */
  o.nsplit = 1;
  CHECK(5, mla_verify_plan(9, 64, 1, 300, 300, 256, &o, &p) == MLAV_OK && p.nsplit == 1 && p.combine == 0);
  CHECK(6, mla_verify_workspace_size(9, 64, 1, 300, 300, 256, &o) == 0);
  o.nsplit = 0;
  /* out-of-range sizes and options */
  CHECK(7, mla_verify_plan(65, 64, 1, 100, 100, 256, &o, &p) == MLAV_ERR_SHAPE);
  CHECK(8, mla_verify_plan(9, 64, 1, 100, 100, 0, &o, &p) == MLAV_ERR_ARG);
  CHECK(9, mla_verify_plan(9, 64, 1, 100, 100, 256, &o, NULL) == MLAV_ERR_NULL);
  o.pv_mode = 3;
  CHECK(10, mla_verify_plan(9, 64, 1, 100, 100, 256, &o, &p) == MLAV_ERR_ARG);
  o.pv_mode = 0;
  /* host tree check */
  {
    const int32_t good[5] = {-1, 0, 0, 1, -1};
    const int32_t bad[3] = {-1, 2, 0};
    CHECK(11, mla_verify_check_tree(good, 5) == MLAV_OK);
    CHECK(12, mla_verify_check_tree(bad, 3) == MLAV_ERR_TREE);
    CHECK(13, mla_verify_check_tree(NULL, 3) == MLAV_ERR_NULL);
  }
  /* validation before any device use: a NULL tensor, a misaligned one */
  {
    static uint16_t buf[64] __attribute__((aligned(16)));
    static float fbuf[64] __attribute__((aligned(16)));
    const int32_t par[1] = {-1};
    CHECK(14, mla_verify(buf, buf, buf, NULL, par, 0, 0.07f, fbuf, fbuf, 1, 1, NULL, 0, NULL) == MLAV_ERR_NULL);
    CHECK(15, mla_verify(buf + 1, buf, buf, buf, par, 0, 0.07f, fbuf, fbuf, 1, 1, NULL, 0, NULL) == MLAV_ERR_ALIGN);
    CHECK(16, mla_verify(buf, buf, buf, buf, par, 0, -1.0f, fbuf, fbuf, 1, 1, NULL, 0, NULL) == MLAV_ERR_ARG);
  }
  CHECK(17, strcmp(mla_verify_strerror(MLAV_OK), "ok") == 0);
  CHECK(18, mlav_probe_mfma_per_wave() == 16);
  printf("c abi ok\n");
  return 0;
}
