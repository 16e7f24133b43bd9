/* The C ABI used from plain C99: include/pa.h compiles as C, the library links, and the
 * calls that need no GPU behave as documented (status strings, workspace sizing, argument
 * checks that return before any device work, and a host block-manager scenario whose
 * expected slots, copy-on-write pairs and free-list order are worked by hand from the
 * append / share / fork / free rules). Exit status 0 = every check held. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pa.h"

static int failures = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main(void) {
  /* a 16-byte aligned stand-in address that no check below dereferences */
  void* fake = (void*)(uintptr_t)0x7F0000000000ull;
  const int32_t* ifake = (const int32_t*)fake;
  int32_t code;
  int64_t slot = 0;
  int32_t src = 0, dst = 0, table[8], free_list[8], n;
  pa_block_manager* m;

  CHECK(pa_version() >= 100);
  for (code = 0; code <= 9; ++code) CHECK(pa_status_string(code) != NULL);
  CHECK(strncmp(pa_status_string(PA_OK), "PA_OK", 5) == 0);
  CHECK(strstr(pa_status_string(12345), "unknown") != NULL);

  /* workspace: grows with the partitions a sequence can have */
  CHECK(pa_decode_splitkv_workspace_bytes(8, 64, 128, 131072, 512) >
        pa_decode_splitkv_workspace_bytes(8, 64, 128, 4096, 512));
  CHECK(pa_decode_splitkv_workspace_bytes(8, 64, 128, 0, 512) == 0);   /* documented: 0 for non-positive sizes */

  /* argument checks (no launch happens on any of these) */
  CHECK(pa_decode(NULL, fake, fake, fake, 16 * 4 * 64, 32, ifake, 3, ifake, 4, 4, 4, 64, 16, 0.125f,
                  PA_DTYPE_F32, NULL) == PA_ERR_NULL_PTR);
  CHECK(pa_decode(fake, fake, fake, fake, 16 * 4 * 64, 32, ifake, 3, ifake, 4, 4, 4, 64, 16, 0.125f, 9,
                  NULL) == PA_ERR_DTYPE);
  CHECK(pa_decode(fake, fake, fake, fake, 16 * 4 * 64, 32, ifake, 3, ifake, 4, 4, 4, 64, 32, 0.125f,
                  PA_DTYPE_F32, NULL) == PA_ERR_UNSUPPORTED);
  CHECK(pa_decode(fake, fake, fake, fake, 16 * 4 * 64, 32, ifake, 3, ifake, 0, 4, 4, 64, 16, 0.125f,
                  PA_DTYPE_F32, NULL) == PA_OK);
  CHECK(pa_reshape_and_cache(fake, fake, 4 * 64, fake, fake, 16 * 4 * 64, 32, NULL, 5, 4, 64, 16,
                             PA_DTYPE_BF16, NULL) == PA_ERR_NULL_PTR);
  CHECK(pa_reshape_and_cache(fake, fake, 4 * 64, fake, fake, 16 * 4 * 64, 32, NULL, 0, 4, 64, 16,
                             PA_DTYPE_BF16, NULL) == PA_OK);

  /* host block manager: 8 blocks of 16 tokens, free list 0..7 */
  m = pa_bm_create(8, 16, NULL);
  CHECK(m != NULL);
  CHECK(pa_bm_allocate(m, 1, 20) == PA_OK);                 /* blocks 0, 1 */
  CHECK(pa_bm_num_free(m) == 6);
  n = pa_bm_block_table(m, 1, table, 8);
  CHECK(n == 2 && table[0] == 0 && table[1] == 1);
  CHECK(pa_bm_append(m, 1, &slot, &src, &dst) == PA_OK);   /* position 20: block 1, row 4 */
  CHECK(slot == 20 && src == -1 && dst == -1);
  CHECK(pa_bm_share_prefix(m, 1, 2, 16) == PA_OK);          /* request 2 shares block 0 */
  CHECK(pa_bm_ref_count(m, 0) == 2 && pa_bm_seq_len(m, 2) == 16);
  CHECK(pa_bm_append(m, 2, &slot, &src, &dst) == PA_OK);   /* block 0 is full: new block 2 */
  CHECK(slot == 32 && src == -1 && dst == -1 && pa_bm_num_free(m) == 5);
  CHECK(pa_bm_fork(m, 1, 3) == PA_OK);                      /* request 3 shares blocks 0, 1 */
  CHECK(pa_bm_ref_count(m, 0) == 3 && pa_bm_ref_count(m, 1) == 2);
  CHECK(pa_bm_append(m, 3, &slot, &src, &dst) == PA_OK);   /* shared, partly filled block 1: copy to 3 */
  CHECK(src == 1 && dst == 3 && slot == 3 * 16 + 5);
  CHECK(pa_bm_ref_count(m, 1) == 1 && pa_bm_num_free(m) == 4);
  CHECK(pa_bm_allocate(m, 4, 200) == PA_ERR_NO_BLOCKS && pa_bm_num_free(m) == 4);
  CHECK(pa_bm_free(m, 99) == PA_ERR_SEQUENCE);
  CHECK(pa_bm_free(m, 1) == PA_OK);                         /* block 1 reaches zero */
  CHECK(pa_bm_free(m, 2) == PA_OK);                         /* block 2 */
  CHECK(pa_bm_free(m, 3) == PA_OK);                         /* blocks 0, 3 */
  CHECK(pa_bm_num_free(m) == 8);
  n = pa_bm_free_list(m, free_list, 8);
  CHECK(n == 8);
  if (n == 8) {
    const int32_t want[8] = {4, 5, 6, 7, 1, 2, 0, 3};        /* head out, tail in, in table order */
    CHECK(memcmp(free_list, want, sizeof(want)) == 0);
  }
  pa_bm_destroy(m);

  if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
  else printf("abi_from_c: all checks held\n");
  return failures ? 1 : 0;
}
