/* Host-side driver of the C ABI's argument checks, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer on the host pass.
 *
 * Every call below is rejected (or is an empty no-op) before any HIP call,
 * so the program runs without a GPU.  It covers each entry point's checks,
 * the workspace-size arithmetic over extreme shapes (where a signed overflow
 * would be reported by UBSan), the error-message formatting, and the timing
 * hooks' argument checks.  Prints "ok <n>" and exits 0 when every status
 * matches; the sanitizers abort on the first report.
 */
#include <limits.h>
#include <stdio.h>
#include <string.h>

#include "hsa_sparse.h"

static int n_checks, n_fail;

static void expect(int line, hsa_sparse_status_t got, hsa_sparse_status_t want) {
  n_checks++;
  if (got != want) {
    printf("line %d: status %d, expected %d (%s)\n", line, (int)got, (int)want, hsa_sparse_last_error());
    n_fail++;
    return;
  }
  if (want != HSA_SPARSE_OK) {
    const char* msg = hsa_sparse_last_error();
    if (!msg || !msg[0] || strlen(msg) > 511) {
      printf("line %d: bad error message\n", line);
      n_fail++;
    }
  }
}
#define EXPECT(call, want) expect(__LINE__, (call), (want))

#define FAKE_U16 ((const uint16_t*)0x1000)
#define FAKE_OUT16 ((uint16_t*)0x1000)
#define FAKE_I32 ((int32_t*)0x1000)
#define FAKE_F32 ((float*)0x1000)
#define FAKE_W ((const int8_t*)0x1000)
#define FAKE_WS ((void*)0x1000)
#define BIG_WS ((size_t)1 << 40)

static hsa_sparse_shape_t base(void) {
  hsa_sparse_shape_t s;
  s.batch = 2;
  s.seq_len = 4096;
  s.n_q = 16;
  s.d_index = 128;
  s.block = 64;
  s.n_landmarks = 1;
  s.top_m = 8;
  s.top_k = 256;
  s.n_heads_q = 16;
  s.n_heads_kv = 2;
  s.head_dim = 128;
  s.scale = 0.088388f;
  return s;
}

static hsa_sparse_status_t forward(const hsa_sparse_shape_t* s, const uint16_t* qI, size_t ws) {
  return hsa_forward(s, qI, FAKE_U16, NULL, 0, FAKE_OUT16, FAKE_U16, FAKE_U16, FAKE_U16, NULL, NULL, FAKE_F32,
                     NULL, FAKE_WS, ws, NULL);
}

/* hsa_forward_noalloc: shapes whose scratch exceeds the static array are
   rejected before anything else happens (no HIP call) */
static void noalloc_checks(void) {
  hsa_sparse_shape_t s = base();
  s.seq_len = 65536; s.n_q = 65536; s.block = 128; s.top_m = 64; s.top_k = 2048;
  s.n_heads_q = 16; s.n_heads_kv = 1;
  EXPECT(hsa_forward_noalloc(&s, FAKE_U16, FAKE_U16, NULL, 0, FAKE_OUT16, FAKE_U16, FAKE_U16, FAKE_U16, NULL, NULL,
                             FAKE_F32, NULL, NULL), HSA_SPARSE_WORKSPACE_TOO_SMALL);
  s = base(); s.top_m = 1;
  EXPECT(hsa_forward_noalloc(&s, FAKE_U16, FAKE_U16, NULL, 0, FAKE_OUT16, FAKE_U16, FAKE_U16, FAKE_U16, NULL, NULL,
                             FAKE_F32, NULL, NULL), HSA_SPARSE_INVALID_ARG);
  s = base();
  EXPECT(hsa_forward_noalloc(&s, FAKE_U16, FAKE_U16, NULL, -1, FAKE_OUT16, FAKE_U16, FAKE_U16, FAKE_U16, NULL, NULL,
                             FAKE_F32, NULL, NULL), HSA_SPARSE_INVALID_ARG);
  s = base(); s.batch = 0;
  EXPECT(hsa_forward_noalloc(&s, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL),
         HSA_SPARSE_OK);
}

static void shape_checks(void) {
  hsa_sparse_shape_t s;
  EXPECT(forward(NULL, FAKE_U16, BIG_WS), HSA_SPARSE_INVALID_ARG);
  s = base(); s.batch = -1;        EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_INVALID_ARG);
  s = base(); s.n_q = s.seq_len + 1; EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_INVALID_ARG);
  s = base(); s.top_m = 1;         EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_INVALID_ARG);
  s = base(); s.top_k = 0;         EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_INVALID_ARG);
  s = base(); s.d_index = 96;      EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.block = 48;        EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.block = INT_MIN;   EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.n_landmarks = 3;   EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.n_landmarks = 4;   EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_INVALID_ARG); /* no W */
  s = base(); s.head_dim = 64;     EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.n_heads_kv = 3;    EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_INVALID_ARG);
  s = base(); s.n_heads_kv = 0;    EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_INVALID_ARG);
  s = base(); s.n_heads_q = 64; s.n_heads_kv = 2; EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.scale = 0.0f / 0.0f; EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_INVALID_ARG);
  s = base(); s.seq_len = INT_MAX; s.n_q = 1; EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.top_m = INT_MAX; s.top_k = 1; EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.batch = 1 << 20; s.n_q = 1 << 10; s.seq_len = 1 << 10; /* 2^34 (query, head) rows */
  EXPECT(forward(&s, FAKE_U16, BIG_WS), HSA_SPARSE_UNSUPPORTED);
  s = base(); EXPECT(forward(&s, NULL, BIG_WS), HSA_SPARSE_INVALID_ARG);
  s = base(); EXPECT(forward(&s, FAKE_U16, 1), HSA_SPARSE_WORKSPACE_TOO_SMALL);
  s = base(); s.batch = 0; EXPECT(forward(&s, NULL, 0), HSA_SPARSE_OK);
  s = base(); s.n_q = 0;   EXPECT(forward(&s, NULL, 0), HSA_SPARSE_OK);
}

static void stage_checks(void) {
  hsa_sparse_shape_t s = base();
  EXPECT(hsa_block_summary(NULL, FAKE_U16, NULL, 0, FAKE_OUT16, NULL), HSA_SPARSE_INVALID_ARG);
  EXPECT(hsa_block_summary(&s, FAKE_U16, NULL, -1, FAKE_OUT16, NULL), HSA_SPARSE_INVALID_ARG);
  EXPECT(hsa_block_summary(&s, NULL, NULL, 0, FAKE_OUT16, NULL), HSA_SPARSE_INVALID_ARG);
  EXPECT(hsa_block_summary(&s, FAKE_U16, NULL, INT_MAX, FAKE_OUT16, NULL), HSA_SPARSE_OK); /* past the end */

  EXPECT(hsa_block_topm(&s, NULL, FAKE_U16, FAKE_I32, FAKE_WS, BIG_WS, NULL), HSA_SPARSE_INVALID_ARG);
  EXPECT(hsa_block_topm(&s, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_WS, 0, NULL), HSA_SPARSE_WORKSPACE_TOO_SMALL);
  EXPECT(hsa_block_score_max(&s, NULL, FAKE_U16, FAKE_F32, FAKE_WS, BIG_WS, NULL), HSA_SPARSE_INVALID_ARG);
  {
    hsa_sparse_shape_t c = s;  /* few queries, many summary tiles: per-chunk maxima in the workspace */
    c.seq_len = 1 << 20; c.n_q = 64; c.block = 64;
    EXPECT(hsa_block_score_max(&c, FAKE_U16, FAKE_U16, FAKE_F32, FAKE_WS, 0, NULL), HSA_SPARSE_WORKSPACE_TOO_SMALL);
  }
  EXPECT(hsa_token_topk(&s, FAKE_U16, FAKE_U16, NULL, FAKE_I32, FAKE_WS, BIG_WS, NULL), HSA_SPARSE_INVALID_ARG);
  EXPECT(hsa_sparse_attn(&s, FAKE_U16, FAKE_U16, FAKE_U16, FAKE_I32, NULL, NULL, FAKE_WS, BIG_WS, NULL),
         HSA_SPARSE_INVALID_ARG);
  EXPECT(hsa_sparse_attn(&s, FAKE_U16, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_F32, NULL, FAKE_WS, 0, NULL),
         HSA_SPARSE_WORKSPACE_TOO_SMALL);

  s = base(); s.n_q = 1;
  EXPECT(hsa_decode_step(&s, NULL, NULL, FAKE_U16, NULL, FAKE_OUT16, FAKE_U16, FAKE_U16, FAKE_U16, NULL, NULL,
                         FAKE_F32, NULL, FAKE_WS, BIG_WS, NULL), HSA_SPARSE_INVALID_ARG);
  s = base();
  EXPECT(hsa_decode_step(&s, FAKE_I32, FAKE_U16, FAKE_U16, NULL, FAKE_OUT16, FAKE_U16, FAKE_U16, FAKE_U16, NULL,
                         NULL, FAKE_F32, NULL, FAKE_WS, BIG_WS, NULL), HSA_SPARSE_INVALID_ARG); /* n_q != 1 */

  s = base(); s.d_index = 32;
  EXPECT(hsa_flat_topk(&s, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_WS, BIG_WS, NULL), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.seq_len = INT_MAX; s.n_q = 1;
  EXPECT(hsa_flat_topk(&s, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_WS, BIG_WS, NULL), HSA_SPARSE_UNSUPPORTED);
  s = base();
  EXPECT(hsa_flat_topk(&s, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_WS, 0, NULL), HSA_SPARSE_WORKSPACE_TOO_SMALL);

  EXPECT(hsa_super_summary(&s, 3, FAKE_U16, 0, FAKE_OUT16, NULL), HSA_SPARSE_UNSUPPORTED);
  EXPECT(hsa_super_summary(&s, 16, FAKE_U16, -1, FAKE_OUT16, NULL), HSA_SPARSE_INVALID_ARG);
  EXPECT(hsa_block_topm_3level(&s, 16, 1, FAKE_U16, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_I32, FAKE_WS, BIG_WS, NULL),
         HSA_SPARSE_INVALID_ARG);
  EXPECT(hsa_block_topm_3level(&s, 16, 4, FAKE_U16, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_I32, FAKE_WS, 0, NULL),
         HSA_SPARSE_WORKSPACE_TOO_SMALL);
  EXPECT(hsa_block_topm_3level(&s, 4096, INT_MAX, FAKE_U16, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_I32, FAKE_WS,
                               BIG_WS, NULL), HSA_SPARSE_UNSUPPORTED);
  EXPECT(hsa_block_topm_3level(&s, INT_MIN, 4, FAKE_U16, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_I32, FAKE_WS,
                               BIG_WS, NULL), HSA_SPARSE_UNSUPPORTED);
  EXPECT(hsa_super_summary(&s, 1 << 30, FAKE_U16, 0, FAKE_OUT16, NULL), HSA_SPARSE_UNSUPPORTED);
  EXPECT(hsa_forward_3level(&s, FAKE_I32, 16, 4, FAKE_U16, FAKE_U16, NULL, 0, FAKE_OUT16, FAKE_OUT16, FAKE_U16,
                            FAKE_U16, FAKE_U16, NULL, NULL, NULL, FAKE_F32, NULL, FAKE_WS, BIG_WS, NULL),
         HSA_SPARSE_INVALID_ARG); /* lengths with n_q != 1 */

  s = base(); s.head_dim = 96;
  EXPECT(hsa_head_landmarks(&s, FAKE_U16, NULL, 0, FAKE_OUT16, NULL), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.n_heads_kv = 32; s.n_heads_q = 32;
  EXPECT(hsa_head_topm(&s, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_WS, BIG_WS, NULL), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.top_m = 4096; s.block = 64;
  EXPECT(hsa_head_topm(&s, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_WS, BIG_WS, NULL), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.top_m = INT_MAX; s.block = 128;
  EXPECT(hsa_head_topm(&s, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_WS, BIG_WS, NULL), HSA_SPARSE_UNSUPPORTED);
  s = base(); s.batch = 1 << 20; s.n_q = 1 << 10; s.seq_len = 1 << 12;
  EXPECT(hsa_head_topm(&s, FAKE_U16, FAKE_U16, FAKE_I32, FAKE_WS, BIG_WS, NULL), HSA_SPARSE_UNSUPPORTED);
  s = base();
  EXPECT(hsa_forward_heads(&s, NULL, NULL, 0, FAKE_U16, FAKE_U16, FAKE_U16, FAKE_OUT16, NULL, FAKE_F32, NULL,
                           FAKE_WS, 0, NULL), HSA_SPARSE_WORKSPACE_TOO_SMALL);
  s = base(); s.batch = 0;
  EXPECT(hsa_forward_heads(&s, NULL, NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL),
         HSA_SPARSE_OK);
}

static void workspace_sizes(void) {
  static const int32_t big[] = {0, 1, 7, 4096, 65535, 65536, 1 << 20, 1 << 24, INT_MAX};
  const int nbig = (int)(sizeof(big) / sizeof(big[0]));
  size_t sink = 0;
  for (int op = -1; op <= 9; op++)
    for (int a = 0; a < nbig; a++)
      for (int c = 0; c < nbig; c++) {
        hsa_sparse_shape_t s = base();
        s.batch = big[a];
        s.seq_len = big[c];
        s.n_q = big[c] < 2 ? big[c] : big[c] / 2;
        sink += hsa_sparse_workspace_size(&s, op);
        s.n_q = 1;
        s.top_m = big[a] < 2 ? 2 : big[a];
        s.top_k = big[c] < 1 ? 1 : big[c];
        sink += hsa_sparse_workspace_size(&s, op);
        s = base();
        s.n_heads_q = 16;
        s.n_heads_kv = 1;
        s.seq_len = big[c];
        s.n_q = big[c];
        s.batch = big[a];
        s.block = 128;
        sink += hsa_sparse_workspace_size(&s, op);
      }
  hsa_sparse_shape_t s = base();
  if (hsa_sparse_workspace_size(&s, HSA_SPARSE_OP_FORWARD) == 0) {
    printf("forward workspace of a valid shape is 0\n");
    n_fail++;
  }
  if (hsa_sparse_workspace_size(NULL, HSA_SPARSE_OP_FORWARD) != 0) {
    printf("workspace of a NULL shape is not 0\n");
    n_fail++;
  }
  printf("workspace sweep checksum %zu\n", sink);
}

static void misc(void) {
  for (int st = -2; st <= 8; st++) {
    const char* m = hsa_sparse_strerror((hsa_sparse_status_t)st);
    n_checks++;
    if (!m || !m[0]) {
      printf("strerror(%d) empty\n", st);
      n_fail++;
    }
  }
  EXPECT(hsa_sparse_set_kernel_events(NULL, NULL, 5), HSA_SPARSE_INVALID_ARG);
  EXPECT(hsa_sparse_set_kernel_events(NULL, NULL, 1000), HSA_SPARSE_INVALID_ARG);
  EXPECT(hsa_sparse_set_kernel_events(NULL, NULL, 0), HSA_SPARSE_OK);
  EXPECT(hsa_sparse_set_stage_events(NULL, 5), HSA_SPARSE_INVALID_ARG);
  EXPECT(hsa_sparse_set_stage_events(NULL, 0), HSA_SPARSE_OK);
  n_checks++;
  if (!hsa_sparse_last_kernels()) {
    printf("last_kernels is NULL\n");
    n_fail++;
  }
}

int main(void) {
  shape_checks();
  stage_checks();
  workspace_sizes();
  noalloc_checks();
  misc();
  if (n_fail) {
    printf("%d of %d checks failed\n", n_fail, n_checks);
    return 1;
  }
  printf("ok %d\n", n_checks);
  return 0;
}
