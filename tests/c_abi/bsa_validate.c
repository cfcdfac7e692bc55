/*
 * Host-side argument validation of the C ABI (include/bsa.h), driven from
 * plain C99 without a GPU: every call below is rejected before any launch
 * (or is host-only), so no device memory is touched.  Built with the host
 * sanitizers (AddressSanitizer, UndefinedBehaviorSanitizer) over the
 * library's validation code, it checks that those paths read and write only
 * what they own.  Prints one line per failed check; exit status 0 when
 * every check holds.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "bsa.h"

static int failures = 0;

#define EXPECT(cond)                                                           \
  do {                                                                         \
    if (!(cond)) {                                                             \
      fprintf(stderr, "%s:%d: check failed: %s (last error: %s)\n", __FILE__, \
              __LINE__, #cond, bsa_last_error());                              \
      ++failures;                                                              \
    }                                                                          \
  } while (0)

static bsa_geometry geo(int32_t B, int32_t H, int32_t text_len, int32_t frames, int32_t lh, int32_t lw,
                        int32_t D, int32_t bq, int32_t bk, int64_t seq_alloc) {
  bsa_geometry g;
  memset(&g, 0, sizeof g);
  g.B = B;
  g.H = H;
  g.text_len = text_len;
  g.frames = frames;
  g.latent_h = lh;
  g.latent_w = lw;
  g.head_dim = D;
  g.q_block = bq;
  g.k_block = bk;
  g.seq_alloc = seq_alloc;
  return g;
}

static bsa_mask_params topk_params(double keep) {
  bsa_mask_params p;
  memset(&p, 0, sizeof p);
  p.mode = BSA_SELECT_TOPK;
  p.keep_ratio = keep;
  p.frame0_dense = 1;
  return p;
}

int main(void) {
  /* never dereferenced: every call below fails validation or is host-only */
  void* fake = (void*)(uintptr_t)0x1000;
  void* mis = (void*)(uintptr_t)0x1004;
  bsa_geometry small = geo(1, 12, 0, 5, 30, 52, 128, 64, 64, 7808);
  bsa_mask_params p = topk_params(0.25);
  bsa_derived d;

  /* derived geometry of the five video workloads */
  const bsa_geometry work[5] = {
      geo(1, 2, 32, 3, 8, 8, 64, 32, 32, 224),
      small,
      geo(1, 12, 0, 21, 30, 52, 128, 64, 64, 32768),
      geo(1, 12, 0, 21, 30, 52, 128, 64, 16, 32768),
      geo(1, 24, 256, 33, 45, 80, 128, 64, 64, 119104),
  };
  const int64_t S[5] = {224, 7800, 32760, 32760, 119056};
  const int32_t nkb[5] = {7, 122, 512, 2048, 1861};
  for (int i = 0; i < 5; ++i) {
    EXPECT(bsa_derive(&work[i], &p, &d) == BSA_OK);
    EXPECT(d.S == S[i] && d.nkb == nkb[i]);
    EXPECT(d.topk == (int32_t)ceil(0.25 * nkb[i]));
  }
  EXPECT(bsa_derive(&work[4], NULL, &d) == BSA_OK && d.frame0_first == 4 && d.frame0_last == 60 &&
         d.text_last == 3);
  EXPECT(bsa_derive(NULL, &p, &d) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_derive(&small, &p, NULL) == BSA_ERR_INVALID_ARGUMENT);
  p.keep_ratio = 0.0;
  EXPECT(bsa_derive(&small, &p, &d) == BSA_ERR_INVALID_ARGUMENT);
  p.keep_ratio = 0.25;
  p.mode = 9;
  EXPECT(bsa_derive(&small, &p, &d) == BSA_ERR_INVALID_ARGUMENT);
  p.mode = BSA_SELECT_TOPK;

  /* geometry checks */
  bsa_geometry bad = small;
  bad.B = 0;
  EXPECT(bsa_derive(&bad, NULL, &d) == BSA_ERR_INVALID_ARGUMENT);
  bad = small;
  bad.head_dim = 96;
  EXPECT(bsa_derive(&bad, NULL, &d) == BSA_ERR_UNSUPPORTED);
  bad = small;
  bad.seq_alloc = 7800; /* shorter than nqb * q_block */
  EXPECT(bsa_derive(&bad, NULL, &d) == BSA_ERR_INVALID_ARGUMENT && strstr(bsa_last_error(), "seq_alloc"));
  bsa_geometry huge = geo(1, 4096, 1 << 26, 0, 0, 0, 128, 64, 64, (int64_t)1 << 26);
  EXPECT(bsa_pool_blocks(fake, 0, &huge, 64, fake, NULL) == BSA_ERR_UNSUPPORTED &&
         strstr(bsa_last_error(), "block rows"));

  /* pooling */
  EXPECT(bsa_pool_blocks(NULL, 0, &small, 64, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_pool_blocks(mis, 0, &small, 64, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_pool_blocks(fake, 7, &small, 64, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_pool_blocks(fake, 0, &small, 48, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);

  EXPECT(bsa_pool_qk(fake, fake, 0, &small, fake, NULL, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_pool_qk(fake, mis, 0, &small, fake, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_pool_qk(fake, fake, 2, &small, fake, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_pool_qk(fake, fake, 0, NULL, fake, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_pool_qk(fake, fake, 0, &huge, fake, fake, NULL) == BSA_ERR_UNSUPPORTED);

  /* mask */
  EXPECT(bsa_build_mask(NULL, fake, &small, &p, NULL, fake, fake, NULL, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_build_mask(fake, fake, &small, NULL, NULL, fake, fake, NULL, NULL) == BSA_ERR_INVALID_ARGUMENT);
  bsa_mask_params ps = p;
  ps.mode = BSA_SELECT_SAMPLE;
  EXPECT(bsa_build_mask(fake, fake, &small, &ps, NULL, fake, fake, NULL, NULL) ==
         BSA_ERR_INVALID_ARGUMENT); /* sampling needs log_w */

  /* forward */
  bad = small;
  bad.q_block = 128;
  bad.seq_alloc = 7808;
  EXPECT(bsa_forward(fake, fake, fake, 0, &bad, fake, fake, NULL, 0.0f, fake, NULL, NULL) == BSA_ERR_UNSUPPORTED);
  EXPECT(bsa_forward(fake, fake, fake, 0, &small, fake, fake, NULL, -1.0f, fake, NULL, NULL) ==
         BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_forward(fake, fake, fake, 0, &small, fake, fake, NULL, NAN, fake, NULL, NULL) ==
         BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_forward(fake, NULL, fake, 0, &small, fake, fake, NULL, 0.0f, fake, NULL, NULL) ==
         BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_forward(fake, fake, fake, 0, &small, fake, fake, mis, 0.0f, fake, NULL, NULL) ==
         BSA_ERR_INVALID_ARGUMENT);
  bsa_forward_options opt;
  memset(&opt, 0, sizeof opt);
  opt.launch_order = 7;
  EXPECT(bsa_forward_ex(fake, fake, fake, 0, &small, fake, fake, NULL, 0.0f, fake, NULL, &opt, NULL) ==
         BSA_ERR_INVALID_ARGUMENT);
  opt.launch_order = BSA_ORDER_FRAME_POSITION;

  /* the key split and its workspace */
  int64_t need = 0;
  EXPECT(bsa_forward_split_workspace_bytes(&small, 2, &need) == BSA_OK);
  EXPECT(need == (int64_t)12 * 25 * 2 * (64 * 128 + 2 * 64) * 4);
  EXPECT(bsa_forward_split_workspace_bytes(&small, 0, &need) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_forward_split_workspace_bytes(&small, 17, &need) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_forward_split_workspace_bytes(&small, 2, NULL) == BSA_ERR_INVALID_ARGUMENT);
  bsa_forward_split_workspace_bytes(&small, 2, &need);
  EXPECT(bsa_forward_split(fake, fake, fake, 0, &small, fake, fake, NULL, 0.0f, fake, NULL, &opt, 2, NULL, need,
                           NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_forward_split(fake, fake, fake, 0, &small, fake, fake, NULL, 0.0f, fake, NULL, &opt, 2, mis, need,
                           NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_forward_split(fake, fake, fake, 0, &small, fake, fake, NULL, 0.0f, fake, NULL, &opt, 2, fake,
                           need - 1, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_forward_split_static(fake, fake, fake, 0, &small, fake, fake, NULL, 0.0f, fake, NULL, &opt, 0,
                                  NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_forward_split_static(NULL, fake, fake, 0, &small, fake, fake, NULL, 0.0f, fake, NULL, &opt, 2,
                                  NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_forward_split_workspace_bytes(&work[4], 16, &need) == BSA_OK && need > BSA_SPLIT_STATIC_MAX_BYTES);
  EXPECT(bsa_forward_split_static(fake, fake, fake, 0, &work[4], fake, fake, NULL, 0.0f, fake, NULL, &opt, 16,
                                  NULL) == BSA_ERR_UNSUPPORTED &&
         strstr(bsa_last_error(), "scratch"));

  /* top-p over competition domains */
  int64_t nb = 0;
  EXPECT(bsa_top_p_workspace_bytes(&small, &nb) == BSA_OK && nb > 0);
  EXPECT(bsa_top_p_workspace_bytes(&small, NULL) == BSA_ERR_INVALID_ARGUMENT);
  bsa_topp_params tp;
  memset(&tp, 0, sizeof tp);
  tp.domain = BSA_DOMAIN_EG;
  tp.top_p = 0.9;
  tp.entropy_eps = 1e-12f;
  bsa_topp_params t2 = tp;
  t2.domain = 5;
  EXPECT(bsa_select_top_p(fake, NULL, &small, &t2, NULL, fake, nb, fake, fake, fake, NULL) ==
         BSA_ERR_INVALID_ARGUMENT);
  t2 = tp;
  t2.top_p = 1.5;
  EXPECT(bsa_select_top_p(fake, NULL, &small, &t2, NULL, fake, nb, fake, fake, fake, NULL) ==
         BSA_ERR_INVALID_ARGUMENT);
  t2 = tp;
  t2.value_aware = 1; /* needs v_pooled */
  EXPECT(bsa_select_top_p(fake, NULL, &small, &t2, NULL, fake, nb, fake, fake, fake, NULL) ==
         BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_select_top_p(fake, NULL, &small, &tp, NULL, fake, nb - 8, fake, fake, fake, NULL) ==
         BSA_ERR_INVALID_ARGUMENT &&
         strstr(bsa_last_error(), "workspace"));
  bsa_geometry wide_k = work[4];
  wide_k.k_block = 32; /* nkb 3721 > 2048 */
  EXPECT(bsa_top_p_workspace_bytes(&wide_k, &nb) == BSA_OK);
  EXPECT(bsa_select_top_p(fake, NULL, &wide_k, &tp, NULL, fake, nb, fake, fake, fake, NULL) ==
         BSA_ERR_UNSUPPORTED);

  /* clustering selector */
  EXPECT(bsa_cluster_importance(fake, 0, fake, &small, 0, 3, 0, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_cluster_importance(fake, 0, fake, &small, 4, 17, 0, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_cluster_importance(NULL, 0, fake, &small, 4, 3, 0, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_select_blocks(NULL, &small, &p, NULL, fake, fake, NULL, NULL) == BSA_ERR_INVALID_ARGUMENT);

  /* structured lists and frame scores */
  bsa_struct_params sp;
  memset(&sp, 0, sizeof sp);
  sp.window = 0;
  EXPECT(bsa_structured_lists(fake, &small, &sp, NULL, fake, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  sp.window = 3;
  EXPECT(bsa_structured_lists(NULL, &small, &sp, NULL, fake, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_structured_lists(fake, &small, &sp, mis, fake, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_frame_scores(fake, &small, 0, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);
  EXPECT(bsa_frame_scores(NULL, &small, 2, fake, NULL) == BSA_ERR_INVALID_ARGUMENT);

  /* head labelling on the host: real work on host arrays */
  {
    const double alpha[2 * 4 * 3] = {
        0.6, 0.3, 0.1, 0.2, 0.7, 0.1, 0.1, 0.1, 0.8, 0.4, 0.4, 0.2, /* batch 0 */
        0.5, 0.4, 0.1, 0.05, 0.05, 0.9, 0.3, 0.6, 0.1, 0.2, 0.2, 0.6, /* batch 1 */
    };
    int32_t cls[8];
    memset(cls, 0x7f, sizeof cls);
    EXPECT(bsa_classify_heads(alpha, 2, 4, 2, cls) == BSA_OK);
    /* batch 0: max(sink, neighbor) = 0.6, 0.7, 0.1, 0.4 -> dummy heads 2 and 3 */
    EXPECT(cls[0] == BSA_HEAD_SINK && cls[1] == BSA_HEAD_NEIGHBOR && cls[2] == BSA_HEAD_DUMMY &&
           cls[3] == BSA_HEAD_DUMMY);
    /* batch 1: 0.5, 0.05, 0.6, 0.2 -> dummy heads 1 and 3 */
    EXPECT(cls[4] == BSA_HEAD_SINK && cls[5] == BSA_HEAD_DUMMY && cls[6] == BSA_HEAD_NEIGHBOR &&
           cls[7] == BSA_HEAD_DUMMY);
    double nan_alpha[3] = {NAN, 0.1, 0.2};
    EXPECT(bsa_classify_heads(nan_alpha, 1, 1, 0, cls) == BSA_ERR_INVALID_ARGUMENT);
    EXPECT(bsa_classify_heads(alpha, 2, 4, 5, cls) == BSA_ERR_INVALID_ARGUMENT);
    EXPECT(bsa_classify_heads(NULL, 2, 4, 1, cls) == BSA_ERR_INVALID_ARGUMENT);
  }

  /* status strings and the error message of every status */
  for (int32_t s = 0; s <= 4; ++s) EXPECT(bsa_status_string(s) != NULL && strlen(bsa_status_string(s)) > 0);
  EXPECT(bsa_abi_version() == BSA_ABI_VERSION);

  if (failures) fprintf(stderr, "%d check(s) failed\n", failures);
  else printf("all validation checks passed\n");
  return failures ? 1 : 0;
}
