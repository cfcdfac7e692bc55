/*
 * A plain C99 client of the C ABI (include/bsa.h, libbsa.so): the three hot-path
 * calls on one geometry, with nothing but the HIP runtime's C API for memory.
 *
 *   bsa_example DIR B H TEXT_LEN FRAMES LATENT_H LATENT_W HEAD_DIM Q_BLOCK K_BLOCK SEQ_ALLOC KEEP_RATIO
 *
 * reads DIR/q.bin, DIR/k.bin, DIR/v.bin (bf16 bits, [B, H, SEQ_ALLOC, HEAD_DIM]),
 * runs bsa_pool_blocks on Q and K, bsa_build_mask (top-k with frame-0 rows
 * dense) and bsa_forward (with the LSE), and writes DIR/cnt.bin (int32
 * [B, H, nqb]), DIR/idx.bin (int32 [B, H, nqb, nkb]), DIR/out.bin (bf16 bits)
 * and DIR/lse.bin (float32 [B, H, SEQ_ALLOC]); then bsa_forward_split with
 * the frame-0 rows split in two (its workspace from
 * bsa_forward_split_workspace_bytes) into DIR/out_split.bin and
 * DIR/lse_split.bin.  Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "bsa.h"

#define HIP_OK(x)                                                              \
  do {                                                                         \
    hipError_t e_ = (x);                                                       \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));           \
      return 2;                                                                \
    }                                                                          \
  } while (0)

#define BSA_OK_(x)                                                             \
  do {                                                                         \
    bsa_status s_ = (x);                                                       \
    if (s_ != BSA_OK) {                                                        \
      fprintf(stderr, "%s: %s: %s\n", #x, bsa_status_string(s_), bsa_last_error()); \
      return 3;                                                                \
    }                                                                          \
  } while (0)

static int read_file(const char* dir, const char* name, void* dst, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return -1;
  size_t n = fread(dst, 1, bytes, f);
  fclose(f);
  return n == bytes ? 0 : -1;
}

static int write_file(const char* dir, const char* name, const void* src, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return -1;
  size_t n = fwrite(src, 1, bytes, f);
  fclose(f);
  return n == bytes ? 0 : -1;
}

int main(int argc, char** argv) {
  if (argc != 13) {
    fprintf(stderr, "usage: %s DIR B H TEXT_LEN FRAMES LATENT_H LATENT_W HEAD_DIM Q_BLOCK K_BLOCK SEQ_ALLOC KEEP_RATIO\n",
            argv[0]);
    return 1;
  }
  const char* dir = argv[1];
  bsa_geometry g;
  memset(&g, 0, sizeof g);
  g.B = atoi(argv[2]);
  g.H = atoi(argv[3]);
  g.text_len = atoi(argv[4]);
  g.frames = atoi(argv[5]);
  g.latent_h = atoi(argv[6]);
  g.latent_w = atoi(argv[7]);
  g.head_dim = atoi(argv[8]);
  g.q_block = atoi(argv[9]);
  g.k_block = atoi(argv[10]);
  g.seq_alloc = atoll(argv[11]);

  bsa_mask_params p;
  memset(&p, 0, sizeof p);
  p.mode = BSA_SELECT_TOPK;
  p.topk = 0;
  p.keep_ratio = atof(argv[12]);
  p.frame0_dense = 1;

  bsa_derived d;
  BSA_OK_(bsa_derive(&g, &p, &d));
  if (bsa_abi_version() != BSA_ABI_VERSION) {
    fprintf(stderr, "ABI version %d, header %d\n", bsa_abi_version(), BSA_ABI_VERSION);
    return 4;
  }

  const size_t BH = (size_t)g.B * g.H;
  const size_t n_x = BH * (size_t)g.seq_alloc * g.head_dim;
  const size_t n_rows = BH * (size_t)d.nqb;
  const size_t n_list = n_rows * (size_t)d.nkb;
  uint16_t* hq = malloc(n_x * 2);
  uint16_t* hk = malloc(n_x * 2);
  uint16_t* hv = malloc(n_x * 2);
  uint16_t* ho = malloc(n_x * 2);
  int32_t* hcnt = malloc(n_rows * 4);
  int32_t* hidx = malloc(n_list * 4);
  float* hlse = malloc(BH * (size_t)g.seq_alloc * 4);
  if (!hq || !hk || !hv || !ho || !hcnt || !hidx || !hlse) return 5;
  if (read_file(dir, "q.bin", hq, n_x * 2) || read_file(dir, "k.bin", hk, n_x * 2) ||
      read_file(dir, "v.bin", hv, n_x * 2)) {
    fprintf(stderr, "cannot read q.bin / k.bin / v.bin in %s\n", dir);
    return 6;
  }

  void *q, *k, *v, *out;
  float *qp, *kp, *lse;
  uint8_t* mask;
  int32_t *cnt, *idx;
  HIP_OK(hipMalloc(&q, n_x * 2));
  HIP_OK(hipMalloc(&k, n_x * 2));
  HIP_OK(hipMalloc(&v, n_x * 2));
  HIP_OK(hipMalloc(&out, n_x * 2));
  HIP_OK(hipMalloc((void**)&qp, BH * (size_t)d.nqb * g.head_dim * 4));
  HIP_OK(hipMalloc((void**)&kp, BH * (size_t)d.nkb * g.head_dim * 4));
  HIP_OK(hipMalloc((void**)&mask, n_list));
  HIP_OK(hipMalloc((void**)&cnt, n_rows * 4));
  HIP_OK(hipMalloc((void**)&idx, n_list * 4));
  HIP_OK(hipMalloc((void**)&lse, BH * (size_t)g.seq_alloc * 4));
  HIP_OK(hipMemcpy(q, hq, n_x * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, hk, n_x * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, hv, n_x * 2, hipMemcpyHostToDevice));

  /* the hot path, on the default stream */
  BSA_OK_(bsa_pool_blocks(q, BSA_DTYPE_BF16, &g, g.q_block, qp, NULL));
  BSA_OK_(bsa_pool_blocks(k, BSA_DTYPE_BF16, &g, g.k_block, kp, NULL));
  BSA_OK_(bsa_build_mask(qp, kp, &g, &p, mask, cnt, idx, NULL, NULL));
  BSA_OK_(bsa_forward(q, k, v, BSA_DTYPE_BF16, &g, cnt, idx, NULL, 0.0f, out, lse, NULL));
  HIP_OK(hipDeviceSynchronize());

  HIP_OK(hipMemcpy(hcnt, cnt, n_rows * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hidx, idx, n_list * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(ho, out, n_x * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hlse, lse, BH * (size_t)g.seq_alloc * 4, hipMemcpyDeviceToHost));
  if (write_file(dir, "cnt.bin", hcnt, n_rows * 4) || write_file(dir, "idx.bin", hidx, n_list * 4) ||
      write_file(dir, "out.bin", ho, n_x * 2) || write_file(dir, "lse.bin", hlse, BH * (size_t)g.seq_alloc * 4)) {
    fprintf(stderr, "cannot write results to %s\n", dir);
    return 7;
  }

  /* the same forward with the frame-0 rows' key lists split in two */
  int64_t ws_bytes = 0;
  BSA_OK_(bsa_forward_split_workspace_bytes(&g, 2, &ws_bytes));
  void* ws = NULL;
  if (ws_bytes > 0) HIP_OK(hipMalloc(&ws, (size_t)ws_bytes));
  BSA_OK_(bsa_forward_split(q, k, v, BSA_DTYPE_BF16, &g, cnt, idx, NULL, 0.0f, out, lse, NULL, 2, ws, ws_bytes,
                            NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(ho, out, n_x * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hlse, lse, BH * (size_t)g.seq_alloc * 4, hipMemcpyDeviceToHost));
  if (write_file(dir, "out_split.bin", ho, n_x * 2) ||
      write_file(dir, "lse_split.bin", hlse, BH * (size_t)g.seq_alloc * 4)) {
    fprintf(stderr, "cannot write results to %s\n", dir);
    return 7;
  }
  if (ws) hipFree(ws);

  /* an invalid call is rejected on the host with a message */
  bsa_geometry bad = g;
  bad.head_dim = 96;
  if (bsa_forward(q, k, v, BSA_DTYPE_BF16, &bad, cnt, idx, NULL, 0.0f, out, lse, NULL) != BSA_ERR_UNSUPPORTED ||
      strlen(bsa_last_error()) == 0) {
    fprintf(stderr, "head_dim 96 was not rejected\n");
    return 8;
  }

  hipFree(q); hipFree(k); hipFree(v); hipFree(out); hipFree(qp); hipFree(kp);
  hipFree(mask); hipFree(cnt); hipFree(idx); hipFree(lse);
  free(hq); free(hk); free(hv); free(ho); free(hcnt); free(hidx); free(hlse);
  printf("ok nqb=%d nkb=%d\n", d.nqb, d.nkb);
  return 0;
}
