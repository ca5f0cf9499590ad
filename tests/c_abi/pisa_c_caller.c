/* A plain C caller of the PISA C ABI (include/pisa.h): no Python, no torch.
 *
 *   pisa_c_caller DIR
 *
 * reads DIR/shape.txt ("B H L D block dtype topk sink variant scale"; dtype 0
 * fp32, 1 bf16; sink -1, 0 or 2147483648 for none is written as "none") and
 * DIR/q.bin, k.bin, v.bin (raw [B,H,L,D] tensors in the I/O dtype), runs the
 * three steps of the forward pass on the default stream with device memory
 * from hipMalloc, and writes DIR/o.bin (same layout and dtype as q) and
 * DIR/idx.bin ([B,H,n,topk] int32). Exit status 0 on success; on any error a
 * message on stderr and a nonzero status. Test fixture for the C ABI. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pisa.h"

static int fail(const char *what, const char *detail) {
  fprintf(stderr, "pisa_c_caller: %s: %s\n", what, detail);
  return 1;
}

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) return fail(#call, hipGetErrorString(e_)); \
  } while (0)

#define PISA_OK_(call)                                                          \
  do {                                                                          \
    pisa_status_t s_ = (call);                                                  \
    if (s_ != PISA_OK) return fail(#call, pisa_status_string(s_));              \
  } while (0)

static int read_file(const char *dir, const char *name, void *buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) return fail("open", path);
  size_t got = fread(buf, 1, bytes, f);
  fclose(f);
  return got == bytes ? 0 : fail("short read", path);
}

static int write_file(const char *dir, const char *name, const void *buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f) return fail("open", path);
  size_t put = fwrite(buf, 1, bytes, f);
  fclose(f);
  return put == bytes ? 0 : fail("short write", path);
}

int main(int argc, char **argv) {
  if (argc != 2) return fail("usage", "pisa_c_caller DIR");
  const char *dir = argv[1];
  char path[4096], sink_s[32];
  snprintf(path, sizeof path, "%s/shape.txt", dir);
  FILE *f = fopen(path, "r");
  if (!f) return fail("open", path);
  pisa_shape_t s;
  memset(&s, 0, sizeof s);
  int topk = 0, variant = 0;
  double scale = 0.0;
  int n_read = fscanf(f, "%d %d %d %d %d %d %d %31s %d %lf", &s.B, &s.H, &s.L, &s.D, &s.block,
                      &s.dtype, &topk, sink_s, &variant, &scale);
  fclose(f);
  if (n_read != 10) return fail("parse", path);
  const int32_t sink = strcmp(sink_s, "none") == 0 ? PISA_SINK_NONE : (int32_t)atoi(sink_s);
  s.layout = PISA_LAYOUT_BHLD;

  const size_t esz = s.dtype == PISA_BF16 ? 2 : 4;
  const size_t n = ((size_t)s.L + s.block - 1) / s.block;
  const size_t bh = (size_t)s.B * s.H;
  const size_t t_bytes = bh * s.L * s.D * esz;
  const size_t idx_bytes = bh * n * topk * sizeof(int32_t);
  const size_t ws_bytes = pisa_workspace_bytes(&s);
  if (ws_bytes == 0) return fail("pisa_workspace_bytes", "shape rejected");

  void *h_q = malloc(t_bytes), *h_k = malloc(t_bytes), *h_v = malloc(t_bytes);
  void *h_o = malloc(t_bytes), *h_idx = malloc(idx_bytes);
  if (!h_q || !h_k || !h_v || !h_o || !h_idx) return fail("malloc", "host buffers");
  if (read_file(dir, "q.bin", h_q, t_bytes) || read_file(dir, "k.bin", h_k, t_bytes) ||
      read_file(dir, "v.bin", h_v, t_bytes))
    return 1;

  void *q, *k, *v, *o, *ws;
  int32_t *idx;
  double *qbar, *kbar, *vsum, *hbar;
  HIP_OK(hipMalloc(&q, t_bytes));
  HIP_OK(hipMalloc(&k, t_bytes));
  HIP_OK(hipMalloc(&v, t_bytes));
  HIP_OK(hipMalloc(&o, t_bytes));
  HIP_OK(hipMalloc((void **)&idx, idx_bytes));
  HIP_OK(hipMalloc((void **)&qbar, bh * n * s.D * sizeof(double)));
  HIP_OK(hipMalloc((void **)&kbar, bh * n * s.D * sizeof(double)));
  HIP_OK(hipMalloc((void **)&vsum, bh * n * s.D * sizeof(double)));
  HIP_OK(hipMalloc((void **)&hbar, bh * s.D * s.D * sizeof(double)));
  HIP_OK(hipMalloc(&ws, ws_bytes));
  HIP_OK(hipMemcpy(q, h_q, t_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(k, h_k, t_bytes, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(v, h_v, t_bytes, hipMemcpyHostToDevice));

  pisa_stats_t st;
  memset(&st, 0, sizeof st);
  st.qbar = qbar;
  st.kbar = kbar;
  st.vsum = vsum;
  st.hbar = hbar;
  st.mnorm = NULL; /* no covariance-aware routing here */
  st.ws = ws;
  st.ws_bytes = ws_bytes;
  PISA_OK_(pisa_block_stats(&s, q, k, v, &st, NULL));
  PISA_OK_(pisa_select(&s, &st, scale, 0.0, topk, sink, idx, NULL));
  PISA_OK_(pisa_attn_fwd(&s, q, &st, variant, idx, topk, scale, o, NULL));
  HIP_OK(hipDeviceSynchronize());

  HIP_OK(hipMemcpy(h_o, o, t_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(h_idx, idx, idx_bytes, hipMemcpyDeviceToHost));
  if (write_file(dir, "o.bin", h_o, t_bytes) || write_file(dir, "idx.bin", h_idx, idx_bytes)) return 1;

  hipFree(q); hipFree(k); hipFree(v); hipFree(o); hipFree(idx);
  hipFree(qbar); hipFree(kbar); hipFree(vsum); hipFree(hbar); hipFree(ws);
  free(h_q); free(h_k); free(h_v); free(h_o); free(h_idx);
  printf("pisa_c_caller: ok\n");
  return 0;
}
