/*
 * Runs pcx_forward and pcx_backward from plain C through include/pcx.h, with
 * device memory taken from the HIP runtime API only (no Python, no PyTorch):
 * a check that the C ABI stands on its own.  Test infrastructure, driven by
 * tests/test_gpu_c_abi.py.
 *
 * Input and output are little-endian binary files (fp32 problem):
 *   in:  int32 N, M, D, V, L_tot, blank, chunk;
 *        float32 X[M*D], W[V*D], b[V];
 *        int32 tgt_off[N+1], tgt[L_tot], frame_counts[N]
 *   out: float64 loss; int32 K, n_unalignable, n_nonfinite;
 *        float32 dX[M*D], dW[V*D], db[V]
 * usage: pcx_c_run IN OUT [callbacks]   (exit status 0 on success)
 * With "callbacks" the context's workspace comes from allocation callbacks
 * (hipMalloc / hipFree behind a counter); the program then fails unless
 * every buffer the library allocated was released by pcx_destroy.
 */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "pcx.h"

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));              \
      return 2;                                                               \
    }                                                                         \
  } while (0)
#define PCX_OK_(call)                                                         \
  do {                                                                        \
    pcx_status s_ = (call);                                                   \
    if (s_ != PCX_OK) {                                                       \
      fprintf(stderr, "%s: status %d: %s\n", #call, (int)s_, pcx_last_error()); \
      return 3;                                                               \
    }                                                                         \
  } while (0)

static void* read_block(FILE* f, size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p && bytes && fread(p, 1, bytes, f) != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

/* Allocation callbacks: device memory from the HIP runtime, counted. */
typedef struct {
  long live;
  long calls;
  size_t bytes;
} alloc_count;

static void* count_alloc(size_t bytes, void* user, void* stream) {
  alloc_count* c = (alloc_count*)user;
  void* p = NULL;
  (void)stream;
  if (hipMalloc(&p, bytes) != hipSuccess) return NULL;
  c->live += 1;
  c->calls += 1;
  c->bytes += bytes;
  return p;
}

static void count_release(void* ptr, size_t bytes, void* user, void* stream) {
  alloc_count* c = (alloc_count*)user;
  (void)stream;
  /* every library call ran on the default stream: wait for it, then free */
  (void)hipDeviceSynchronize();
  (void)hipFree(ptr);
  c->live -= 1;
  c->bytes -= bytes;
}

static int to_device(void** d, const void* h, size_t bytes) {
  if (hipMalloc(d, bytes ? bytes : 4) != hipSuccess) return 0;
  return bytes == 0 || hipMemcpy(*d, h, bytes, hipMemcpyHostToDevice) == hipSuccess;
}

int main(int argc, char** argv) {
  if (argc != 3 && argc != 4) {
    fprintf(stderr, "usage: %s IN OUT [callbacks]\n", argv[0]);
    return 1;
  }
  const int use_callbacks = argc == 4;
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  int32_t hdr[7];
  if (fread(hdr, sizeof(int32_t), 7, in) != 7) {
    fprintf(stderr, "short header\n");
    return 1;
  }
  const int32_t N = hdr[0], M = hdr[1], D = hdr[2], V = hdr[3], L_tot = hdr[4];
  const int32_t blank = hdr[5], chunk = hdr[6];
  const size_t xb = (size_t)M * D * 4, wb = (size_t)V * D * 4, bb = (size_t)V * 4;
  float* X = read_block(in, xb);
  float* W = read_block(in, wb);
  float* b = read_block(in, bb);
  int32_t* off = read_block(in, (size_t)(N + 1) * 4);
  int32_t* tgt = read_block(in, (size_t)L_tot * 4);
  int32_t* fc = read_block(in, (size_t)N * 4);
  fclose(in);
  if (!X || !W || !b || !off || !tgt || !fc) {
    fprintf(stderr, "short input\n");
    return 1;
  }

  void *dX_in, *dW_in, *db_in, *d_off, *d_tgt, *d_fc, *gX, *gW, *gb;
  if (!to_device(&dX_in, X, xb) || !to_device(&dW_in, W, wb) || !to_device(&db_in, b, bb) ||
      !to_device(&d_off, off, (size_t)(N + 1) * 4) || !to_device(&d_tgt, tgt, (size_t)L_tot * 4) ||
      !to_device(&d_fc, fc, (size_t)N * 4)) {
    fprintf(stderr, "device copy failed\n");
    return 2;
  }
  HIP_OK(hipMalloc(&gX, xb ? xb : 4));
  HIP_OK(hipMalloc(&gW, wb));
  HIP_OK(hipMalloc(&gb, bb));

  pcx_ctx* ctx = NULL;
  alloc_count counts_alloc = {0, 0, 0};
  if (use_callbacks)
    PCX_OK_(pcx_create(&ctx, count_alloc, count_release, &counts_alloc));
  else
    PCX_OK_(pcx_create(&ctx, NULL, NULL, NULL));
  double loss = 0.0;
  pcx_fwd_info info;
  PCX_OK_(pcx_forward(ctx, dX_in, dW_in, db_in, PCX_F32, M, D, V, N, (const int32_t*)d_off,
                      (const int32_t*)d_tgt, L_tot, (const int32_t*)d_fc, blank, chunk, NULL,
                      &loss, &info));
  PCX_OK_(pcx_backward(ctx, 1.0, gX, gW, gb, NULL));
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(X, gX, xb, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(W, gW, wb, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(b, gb, bb, hipMemcpyDeviceToHost));
  pcx_destroy(ctx);
  if (use_callbacks && (counts_alloc.calls == 0 || counts_alloc.live != 0 || counts_alloc.bytes != 0)) {
    fprintf(stderr, "allocation callbacks: %ld calls, %ld buffers / %zu bytes not released\n",
            counts_alloc.calls, counts_alloc.live, counts_alloc.bytes);
    return 4;
  }

  FILE* out = fopen(argv[2], "wb");
  if (!out) {
    perror(argv[2]);
    return 1;
  }
  const int32_t counts[3] = {info.K, info.n_unalignable, info.n_nonfinite};
  int ok = fwrite(&loss, sizeof(double), 1, out) == 1 &&
           fwrite(counts, sizeof(int32_t), 3, out) == 3 && fwrite(X, 1, xb, out) == xb &&
           fwrite(W, 1, wb, out) == wb && fwrite(b, 1, bb, out) == bb;
  fclose(out);
  void* bufs[] = {dX_in, dW_in, db_in, d_off, d_tgt, d_fc, gX, gW, gb};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) (void)hipFree(bufs[i]);
  free(X);
  free(W);
  free(b);
  free(off);
  free(tgt);
  free(fc);
  if (!ok) {
    fprintf(stderr, "write failed\n");
    return 1;
  }
  printf("loss %.17g K %d callbacks %ld\n", loss, info.K, counts_alloc.calls);
  return 0;
}
