/*
 * A plain C consumer of libfll: the boundary used without Python or torch.
 *
 *   fll_client plan         host only (no GPU needed): plans a problem and
 *                           checks that bad problems get the documented
 *                           status codes; prints "ok".
 *   fll_client run DIR      reads a bf16 selective-log-prob problem from
 *                           DIR (meta.txt and raw little-endian arrays),
 *                           runs fll_fwd_bwd on a HIP stream of its own
 *                           with device memory from hipMalloc, and writes
 *                           loss.bin, per_row.bin, dX.bin, dW.bin, db.bin.
 *
 * meta.txt: "BT H V reduction has_bias compute_dW compute_db temperature
 * has_weights ignore_index". Arrays: X.bin (bf16 [BT x H]), W.bin (bf16
 * [V x H]), b.bin (bf16 [V], if has_bias), labels.bin (int64 [BT]),
 * weights.bin (fp32 [BT], if has_weights).
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fll.h"

#define HIP_OK(call)                                                         \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call,          \
              hipGetErrorString(e_));                                        \
      exit(2);                                                               \
    }                                                                        \
  } while (0)

static fll_problem base_problem(void) {
  fll_problem p;
  memset(&p, 0, sizeof(p));
  p.BT = 1000;
  p.H = 64;
  p.V = 5000;
  p.dtype = FLL_BF16;
  p.head = FLL_HEAD_SELECTIVE_LOGPROB;
  p.reduction = FLL_RED_MEAN;
  p.ignore_index = -100;
  p.temperature = 1.0f;
  p.eps = 1e-10f;
  return p;
}

static int expect(const char *what, int got, int want) {
  if (got == want) return 0;
  fprintf(stderr, "%s: status %d (%s), expected %d (%s); %s\n", what, got,
          fll_strerror(got), want, fll_strerror(want), fll_last_error());
  return 1;
}

static int plan_checks(void) {
  int bad = 0;
  if (fll_version() != FLL_VERSION) {
    fprintf(stderr, "library version %d, header %d\n", fll_version(), FLL_VERSION);
    return 1;
  }
  fll_problem p = base_problem();
  fll_plan_t plan;
  bad |= expect("plan", fll_plan(&p, 0, 0, &plan), FLL_OK);
  if (!bad && (plan.n_chunks < 2 || plan.chunk_rows * plan.n_chunks < p.BT ||
               plan.workspace_bytes == 0)) {
    fprintf(stderr, "plan: C %lld x %lld chunks, %zu bytes\n", (long long)plan.chunk_rows,
            (long long)plan.n_chunks, plan.workspace_bytes);
    bad = 1;
  }
  fll_problem q = p;
  q.reduction = FLL_RED_NONE;
  bad |= expect("reduction none", fll_plan(&q, 0, 0, &plan), FLL_ERR_UNSUPPORTED);
  q = p;
  q.H = 12;
  bad |= expect("H not a multiple of 8", fll_plan(&q, 0, 0, &plan), FLL_ERR_INVALID_ARG);
  q = p;
  q.compute_db = 1;
  bad |= expect("db without bias", fll_plan(&q, 0, 0, &plan), FLL_ERR_INVALID_ARG);
  bad |= expect("budget of 1 KiB", fll_plan(&p, 1024, 0, &plan), FLL_ERR_WORKSPACE);
  bad |= expect("null problem", fll_plan(NULL, 0, 0, &plan), FLL_ERR_INVALID_ARG);
  if (!bad) printf("ok\n");
  return bad;
}

static void *read_file(const char *dir, const char *name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) {
    perror(path);
    exit(2);
  }
  void *buf = malloc(bytes ? bytes : 1);
  if (!buf || fread(buf, 1, bytes, f) != bytes) {
    fprintf(stderr, "%s: short read\n", path);
    exit(2);
  }
  fclose(f);
  return buf;
}

static void write_file(const char *dir, const char *name, const void *buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(buf, 1, bytes, f) != bytes) {
    perror(path);
    exit(2);
  }
  fclose(f);
}

/* host buffer -> new device buffer (NULL stays NULL) */
static void *to_device(const void *host, size_t bytes) {
  if (!host) return NULL;
  void *d = NULL;
  HIP_OK(hipMalloc(&d, bytes ? bytes : 1));
  HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

static void *from_device(const void *dev, size_t bytes) {
  void *h = malloc(bytes ? bytes : 1);
  if (!h) exit(2);
  HIP_OK(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
  return h;
}

static int run(const char *dir) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/meta.txt", dir);
  FILE *f = fopen(path, "r");
  if (!f) {
    perror(path);
    return 2;
  }
  long long BT, H, V, ignore_index;
  int reduction, has_bias, compute_dW, compute_db, has_weights;
  float temperature;
  if (fscanf(f, "%lld %lld %lld %d %d %d %d %f %d %lld", &BT, &H, &V, &reduction,
             &has_bias, &compute_dW, &compute_db, &temperature, &has_weights,
             &ignore_index) != 10) {
    fprintf(stderr, "%s: bad meta\n", path);
    return 2;
  }
  fclose(f);

  fll_problem p = base_problem();
  p.BT = BT;
  p.H = H;
  p.V = V;
  p.reduction = reduction;
  p.has_bias = has_bias;
  p.compute_dW = compute_dW;
  p.compute_db = compute_db;
  p.temperature = temperature;
  p.ignore_index = ignore_index;
  fll_plan_t plan;
  int st = fll_plan(&p, 0, 0, &plan);
  if (st != FLL_OK) {
    fprintf(stderr, "fll_plan: %s: %s\n", fll_strerror(st), fll_last_error());
    return 1;
  }

  const size_t nx = (size_t)BT * H, nw = (size_t)V * H;
  void *hX = read_file(dir, "X.bin", nx * 2);
  void *hW = read_file(dir, "W.bin", nw * 2);
  void *hb = has_bias ? read_file(dir, "b.bin", (size_t)V * 2) : NULL;
  void *hl = read_file(dir, "labels.bin", (size_t)BT * 8);
  void *hw = has_weights ? read_file(dir, "weights.bin", (size_t)BT * 4) : NULL;

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  fll_args a;
  memset(&a, 0, sizeof(a));
  a.X = to_device(hX, nx * 2);
  a.W = to_device(hW, nw * 2);
  a.b = to_device(hb, (size_t)V * 2);
  a.labels = (const int64_t *)to_device(hl, (size_t)BT * 8);
  a.weights = (const float *)to_device(hw, (size_t)BT * 4);
  HIP_OK(hipMalloc(&a.dX, nx * 2 + 1));
  HIP_OK(hipMalloc((void **)&a.loss, 4));
  HIP_OK(hipMalloc((void **)&a.per_row, (size_t)BT * 4 + 4));
  if (compute_dW) HIP_OK(hipMalloc((void **)&a.dW, nw * 4));
  if (compute_db) HIP_OK(hipMalloc((void **)&a.db, (size_t)V * 4));
  HIP_OK(hipMalloc(&a.workspace, plan.workspace_bytes));
  a.workspace_bytes = plan.workspace_bytes;

  st = fll_fwd_bwd(&plan, &a, (fll_stream)stream);
  if (st != FLL_OK) {
    fprintf(stderr, "fll_fwd_bwd: %s: %s\n", fll_strerror(st), fll_last_error());
    return 1;
  }
  HIP_OK(hipStreamSynchronize(stream));

  void *o;
  o = from_device(a.loss, 4);
  write_file(dir, "loss.bin", o, 4);
  free(o);
  o = from_device(a.per_row, (size_t)BT * 4);
  write_file(dir, "per_row.bin", o, (size_t)BT * 4);
  free(o);
  o = from_device(a.dX, nx * 2);
  write_file(dir, "dX.bin", o, nx * 2);
  free(o);
  if (compute_dW) {
    o = from_device(a.dW, nw * 4);
    write_file(dir, "dW.bin", o, nw * 4);
    free(o);
  }
  if (compute_db) {
    o = from_device(a.db, (size_t)V * 4);
    write_file(dir, "db.bin", o, (size_t)V * 4);
    free(o);
  }
  HIP_OK(hipFree((void *)a.X));
  HIP_OK(hipFree((void *)a.W));
  if (a.b) HIP_OK(hipFree((void *)a.b));
  HIP_OK(hipFree((void *)a.labels));
  if (a.weights) HIP_OK(hipFree((void *)a.weights));
  HIP_OK(hipFree(a.dX));
  HIP_OK(hipFree(a.loss));
  HIP_OK(hipFree(a.per_row));
  if (a.dW) HIP_OK(hipFree(a.dW));
  if (a.db) HIP_OK(hipFree(a.db));
  HIP_OK(hipFree(a.workspace));
  HIP_OK(hipStreamDestroy(stream));
  free(hX);
  free(hW);
  free(hb);
  free(hl);
  free(hw);
  printf("ok\n");
  return 0;
}

int main(int argc, char **argv) {
  if (argc == 2 && strcmp(argv[1], "plan") == 0) return plan_checks();
  if (argc == 3 && strcmp(argv[1], "run") == 0) return run(argv[2]);
  fprintf(stderr, "usage: %s plan | run DIR\n", argv[0]);
  return 2;
}
