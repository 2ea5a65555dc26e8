// ssm_proj.hip -- ssm_proj_* of include/ssm_proj.h: the channel-sliced projections around the
// scan ("Scaling State-Space Models on Multiple GPUs with Tensor Parallelism", euno.news
// summary of arXiv 2602.21144, Methodology items 1-2) as hipBLASLt GEMMs on the matrix cores,
// except one-token calls (a decode step), which ssm_gemv.hip streams as matrix-vector products,
// and channel-major outputs with a small inner dimension (the step-size projection), which
// ssm_lowk.hip runs.
//
// hipBLASLt is column-major.  A row-major [R, C] matrix is a column-major [C, R] one, so:
//   channel-major out (IN, DT): out_b[M, L] (row-major) is column-major [L, M] = in_b * W^T
//     where in_b row-major [L, K] is column-major [K, L] (op T) and W row-major [M, K] is
//     column-major [K, M] (op N): m = L, n = M, k = K, lda = K, ldb = K, ldd = L;
//   token-major out (X, OUT): out_b[L, M] (row-major) is column-major [M, L] = W * in_b
//     where W is column-major [K, M] (op T) and in_b row-major [K, L] is column-major [L, K]
//     (op T): m = M, n = L, k = K, lda = K, ldb = L, ldd = M.
// The batch is a strided batch (the weight's batch stride is 0).  Algorithms are chosen once
// per shape and cached in the context: hipBLASLt's heuristic offers up to 8, and for a shape of
// at least 1e10 flops the first call times them and keeps the fastest.
#include <hipblaslt/hipblaslt.h>
#include <string.h>

#include <new>
#include <vector>

#include "../../include/ssm_proj.h"
#include "ssm_gemv.h"
#include "ssm_lowk.h"

namespace {

constexpr size_t kWorkspace = size_t(64) << 20;  // device scratch a projection may use

constexpr int kCandidates = 8;           // heuristic candidates timed on a large shape's first call
constexpr double kTuneFlops = 1e10;      // shapes with fewer flops keep the heuristic's first choice

struct Plan {
  int32_t kind, io, out;
  int64_t B, L, K, M;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, d = nullptr;
  hipblasLtMatmulAlgo_t algo;
  hipblasLtMatmulAlgo_t cand[kCandidates];
  int ncand = 0;
  bool tuned = false;
};

bool channel_major_out(int32_t kind) { return kind == SSM_PROJ_IN || kind == SSM_PROJ_DT; }

hipDataType dtype_of(int32_t io) { return io == SSM_BF16 ? HIP_R_16BF : HIP_R_32F; }

void destroy_plan(Plan& p) {
  if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
  if (p.a) hipblasLtMatrixLayoutDestroy(p.a);
  if (p.b) hipblasLtMatrixLayoutDestroy(p.b);
  if (p.d) hipblasLtMatrixLayoutDestroy(p.d);
  p.desc = nullptr;
  p.a = p.b = p.d = nullptr;
}

hipblasStatus_t layout(hipblasLtMatrixLayout_t* out, hipDataType t, int64_t rows, int64_t cols, int64_t ld,
                       int32_t batch, int64_t stride) {
  hipblasStatus_t st = hipblasLtMatrixLayoutCreate(out, t, rows, cols, ld);
  if (st != HIPBLAS_STATUS_SUCCESS) return st;
  st = hipblasLtMatrixLayoutSetAttribute(*out, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &batch, sizeof batch);
  if (st != HIPBLAS_STATUS_SUCCESS) return st;
  return hipblasLtMatrixLayoutSetAttribute(*out, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &stride, sizeof stride);
}

}  // namespace

struct ssm_proj_ctx {
  hipblasLtHandle_t handle = nullptr;
  std::vector<Plan> plans;
};

namespace {

// Build (or find) the plan of one projection shape; false when hipBLASLt has no algorithm.
bool get_plan(ssm_proj_ctx* ctx, int32_t kind, int32_t io, int32_t out, int64_t B, int64_t L, int64_t K, int64_t M,
              Plan** result) {
  for (Plan& p : ctx->plans)
    if (p.kind == kind && p.io == io && p.out == out && p.B == B && p.L == L && p.K == K && p.M == M) {
      *result = &p;
      return true;
    }
  Plan p;
  p.kind = kind;
  p.io = io;
  p.out = out;
  p.B = B;
  p.L = L;
  p.K = K;
  p.M = M;
  const hipDataType ti = dtype_of(io), to = dtype_of(out);
  const int32_t nb = (int32_t)B;
  const bool cm = channel_major_out(kind);
  hipblasOperation_t opa = HIPBLAS_OP_T, opb = cm ? HIPBLAS_OP_N : HIPBLAS_OP_T;
  bool ok = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof opa) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof opb) ==
                HIPBLAS_STATUS_SUCCESS;
  if (ok && cm) {  // A = in (column-major [K, L]), B = W (column-major [K, M]), D column-major [L, M]
    ok = layout(&p.a, ti, K, L, K, nb, L * K) == HIPBLAS_STATUS_SUCCESS &&
         layout(&p.b, ti, K, M, K, nb, 0) == HIPBLAS_STATUS_SUCCESS &&
         layout(&p.d, to, L, M, L, nb, L * M) == HIPBLAS_STATUS_SUCCESS;
  } else if (ok) {  // A = W (column-major [K, M]), B = in (column-major [L, K]), D column-major [M, L]
    ok = layout(&p.a, ti, K, M, K, nb, 0) == HIPBLAS_STATUS_SUCCESS &&
         layout(&p.b, ti, L, K, L, nb, K * L) == HIPBLAS_STATUS_SUCCESS &&
         layout(&p.d, to, M, L, M, nb, L * M) == HIPBLAS_STATUS_SUCCESS;
  }
  hipblasLtMatmulPreference_t pref = nullptr;
  uint64_t ws = kWorkspace;
  ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
       hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof ws) ==
           HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulHeuristicResult_t heur[kCandidates];
  int found = 0;
  ok = ok && hipblasLtMatmulAlgoGetHeuristic(ctx->handle, p.desc, p.a, p.b, p.d, p.d, pref, kCandidates, heur,
                                             &found) == HIPBLAS_STATUS_SUCCESS;
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  for (int i = 0; ok && i < found; ++i)
    if (heur[i].state == HIPBLAS_STATUS_SUCCESS && heur[i].workspaceSize <= kWorkspace) p.cand[p.ncand++] = heur[i].algo;
  if (!ok || p.ncand == 0) {
    destroy_plan(p);
    return false;
  }
  p.algo = p.cand[0];
  p.tuned = p.ncand == 1 || 2.0 * (double)B * (double)L * (double)K * (double)M < kTuneFlops;
  ctx->plans.push_back(p);
  *result = &ctx->plans.back();
  return true;
}

// The first call of a large shape: time each heuristic candidate on the caller's own buffers
// (one untimed run, then two between events on the stream; the host waits) and keep the fastest.
// Skipped while the stream is being captured into a graph (the plan stays untuned until a call
// outside capture); a candidate that fails to run is passed over.
template <typename Run>
void tune(Plan* p, hipStream_t s, Run run) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    p->tuned = true;
    return;
  }
  float best = -1.0f;
  int pick = 0;
  for (int i = 0; i < p->ncand; ++i) {
    if (run(&p->cand[i]) != HIPBLAS_STATUS_SUCCESS) continue;
    float ms = 0.0f;
    if (hipEventRecord(e0, s) != hipSuccess || run(&p->cand[i]) != HIPBLAS_STATUS_SUCCESS ||
        run(&p->cand[i]) != HIPBLAS_STATUS_SUCCESS || hipEventRecord(e1, s) != hipSuccess ||
        hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess)
      continue;
    if (best < 0.0f || ms < best) {
      best = ms;
      pick = i;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  p->algo = p->cand[pick];
  p->tuned = true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

}  // namespace

extern "C" {

int ssm_proj_create(ssm_proj_ctx** ctx) {
  if (!ctx) return SSM_ERR_NULL;
  *ctx = nullptr;
  ssm_proj_ctx* c = new (std::nothrow) ssm_proj_ctx;
  if (!c) return SSM_ERR_LAUNCH;
  if (hipblasLtCreate(&c->handle) != HIPBLAS_STATUS_SUCCESS) {
    delete c;
    return SSM_ERR_LAUNCH;
  }
  *ctx = c;
  return SSM_OK;
}

void ssm_proj_destroy(ssm_proj_ctx* ctx) {
  if (!ctx) return;
  for (Plan& p : ctx->plans) destroy_plan(p);
  if (ctx->handle) hipblasLtDestroy(ctx->handle);
  delete ctx;
}

size_t ssm_proj_workspace_bytes(void) { return kWorkspace; }

int ssm_proj(ssm_proj_ctx* ctx, int32_t kind, int64_t batch, int64_t seqlen, int64_t in_features,
             int64_t out_features, int32_t io_dtype, int32_t out_dtype, const void* in, const void* w, void* out,
             void* workspace, size_t workspace_bytes, void* stream) {
  if (!ctx || !in || !w || !out) return SSM_ERR_NULL;
  if (kind < SSM_PROJ_IN || kind > SSM_PROJ_OUT || batch < 1 || seqlen < 1 || in_features < 1 || out_features < 1)
    return SSM_ERR_SHAPE;
  if ((io_dtype != SSM_F32 && io_dtype != SSM_BF16) || (out_dtype != SSM_F32 && out_dtype != SSM_BF16))
    return SSM_ERR_DTYPE;
  const int64_t ei = io_dtype == SSM_BF16 ? 2 : 4, eo = out_dtype == SSM_BF16 ? 2 : 4;
  int64_t t, in_bytes, w_bytes, out_bytes;
  if (batch > INT32_MAX || __builtin_mul_overflow(batch, seqlen, &t) ||
      __builtin_mul_overflow(t, in_features, &in_bytes) || __builtin_mul_overflow(in_bytes, ei, &in_bytes) ||
      __builtin_mul_overflow(in_features, out_features, &w_bytes) || __builtin_mul_overflow(w_bytes, ei, &w_bytes) ||
      __builtin_mul_overflow(t, out_features, &out_bytes) || __builtin_mul_overflow(out_bytes, eo, &out_bytes))
    return SSM_ERR_SHAPE;
  if (!aligned16(in) || !aligned16(w) || !aligned16(out)) return SSM_ERR_ALIGN;
  if (overlaps(out, out_bytes, in, in_bytes) || overlaps(out, out_bytes, w, w_bytes)) return SSM_ERR_ALIAS;
  if (!workspace || workspace_bytes < kWorkspace) return SSM_ERR_WORKSPACE;
  // One token per batch row (a decode step): a matrix-vector product, streamed by ssm_gemv.hip.
  if (seqlen == 1 && ssm::gemv_fits(batch, in_features, out_features, io_dtype == SSM_BF16))
    return ssm::gemv(io_dtype == SSM_BF16, out_dtype == SSM_BF16, batch, in_features, out_features, in, w, out,
                     static_cast<hipStream_t>(stream))
               ? SSM_OK
               : SSM_ERR_LAUNCH;
  // A small inner dimension with a channel-major output (the step-size projection): bound by
  // writing the output, streamed by ssm_lowk.hip.
  if ((kind == SSM_PROJ_IN || kind == SSM_PROJ_DT) &&
      ssm::lowk_fits(batch, seqlen, in_features, out_features, io_dtype == SSM_BF16, out_dtype == SSM_BF16))
    return ssm::lowk(batch, seqlen, in_features, out_features, in, w, out, static_cast<hipStream_t>(stream))
               ? SSM_OK
               : SSM_ERR_LAUNCH;
  Plan* p = nullptr;
  if (!get_plan(ctx, kind, io_dtype, out_dtype, batch, seqlen, in_features, out_features, &p)) return SSM_ERR_LAUNCH;
  const float alpha = 1.0f, beta = 0.0f;
  const bool cm = channel_major_out(kind);
  const void* A = cm ? in : w;
  const void* Bop = cm ? w : in;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto run = [&](const hipblasLtMatmulAlgo_t* algo) {
    return hipblasLtMatmul(ctx->handle, p->desc, &alpha, A, p->a, Bop, p->b, &beta, out, p->d, out, p->d, algo,
                           workspace, workspace_bytes, s);
  };
  if (!p->tuned) tune(p, s, run);
  return run(&p->algo) == HIPBLAS_STATUS_SUCCESS ? SSM_OK : SSM_ERR_LAUNCH;
}

}  // extern "C"
