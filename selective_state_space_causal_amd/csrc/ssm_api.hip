// ssm_api.hip -- the C ABI declared in include/ssm.h: argument validation on the host
// (before any HIP call), choice of decomposition, and launches on the caller's stream.
#include <string.h>

#include "../../include/ssm.h"
#include "ssm_internal.h"

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi), empty when lo == hi
};

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// bytes = n0 * n1 * n2 * esize, false on overflow
bool tensor_bytes(int64_t n0, int64_t n1, int64_t n2, int64_t esize, int64_t* bytes) {
  int64_t t;
  return mul_ok(n0, n1, &t) && mul_ok(t, n2, &t) && mul_ok(t, esize, bytes);
}

Range span(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, p ? lo + (uintptr_t)bytes : lo};
}

bool overlaps(Range a, Range b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

// Shape / dtype checks shared by both entry points.  L is validated only when use_L.
int check_dims(const ssm_dims* d, bool use_L) {
  if (!d) return SSM_ERR_NULL;
  if (d->batch < 1 || d->d_inner < 1 || d->d_inner > SSM_MAX_D_INNER || d->d_state < 1 || d->d_state > SSM_MAX_STATE ||
      d->d_conv != SSM_CONV_WIDTH || (use_L && d->seqlen < 1) ||
      (use_L && d->chunk_hint != 0 && d->chunk_hint != 1 && d->chunk_hint != 8))
    return SSM_ERR_SHAPE;
  if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  // Every byte count the kernels index must fit in int64.  (Large batches are split into
  // several launches over batch rows, so batch * d_inner has no bound of its own.)
  const int64_t L = use_L ? d->seqlen : 1, es = d->io_dtype == SSM_BF16 ? 2 : 4;
  int64_t bytes;
  if (!tensor_bytes(d->batch, d->d_inner, L, es, &bytes) || !tensor_bytes(d->batch, L, d->d_state, es, &bytes) ||
      !tensor_bytes(d->batch, d->d_inner, d->d_state, 4, &bytes))
    return SSM_ERR_SHAPE;
  return SSM_OK;
}

int check_params(const ssm_params* p, const void* const* outs, const int64_t* out_bytes, int nouts, int64_t D,
                 int64_t N) {
  if (!p || !p->A || !p->Dskip || !p->dt_bias || !p->conv_w) return SSM_ERR_NULL;
  const void* ptrs[5] = {p->A, p->Dskip, p->dt_bias, p->conv_w, p->conv_b};
  const int64_t bytes[5] = {D * N * 4, D * 4, D * 4, D * 4 * 4, D * 4};
  const uintptr_t align[5] = {16, 4, 4, 16, 4};  // A and conv_w rows are read as 16-byte vectors
  for (int i = 0; i < 5; ++i) {
    if (!ptrs[i]) continue;
    if (!aligned(ptrs[i], align[i])) return SSM_ERR_ALIGN;
    for (int o = 0; o < nouts; ++o)
      if (overlaps(span(ptrs[i], bytes[i]), span(outs[o], out_bytes[o]))) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

ssm::ScanArgs make_args(const ssm_dims* d, const ssm_params* p) {
  ssm::ScanArgs a;
  memset(&a, 0, sizeof a);
  a.A = p->A;
  a.Dskip = p->Dskip;
  a.dt_bias = p->dt_bias;
  a.conv_w = p->conv_w;
  a.conv_b = p->conv_b;
  a.B = d->batch;
  a.L = d->seqlen;
  a.D = d->d_inner;
  a.N = (int)d->d_state;
  a.bf16 = d->io_dtype == SSM_BF16;
  a.chunk_hint = d->chunk_hint;
  return a;
}

// Every output range must miss every input range and every other output range.
int check_overlaps(const void* const* ins, const int64_t* in_bytes, int nins, const void* const* outs,
                   const int64_t* out_bytes, int nouts) {
  for (int o = 0; o < nouts; ++o) {
    for (int i = 0; i < nins; ++i)
      if (overlaps(span(outs[o], out_bytes[o]), span(ins[i], in_bytes[i]))) return SSM_ERR_ALIAS;
    for (int q = o + 1; q < nouts; ++q)
      if (overlaps(span(outs[o], out_bytes[o]), span(outs[q], out_bytes[q]))) return SSM_ERR_ALIAS;
  }
  return SSM_OK;
}

// Cache-pool sizes: S * D * N and S * D * 3 fp32 values must not overflow.
int check_pool(const ssm_dims* d, int64_t pool) {
  int64_t bytes;
  if (pool < 1 || !tensor_bytes(pool, d->d_inner, d->d_state, 4, &bytes) ||
      !tensor_bytes(pool, d->d_inner, 3, 4, &bytes))
    return SSM_ERR_SHAPE;
  return SSM_OK;
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_str(int s) {
  switch (s) {
    case SSM_OK: return "ok";
    case SSM_ERR_NULL: return "a required pointer is NULL";
    case SSM_ERR_SHAPE:
      return "invalid sizes (batch/seqlen >= 1, 1 <= d_inner <= 2^24, 1 <= d_state <= 16, d_conv == 4)";
    case SSM_ERR_DTYPE: return "io_dtype must be SSM_F32 or SSM_BF16";
    case SSM_ERR_ALIGN: return "a tensor base pointer is misaligned (see the alignment rule in ssm.h)";
    case SSM_ERR_ALIAS: return "an output overlaps an input or another output";
    case SSM_ERR_WORKSPACE: return "workspace missing or smaller than ssm_prefill_workspace_bytes()";
    case SSM_ERR_LAUNCH: return "kernel launch failed";
    case SSM_ERR_SCRATCH: return "the sizes need more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

size_t ssm_prefill_workspace_bytes(const ssm_dims* d) {
  if (check_dims(d, true) != SSM_OK) return 0;
  ssm_params none;
  memset(&none, 0, sizeof none);
  return ssm::prefill_workspace_bytes(make_args(d, &none));
}

int ssm_prefill(const ssm_dims* d, const ssm_params* p, const void* x, const void* dt, const void* z,
                const void* Bm, const void* Cm, const float* h0, const float* conv0, void* y, float* h_out,
                float* conv_out, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(d, true);
  if (st != SSM_OK) return st;
  if (!x || !dt || !Bm || !Cm || !y || !h_out || !conv_out) return SSM_ERR_NULL;
  const int64_t B = d->batch, L = d->seqlen, D = d->d_inner, N = d->d_state;
  const int64_t es = d->io_dtype == SSM_BF16 ? 2 : 4;
  const int64_t seq = B * D * L * es, bc = B * L * N * es, hb = B * D * N * 4, cvb = B * D * 3 * 4;

  const void* ins[7] = {x, dt, z, Bm, Cm, h0, conv0};
  const int64_t in_bytes[7] = {seq, seq, seq, bc, bc, hb, cvb};
  const void* outs[3] = {y, h_out, conv_out};
  const int64_t out_bytes[3] = {seq, hb, cvb};
  for (int i = 0; i < 7; ++i)
    if (ins[i] && !aligned16(ins[i])) return SSM_ERR_ALIGN;
  for (int o = 0; o < 3; ++o)
    if (!aligned16(outs[o])) return SSM_ERR_ALIGN;
  st = check_params(p, outs, out_bytes, 3, D, N);
  if (st != SSM_OK) return st;
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 7; ++i)
      if (overlaps(span(outs[o], out_bytes[o]), span(ins[i], in_bytes[i]))) return SSM_ERR_ALIAS;
    for (int q = o + 1; q < 3; ++q)
      if (overlaps(span(outs[o], out_bytes[o]), span(outs[q], out_bytes[q]))) return SSM_ERR_ALIAS;
  }

  ssm::ScanArgs a = make_args(d, p);
  a.x = x;
  a.dt = dt;
  a.z = z;
  a.Bm = Bm;
  a.Cm = Cm;
  a.h0 = h0;
  a.conv0 = conv0;
  a.y = y;
  a.h_out = h_out;
  a.conv_out = conv_out;
  const size_t need = ssm::prefill_workspace_bytes(a);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return SSM_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SSM_ERR_ALIGN;
    const Range ws = span(workspace, (int64_t)need);
    for (int i = 0; i < 7; ++i)
      if (overlaps(ws, span(ins[i], in_bytes[i]))) return SSM_ERR_ALIAS;
    for (int o = 0; o < 3; ++o)
      if (overlaps(ws, span(outs[o], out_bytes[o]))) return SSM_ERR_ALIAS;
  }
  (void)hipGetLastError();  // drop a stale error so a launch failure is reported as ours
  if (ssm::launch_prefill(a, workspace, static_cast<hipStream_t>(stream)) != hipSuccess) return SSM_ERR_LAUNCH;
  return SSM_OK;
}

int ssm_decode_step(const ssm_dims* d, const ssm_params* p, const void* x_t, const void* dt_t, const void* z_t,
                    const void* B_t, const void* C_t, void* y_t, float* h, float* conv_state, void* stream) {
  int st = check_dims(d, false);
  if (st != SSM_OK) return st;
  if (!x_t || !dt_t || !B_t || !C_t || !y_t || !h || !conv_state) return SSM_ERR_NULL;
  const int64_t B = d->batch, D = d->d_inner, N = d->d_state;
  const int64_t es = d->io_dtype == SSM_BF16 ? 2 : 4;
  const int64_t tok = B * D * es, bc = B * N * es, hb = B * D * N * 4, cvb = B * D * 3 * 4;
  const void* ins[5] = {x_t, dt_t, z_t, B_t, C_t};
  const int64_t in_bytes[5] = {tok, tok, tok, bc, bc};
  const void* outs[3] = {y_t, h, conv_state};
  const int64_t out_bytes[3] = {tok, hb, cvb};
  // Decode reads io tensors element by element: natural alignment suffices.  h moves as
  // 16-byte vectors; the conv window as floats.
  for (int i = 0; i < 5; ++i)
    if (ins[i] && !aligned(ins[i], (uintptr_t)es)) return SSM_ERR_ALIGN;
  if (!aligned(y_t, (uintptr_t)es) || !aligned16(h) || !aligned(conv_state, 4)) return SSM_ERR_ALIGN;
  st = check_params(p, outs, out_bytes, 3, D, N);
  if (st != SSM_OK) return st;
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 5; ++i)
      if (overlaps(span(outs[o], out_bytes[o]), span(ins[i], in_bytes[i]))) return SSM_ERR_ALIAS;
    for (int q = o + 1; q < 3; ++q)
      if (overlaps(span(outs[o], out_bytes[o]), span(outs[q], out_bytes[q]))) return SSM_ERR_ALIAS;
  }
  ssm::ScanArgs a = make_args(d, p);
  a.L = 1;
  a.x = x_t;
  a.dt = dt_t;
  a.z = z_t;
  a.Bm = B_t;
  a.Cm = C_t;
  a.h0 = h;
  a.conv0 = conv_state;
  a.y = y_t;
  a.h_out = h;
  a.conv_out = conv_state;
  (void)hipGetLastError();
  if (ssm::launch_decode(a, static_cast<hipStream_t>(stream)) != hipSuccess) return SSM_ERR_LAUNCH;
  return SSM_OK;
}

int ssm_prefill_pool(const ssm_dims* d, const ssm_params* p, const void* x, const void* dt, const void* z,
                     const void* Bm, const void* Cm, const int32_t* seqlens, const int32_t* slots,
                     int64_t pool_size, int resume, void* y, float* h_pool, float* conv_pool, void* stream) {
  int st = check_dims(d, true);
  if (st != SSM_OK) return st;
  if (!x || !dt || !Bm || !Cm || !slots || !y || !h_pool || !conv_pool) return SSM_ERR_NULL;
  st = check_pool(d, pool_size);
  if (st != SSM_OK) return st;
  const int64_t B = d->batch, L = d->seqlen, D = d->d_inner, N = d->d_state, S = pool_size;
  const int64_t es = d->io_dtype == SSM_BF16 ? 2 : 4;
  const int64_t seq = B * D * L * es, bc = B * L * N * es, hb = S * D * N * 4, cvb = S * D * 3 * 4;
  const void* ins[7] = {x, dt, z, Bm, Cm, seqlens, slots};
  const int64_t in_bytes[7] = {seq, seq, seq, bc, bc, B * 4, B * 4};
  const void* outs[3] = {y, h_pool, conv_pool};
  const int64_t out_bytes[3] = {seq, hb, cvb};
  for (int i = 0; i < 5; ++i)
    if (ins[i] && !aligned16(ins[i])) return SSM_ERR_ALIGN;
  if ((seqlens && !aligned(seqlens, 4)) || !aligned(slots, 4)) return SSM_ERR_ALIGN;
  for (int o = 0; o < 3; ++o)
    if (!aligned16(outs[o])) return SSM_ERR_ALIGN;
  st = check_params(p, outs, out_bytes, 3, D, N);
  if (st != SSM_OK) return st;
  st = check_overlaps(ins, in_bytes, 7, outs, out_bytes, 3);
  if (st != SSM_OK) return st;

  ssm::ScanArgs a = make_args(d, p);
  a.x = x;
  a.dt = dt;
  a.z = z;
  a.Bm = Bm;
  a.Cm = Cm;
  a.h0 = resume ? h_pool : nullptr;  // each cache entry is read before it is rewritten, by the same wave
  a.conv0 = resume ? conv_pool : nullptr;
  a.y = y;
  a.h_out = h_pool;
  a.conv_out = conv_pool;
  a.seqlens = seqlens;
  a.slots = slots;
  a.pool = S;
  if (ssm::prefill_workspace_bytes(a) != 0) return SSM_ERR_WORKSPACE;  // no variant here needs scratch
  (void)hipGetLastError();
  if (ssm::launch_prefill(a, nullptr, static_cast<hipStream_t>(stream)) != hipSuccess) return SSM_ERR_LAUNCH;
  return SSM_OK;
}

int ssm_decode_step_pool(const ssm_dims* d, const ssm_params* p, const void* x_t, const void* dt_t,
                         const void* z_t, const void* B_t, const void* C_t, const int32_t* slots,
                         int64_t pool_size, void* y_t, float* h_pool, float* conv_pool, void* stream) {
  int st = check_dims(d, false);
  if (st != SSM_OK) return st;
  if (!x_t || !dt_t || !B_t || !C_t || !slots || !y_t || !h_pool || !conv_pool) return SSM_ERR_NULL;
  st = check_pool(d, pool_size);
  if (st != SSM_OK) return st;
  const int64_t B = d->batch, D = d->d_inner, N = d->d_state, S = pool_size;
  const int64_t es = d->io_dtype == SSM_BF16 ? 2 : 4;
  const int64_t tok = B * D * es, bc = B * N * es, hb = S * D * N * 4, cvb = S * D * 3 * 4;
  const void* ins[6] = {x_t, dt_t, z_t, B_t, C_t, slots};
  const int64_t in_bytes[6] = {tok, tok, tok, bc, bc, B * 4};
  const void* outs[3] = {y_t, h_pool, conv_pool};
  const int64_t out_bytes[3] = {tok, hb, cvb};
  for (int i = 0; i < 5; ++i)
    if (ins[i] && !aligned(ins[i], (uintptr_t)es)) return SSM_ERR_ALIGN;
  if (!aligned(slots, 4) || !aligned(y_t, (uintptr_t)es) || !aligned16(h_pool) || !aligned(conv_pool, 4))
    return SSM_ERR_ALIGN;
  st = check_params(p, outs, out_bytes, 3, D, N);
  if (st != SSM_OK) return st;
  st = check_overlaps(ins, in_bytes, 6, outs, out_bytes, 3);
  if (st != SSM_OK) return st;
  ssm::ScanArgs a = make_args(d, p);
  a.L = 1;
  a.x = x_t;
  a.dt = dt_t;
  a.z = z_t;
  a.Bm = B_t;
  a.Cm = C_t;
  a.h0 = h_pool;
  a.conv0 = conv_pool;
  a.y = y_t;
  a.h_out = h_pool;
  a.conv_out = conv_pool;
  a.slots = slots;
  a.pool = S;
  (void)hipGetLastError();
  if (ssm::launch_decode(a, static_cast<hipStream_t>(stream)) != hipSuccess) return SSM_ERR_LAUNCH;
  return SSM_OK;
}

}  // extern "C"
