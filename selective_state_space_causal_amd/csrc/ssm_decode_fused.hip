// ssm_decode_fused.hip -- ssm_decode_fused of include/ssm_layer.h: one decoded token through the
// conv front, x_proj, dt_proj and the decode step of one rank's mixer layer in two kernels
// ("Scaling State-Space Models on Multiple GPUs with Tensor Parallelism", euno.news summary of
// arXiv 2602.21144, Methodology items 1 and 3).
//
// x_proj contracts over every channel of the slice, and dt_proj and the step of every channel
// need its result, so the work splits at that reduction:
//   xproj_partial  one workgroup per (batch row, block of 64 channels, block of 64 outputs): the
//                  block's conv front from the cache (rounded to the io dtype, as the unfused layer
//                  stores u), then the channel block's share of 64 of the R + 2N x_proj outputs,
//                  four threads per output, written as an fp32 partial sum into the workspace;
//   dt_decode      one workgroup per (batch row, block of 32 channels), four lanes per channel:
//                  the batch row's R + 2N outputs as the sum of the blocks' partials (in block
//                  order, then rounded to the io dtype), then per channel its dt_proj dot product
//                  split over the four lanes (rounded to the io dtype), then the decode step of
//                  ssm_decode_step (decode_quad_step: the same arithmetic, the same bits).
// The step rewrites the conv cache that xproj_partial reads; the two launches are stream-ordered.
#include <string.h>

#include <mutex>

#include "../../include/ssm_layer.h"
#include "ssm_decode_quad.h"
#include "ssm_device.h"

namespace ssm {
namespace {

constexpr int kCB = 64;         // xproj_partial: channels per workgroup
constexpr int kThreads = 256;   // xproj_partial: threads per workgroup
// dt_decode: 32 quads (one channel each) per workgroup, so that the 7B-class slice's 2048
// channels run as 64 workgroups (0.3 us per token faster than 256 threads and 32 workgroups;
// 64 threads and 512 threads are 0.9 and 2.4 us slower).
constexpr int kDtThreads = 128;
constexpr int kDtCB = kDtThreads / 4;
constexpr int kNS = 16;         // d_state
constexpr int kMaxRows = SSM_FUSED_MAX_ROWS;

struct FusedArgs {
  const void* x;
  const void* z;  // nullable: no gate
  void* y;
  const float* A;
  const float* Dskip;
  const float* dt_bias;
  const float* conv_w;
  const float* conv_b;  // nullable
  float* h;
  float* conv;
  const void* wx;   // [M, D]
  const void* wdt;  // [D, R]
  float* part;      // [B, nblk, M]
  int64_t B, D;
  int R, M, nblk;  // nblk: xproj_partial's channel blocks
  int ndb;         // dt_decode's channel blocks
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Eight io values from 16 bytes at p (16-byte aligned).
template <typename IO>
__device__ __forceinline__ void load8(const IO* p, float (&v)[8]) {
  if constexpr (sizeof(IO) == 2) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// xproj_partial: a workgroup takes one batch row's block of 64 channels and 64 of the M rows,
// four threads per row (16 channels each; the four sums added across the quad), so that a call
// runs B x ceil(D / 64) x ceil(M / 64) workgroups of short loads (the 7B-class slice: 160; with
// one workgroup per channel block and one thread per row, 32 workgroups, 0.8 us slower per token).
constexpr int kRowsPerWG = kThreads / 4;
constexpr int kQuarter = kCB / 4;  // channels per thread

// VEC: D is a multiple of 8 and w_x 16-byte aligned, so a quarter row is whole 16-byte pieces.
// Every global load is issued before the barrier: the thread's two weight pieces and, on the
// first 64 threads, the conv front's inputs.
template <typename IO, bool VEC>
__global__ __launch_bounds__(kThreads) void xproj_partial(FusedArgs a) {
  __shared__ float us[kCB];
  const int nrb = (a.M + kRowsPerWG - 1) / kRowsPerWG;
  const int rb = (int)(blockIdx.x % (unsigned)nrb);
  const int64_t bb = blockIdx.x / (unsigned)nrb;
  const int64_t b = bb / a.nblk;
  const int blk = (int)(bb - b * a.nblk);
  const int t = threadIdx.x;
  const int r = rb * kRowsPerWG + (t >> 2), k = t & 3;
  const int rc = r < a.M ? r : a.M - 1;  // rows past M repeat the last one and store nothing
  const int64_t c0 = (int64_t)blk * kCB;
  const int ncb = (int)min((int64_t)kCB, a.D - c0);
  const bool full = VEC && ncb == kCB;
  // The quarter row as raw 16-byte pieces, unpacked only after the barrier, so that the loads
  // stay in flight with the conv front's.
  constexpr int kPer = 16 / (int)sizeof(IO);
  constexpr int kQP = kQuarter / kPer;
  u32x4 wraw[kQP];
  if (full) {
    const u32x4* wp =
        reinterpret_cast<const u32x4*>(static_cast<const IO*>(a.wx) + (int64_t)rc * a.D + c0 + kQuarter * k);
#pragma unroll
    for (int i = 0; i < kQP; ++i) wraw[i] = wp[i];
  }
  if (t < kCB) {
    float u = 0.0f;
    if (t < ncb) {
      const int64_t c = c0 + t, row = b * a.D + c;
      const float* cv = a.conv + row * 3;
      const float4 w = *reinterpret_cast<const float4*>(a.conv_w + c * 4);
      const float cb = a.conv_b ? a.conv_b[c] : 0.0f;
      const float xt = to_f32(static_cast<const IO*>(a.x)[row]);
      // The standalone conv front's order (ssm_conv.hip), then the io rounding of the stored u.
      const float v = fmaf(w.w, xt, fmaf(w.z, cv[2], fmaf(w.y, cv[1], fmaf(w.x, cv[0], cb))));
      u = to_f32(from_f32<IO>(silu(v)));
    }
    us[t] = u;
  }
  __syncthreads();
  float acc = 0.0f;
  if (full) {
#pragma unroll
    for (int i = 0; i < kQP; ++i) {
      float v[kPer];
      if constexpr (sizeof(IO) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = __uint_as_float(wraw[i][e] << 16);
          v[2 * e + 1] = __uint_as_float(wraw[i][e] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(wraw[i][e]);
      }
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc = fmaf(v[e], us[kQuarter * k + kPer * i + e], acc);
    }
  } else {
    const IO* wr = static_cast<const IO*>(a.wx) + (int64_t)rc * a.D + c0;
    const int hi = min(kQuarter * k + kQuarter, ncb);
    for (int c = kQuarter * k; c < hi; ++c) acc = fmaf(to_f32(wr[c]), us[c], acc);
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  if (k == 0 && r < a.M) a.part[((int64_t)b * a.nblk + blk) * a.M + r] = acc;
}

constexpr int kPartBatch = 32;  // partial sums read together (one round trip for up to 2048 channels)
constexpr int kMaxQuarter = (kMaxRows - 2 * kNS + 3) / 4;  // a lane's share of a dt_proj row

// VEC: R is a multiple of 32 and w_dt 16-byte aligned, so each lane's quarter of a row is whole
// 16-byte pieces.  The channel's weights, state and inputs are loaded before the reduction of
// the partial sums, which they do not depend on.
template <typename IO, bool VEC>
__global__ __launch_bounds__(kDtThreads) void dt_decode(FusedArgs a) {
  __shared__ float rs[kMaxRows];
  const int64_t b = blockIdx.x / a.ndb;
  const int blk = (int)(blockIdx.x - b * a.ndb);
  const int t = threadIdx.x;
  const int q = t & 3;
  const int64_t c_raw = (int64_t)blk * kDtCB + (t >> 2);
  const bool live = c_raw < a.D;
  const int64_t c = live ? c_raw : a.D - 1;  // a ragged last block repeats the last channel, writes nothing
  const int quarter = (a.R + 3) / 4;
  const int r0 = q * quarter, r1 = min(a.R, r0 + quarter);
  const IO* wr = static_cast<const IO*>(a.wdt) + c * a.R;
  // The quarter row as raw 16-byte pieces, unpacked only where it is used (after the barrier),
  // so that its loads stay in flight with the others below.
  constexpr int kPer = 16 / (int)sizeof(IO);                 // weights per piece
  constexpr int kPieces = (kMaxQuarter + kPer - 1) / kPer;
  u32x4 wraw[VEC ? kPieces : 1];
  if (VEC) {
    const u32x4* wp = reinterpret_cast<const u32x4*>(wr + r0);
#pragma unroll
    for (int i = 0; i < kPieces; ++i)
      if (i * kPer < quarter) wraw[i] = wp[i];
  }
  const int64_t row = b * a.D + c;
  const float4 w = *reinterpret_cast<const float4*>(a.conv_w + c * 4);
  const float cb = a.conv_b ? a.conv_b[c] : 0.0f;
  const float dtb = a.dt_bias[c], dsk = a.Dskip[c];
  const float4 A4 = *reinterpret_cast<const float4*>(a.A + c * kNS + q * QS);
  const float4 h4 = *reinterpret_cast<const float4*>(a.h + row * kNS + q * QS);
  const float* cv = a.conv + row * 3;
  const float x0 = cv[0], x1 = cv[1], x2 = cv[2];
  const float xt = to_f32(static_cast<const IO*>(a.x)[row]);
  const float zt = to_f32(static_cast<const IO*>(a.z ? a.z : a.x)[row]);

  // This batch row's x_proj outputs: the blocks' partial sums in block order, rounded to io.
  // A thread sums outputs t, t + kDtThreads, ... (kOut of them), all their partials loaded
  // together, so the reads are one round trip per batch of partials (with clamped indices and
  // the values past the end dropped, so that no load sits under a branch).
  const float* pb = a.part + b * a.nblk * a.M;
  if constexpr (VEC) {
    // R a multiple of 32 and N = 16, so M is a multiple of 4: thread t sums outputs 4t .. 4t + 3,
    // each block's four partials one 16-byte load.
    const int j0 = 4 * t;
    const int jc = j0 < a.M ? j0 : a.M - 4;
    float4 s4 = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 0; k0 < a.nblk; k0 += kPartBatch) {
      float4 v[kPartBatch];
#pragma unroll
      for (int i = 0; i < kPartBatch; ++i) {
        const int64_t k = k0 + i < a.nblk ? k0 + i : a.nblk - 1;
        v[i] = *reinterpret_cast<const float4*>(pb + k * a.M + jc);
      }
#pragma unroll
      for (int i = 0; i < kPartBatch; ++i) {  // blocks in order, as the unfused x_proj sums them
        const bool in = k0 + i < a.nblk;
        s4.x += in ? v[i].x : 0.0f;
        s4.y += in ? v[i].y : 0.0f;
        s4.z += in ? v[i].z : 0.0f;
        s4.w += in ? v[i].w : 0.0f;
      }
    }
    if (j0 < a.M) {
      rs[j0] = to_f32(from_f32<IO>(s4.x));
      rs[j0 + 1] = to_f32(from_f32<IO>(s4.y));
      rs[j0 + 2] = to_f32(from_f32<IO>(s4.z));
      rs[j0 + 3] = to_f32(from_f32<IO>(s4.w));
    }
  } else {
    constexpr int kOut = (kMaxRows + kDtThreads - 1) / kDtThreads;
    int jc[kOut];
    float sj[kOut];
#pragma unroll
    for (int o = 0; o < kOut; ++o) {
      const int j = t + o * kDtThreads;
      jc[o] = j < a.M ? j : a.M - 1;
      sj[o] = 0.0f;
    }
    for (int k0 = 0; k0 < a.nblk; k0 += kPartBatch) {
      float v[kOut][kPartBatch];
#pragma unroll
      for (int i = 0; i < kPartBatch; ++i) {
        const int64_t k = k0 + i < a.nblk ? k0 + i : a.nblk - 1;
#pragma unroll
        for (int o = 0; o < kOut; ++o) v[o][i] = pb[k * a.M + jc[o]];
      }
#pragma unroll
      for (int i = 0; i < kPartBatch; ++i)  // blocks in order, as the unfused x_proj sums them
#pragma unroll
        for (int o = 0; o < kOut; ++o) sj[o] += k0 + i < a.nblk ? v[o][i] : 0.0f;
    }
#pragma unroll
    for (int o = 0; o < kOut; ++o)
      if (t + o * kDtThreads < a.M) rs[t + o * kDtThreads] = to_f32(from_f32<IO>(sj[o]));
  }
  __syncthreads();

  // dt_proj of channel c: lane q sums its quarter of the row, the quad adds the quarters.
  float dtp = 0.0f;
  if (VEC) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      if (i * kPer < quarter) {
        float v[kPer];
        if constexpr (sizeof(IO) == 2) {
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            v[2 * k] = __uint_as_float(wraw[i][k] << 16);
            v[2 * k + 1] = __uint_as_float(wraw[i][k] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) v[k] = __uint_as_float(wraw[i][k]);
        }
#pragma unroll
        for (int e = 0; e < kPer; ++e) dtp = fmaf(v[e], rs[r0 + i * kPer + e], dtp);
      }
    }
  } else {
    for (int r = r0; r < r1; ++r) dtp = fmaf(to_f32(wr[r]), rs[r], dtp);
  }
  const float dtr = to_f32(from_f32<IO>(quad_sum(dtp)));

  // The decode step of channel c (ssm_decode_step's arithmetic).
  float Bq[QS], Cq[QS];
#pragma unroll
  for (int n = 0; n < QS; ++n) {
    Bq[n] = rs[a.R + q * QS + n];
    Cq[n] = rs[a.R + kNS + q * QS + n];
  }
  float h[QS] = {h4.x, h4.y, h4.z, h4.w};
  const float r = decode_quad_step(w, cb, dtb, dsk, A4, x0, x1, x2, xt, dtr, zt, a.z != nullptr, Bq, Cq, h);
  if (!live) return;
  *reinterpret_cast<float4*>(a.h + row * kNS + q * QS) = make_float4(h[0], h[1], h[2], h[3]);
  if (q == 0) {
    static_cast<IO*>(a.y)[row] = from_f32<IO>(r);
    float* co = a.conv + row * 3;
    co[0] = x1;
    co[1] = x2;
    co[2] = xt;
  }
}

template <typename IO>
hipError_t launch(const FusedArgs& a, bool vec_x, bool vec_dt, hipStream_t s) {
  const dim3 xgrid((unsigned)(a.B * a.nblk * ((a.M + kRowsPerWG - 1) / kRowsPerWG))), xblock(kThreads);
  const dim3 dgrid((unsigned)(a.B * a.ndb)), dblock(kDtThreads);
  if (vec_x) xproj_partial<IO, true><<<xgrid, xblock, 0, s>>>(a);
  else xproj_partial<IO, false><<<xgrid, xblock, 0, s>>>(a);
  if (vec_dt) dt_decode<IO, true><<<dgrid, dblock, 0, s>>>(a);
  else dt_decode<IO, false><<<dgrid, dblock, 0, s>>>(a);
  return hipGetLastError();
}

struct Span {
  uintptr_t lo, hi;
};
Span span(const void* p, int64_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Span{lo, p ? lo + (uintptr_t)bytes : lo};
}
bool overlaps(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }
bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

// Sizes of one call, or false when they are invalid.
bool fused_sizes(const ssm_dims* d, int64_t rank, int64_t* nblk, int64_t* ws_bytes) {
  if (!d || d->batch < 1 || d->d_inner < 1 || d->d_inner > SSM_MAX_D_INNER || d->d_state != kNS ||
      d->d_conv != SSM_CONV_WIDTH || rank < 1 || rank + 2 * kNS > kMaxRows)
    return false;
  *nblk = (d->d_inner + kCB - 1) / kCB;
  const int64_t nrb = (rank + 2 * kNS + kRowsPerWG - 1) / kRowsPerWG;  // x_proj row blocks
  int64_t t;
  const int64_t ndb = (d->d_inner + kDtCB - 1) / kDtCB;  // dt_decode's channel blocks
  if (__builtin_mul_overflow(d->batch, *nblk, &t) || t * nrb >= ((int64_t)1 << 31) ||
      d->batch * ndb >= ((int64_t)1 << 31) ||
      __builtin_mul_overflow(t, (rank + 2 * kNS) * 4, ws_bytes) ||
      __builtin_mul_overflow(d->batch, d->d_inner * kNS * 4, &t))
    return false;
  return true;
}

// The no-allocation entry point's scratch: one array per GPU in this code object, loaded with
// it and held until the process ends.  Host code never uses its name as an address (in host
// code it is a stand-in for the device symbol): the device address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept per device.
constexpr size_t kScratchBytes = SSM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipErrorUnknown;
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's scratch address (looked up on its first use), or nullptr.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&s] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  return s.err == hipSuccess ? s.ptr : nullptr;
}

// Validation and launch shared by both entry points; ws == nullptr means the device scratch.
ssm_status decode_fused(const ssm_dims* d, const ssm_params* p, const void* w_x, const void* w_dt, int64_t rank,
                        const void* x_t, const void* z_t, void* y_t, float* h, float* conv_state, void* workspace,
                        size_t workspace_bytes, bool use_scratch, void* stream) {
  if (!d) return SSM_ERR_NULL;
  int64_t nblk, ws_bytes;
  if (!fused_sizes(d, rank, &nblk, &ws_bytes)) return SSM_ERR_SHAPE;
  if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (!p || !p->A || !p->Dskip || !p->dt_bias || !p->conv_w || !w_x || !w_dt || !x_t || !y_t || !h || !conv_state)
    return SSM_ERR_NULL;
  if (use_scratch) {
    if ((size_t)ws_bytes > kScratchBytes) return SSM_ERR_SCRATCH;
  } else if (!workspace || workspace_bytes < (size_t)ws_bytes) {
    return SSM_ERR_WORKSPACE;
  }
  const int64_t B = d->batch, D = d->d_inner, M = rank + 2 * kNS;
  const int64_t es = d->io_dtype == SSM_BF16 ? 2 : 4;
  const int64_t tok = B * D * es;
  const void* ins[9] = {x_t, z_t, w_x, w_dt, p->A, p->Dskip, p->dt_bias, p->conv_w, p->conv_b};
  const int64_t in_bytes[9] = {tok, tok, M * D * es, D * rank * es, D * kNS * 4, D * 4, D * 4, D * 16, D * 4};
  const uintptr_t in_align[9] = {(uintptr_t)es, (uintptr_t)es, (uintptr_t)es, (uintptr_t)es, 16, 4, 4, 16, 4};
  const int nouts = use_scratch ? 3 : 4;
  void* outs[4] = {y_t, h, conv_state, workspace};
  const int64_t out_bytes[4] = {tok, B * D * kNS * 4, B * D * 3 * 4, ws_bytes};
  const uintptr_t out_align[4] = {(uintptr_t)es, 16, 4, 4};
  for (int i = 0; i < 9; ++i)
    if (ins[i] && !aligned(ins[i], in_align[i])) return SSM_ERR_ALIGN;
  for (int o = 0; o < nouts; ++o)
    if (!aligned(outs[o], out_align[o])) return SSM_ERR_ALIGN;
  for (int o = 0; o < nouts; ++o) {
    for (int i = 0; i < 9; ++i)
      if (overlaps(span(outs[o], out_bytes[o]), span(ins[i], in_bytes[i]))) return SSM_ERR_ALIAS;
    for (int q = o + 1; q < nouts; ++q)
      if (overlaps(span(outs[o], out_bytes[o]), span(outs[q], out_bytes[q]))) return SSM_ERR_ALIAS;
  }
  if (use_scratch) {
    workspace = device_scratch();
    if (!workspace) return SSM_ERR_LAUNCH;
  }
  FusedArgs a;
  memset(&a, 0, sizeof a);
  a.x = x_t;
  a.z = z_t;
  a.y = y_t;
  a.A = p->A;
  a.Dskip = p->Dskip;
  a.dt_bias = p->dt_bias;
  a.conv_w = p->conv_w;
  a.conv_b = p->conv_b;
  a.h = h;
  a.conv = conv_state;
  a.wx = w_x;
  a.wdt = w_dt;
  a.part = static_cast<float*>(workspace);
  a.B = B;
  a.D = D;
  a.R = (int)rank;
  a.M = (int)M;
  a.nblk = (int)nblk;
  a.ndb = (int)((D + kDtCB - 1) / kDtCB);
  const bool vec_x = D % 8 == 0 && aligned(w_x, 16);
  const bool vec_dt = rank % 32 == 0 && aligned(w_dt, 16) && aligned(workspace, 16);  // 16-byte partial loads
  (void)hipGetLastError();  // drop a stale error so a launch failure is reported as ours
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = d->io_dtype == SSM_BF16 ? launch<bf16_t>(a, vec_x, vec_dt, s) : launch<float>(a, vec_x, vec_dt, s);
  return e == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}

}  // namespace
}  // namespace ssm

extern "C" {

size_t ssm_decode_fused_workspace_bytes(const ssm_dims* d, int64_t rank) {
  int64_t nblk, ws;
  return ssm::fused_sizes(d, rank, &nblk, &ws) ? (size_t)ws : 0;
}

ssm_status ssm_decode_fused(const ssm_dims* d, const ssm_params* p, const void* w_x, const void* w_dt, int64_t rank,
                            const void* x_t, const void* z_t, void* y_t, float* h, float* conv_state,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return ssm::decode_fused(d, p, w_x, w_dt, rank, x_t, z_t, y_t, h, conv_state, workspace, workspace_bytes, false,
                           stream);
}

ssm_status ssm_decode_fused_noalloc(const ssm_dims* d, const ssm_params* p, const void* w_x, const void* w_dt,
                                    int64_t rank, const void* x_t, const void* z_t, void* y_t, float* h,
                                    float* conv_state, void* stream) {
  return ssm::decode_fused(d, p, w_x, w_dt, rank, x_t, z_t, y_t, h, conv_state, nullptr, 0, true, stream);
}

}  // extern "C"
