// ssm_conv_xproj.hip -- ssm_conv_xproj of include/ssm_proj.h: the conv front fused into the
// projection that reads it ("Scaling State-Space Models on Multiple GPUs with Tensor
// Parallelism", euno.news summary of arXiv 2602.21144, Methodology item 1: the local mixing
// kernels and the channel-sliced projections of one GPU).
//
//   out[b, t, m] = sum_c W[m, c] * u[b, c, t],   u = bf16(silu(conv(x)))   (never stored)
//
// with m over the stacked rows of W: the low-rank step input (rank rows), then B (N rows),
// then C (N rows); each row group lands in its own token-major tensor.
//
// One workgroup (8 waves) owns 128 tokens of one batch row and up to 320 output rows, and
// walks the channels in steps of 64.  Per step, double-buffered in LDS:
//   - every thread computes 8 tokens of u for two channels (c and c + 32) from x, with the
//     arithmetic, in the same order, of the conv front kernel, rounds it to bf16 (nearest
//     even) and writes it transposed, [token][channel]; the 32 lanes of a half-wave take 32
//     channels of one token group, so these 2-byte writes fill distinct banks.  Each lane
//     reads its own channel row (one 16-byte load plus the 8 bytes before it for the conv
//     history), so x is read with plain global loads: a buffer view needs one base per wave;
//   - the W rows of the step's 64 channels are staged as they are, [row][channel];
//   - wave w multiplies its 32-token block (w & 3) by the row blocks w >> 2, w >> 2 + 2, ... of
//     32 rows on the matrix cores: v_mfma_f32_32x32x16_bf16, fp32 accumulation, four per row
//     block per step.  Operand fragments are 16-byte LDS reads: lane l takes row l % 32 and
//     channels 8 (l / 32) .. + 7 of both tiles; the padded row pitch (144 bytes) keeps them
//     free of bank conflicts.  Rows past M are zero in the W tile, so the products are
//     unconditional (a guard per block made each product wait for its operand read).
// The next step's x, conv weights and W are loaded into registers while the current step
// multiplies.  The sums are rounded to bf16 (nearest even) once, at the end.
#include <string.h>

#include "../../include/ssm_proj.h"
#include "ssm_device.h"

namespace ssm {
namespace {

constexpr int TT = 128;                    // tokens per workgroup
constexpr int KC = 64;                     // channels per step
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;
constexpr int MB = 10;                     // row blocks of 32 per workgroup (320 rows)
constexpr int ROWS = MB * 32;
constexpr int PITCH = KC + 8;              // bf16 per LDS row (144 bytes)
constexpr int WCHUNKS = ROWS * KC / 8;     // 16-byte chunks of a W step tile
constexpr int WPT = (WCHUNKS + THREADS - 1) / THREADS;
constexpr int MB_PER_WAVE = MB / 2;        // row blocks per wave (two row-block sets)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct XprojArgs {
  const void* x;        // [B, D, L] bf16
  const float* conv_w;  // [D, 4]
  const float* conv_b;  // [D] or null
  const float* conv0;   // [B, D, 3] or null
  const void* w;        // [M, D] bf16
  void* out0;           // [B, L, R]
  void* out1;           // [B, L, N]
  void* out2;           // [B, L, N]
  int64_t B, L, D;
  int M, R, N;
};

struct Tiles {
  uint16_t u[2][TT * PITCH];
  uint16_t w[2][ROWS * PITCH];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr int CPT = KC / 32;  // channels per thread (c and c + 32)

// One thread's share of a step's loads: 8 tokens (plus the 4 before) of channels c and c + 32
// of x with their conv weights, and up to WPT 16-byte chunks of W.
struct StepRegs {
  u32x4 xv[CPT];
  u32x2 xh[CPT];
  float4 cw[CPT];
  float cb[CPT];
  u32x4 wv[WPT];
};

__device__ __forceinline__ void load_step(const XprojArgs& a, int64_t b, int64_t t0, int64_t k0, int m0,
                                          StepRegs& r) {
  const int g = threadIdx.x >> 5;
#pragma unroll
  for (int h = 0; h < CPT; ++h) {
    const int c = (threadIdx.x & 31) + 32 * h;
    const int64_t ch = k0 + c;
    r.xv[h] = u32x4{0u, 0u, 0u, 0u};
    r.xh[h] = u32x2{0u, 0u};
    r.cw[h] = float4{0.0f, 0.0f, 0.0f, 0.0f};
    r.cb[h] = 0.0f;
    if (ch < a.D) {
      r.cw[h] = *reinterpret_cast<const float4*>(a.conv_w + ch * 4);
      r.cb[h] = a.conv_b ? a.conv_b[ch] : 0.0f;
      // L and t are multiples of 8: a group of 8 tokens is wholly inside or past the row end,
      // and both loads are naturally aligned.
      const uint16_t* xr = static_cast<const uint16_t*>(a.x) + (b * a.D + ch) * a.L;
      const int64_t t = t0 + 8 * g;
      if (t < a.L) r.xv[h] = *reinterpret_cast<const u32x4*>(xr + t);
      if (t > 0 && t < a.L) r.xh[h] = *reinterpret_cast<const u32x2*>(xr + t - 4);
    }
  }
  const auto rw = rsrc(a.w, (int64_t)a.M * a.D * 2);
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int ci = threadIdx.x + i * THREADS;  // chunk: row ci / (KC / 8), channels 8 (ci % (KC / 8)) ..
    const int row = m0 + ci / (KC / 8), q = ci % (KC / 8);
    r.wv[i] = u32x4{0u, 0u, 0u, 0u};
    if (ci < WCHUNKS && row < a.M && k0 + 8 * q < a.D)
      r.wv[i] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(((int64_t)row * a.D + k0 + 8 * q) * 2), 0, 0);
  }
}

// u for this thread's 8 tokens of its two channels, bf16, into the transposed tile; W chunks
// into the W tile.
__device__ __forceinline__ void stage_step(const XprojArgs& a, int64_t b, int64_t t0, int64_t k0, const StepRegs& r,
                                           uint16_t* ut, uint16_t* wt) {
  const int g = threadIdx.x >> 5;
#pragma unroll
  for (int h = 0; h < CPT; ++h) {
    const int c = (threadIdx.x & 31) + 32 * h;
    const int64_t ch = k0 + c;
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    if (ch < a.D) {
      float xv[11];  // xv[0..2] = raw inputs t-3 .. t-1, xv[3 + j] = token t + j
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        xv[3 + 2 * k] = __uint_as_float(r.xv[h][k] << 16);
        xv[4 + 2 * k] = __uint_as_float(r.xv[h][k] & 0xFFFF0000u);
      }
      const int64_t t = t0 + 8 * g;
      if (t > 0) {
        xv[0] = __uint_as_float(r.xh[h][0] & 0xFFFF0000u);
        xv[1] = __uint_as_float(r.xh[h][1] << 16);
        xv[2] = __uint_as_float(r.xh[h][1] & 0xFFFF0000u);
      } else {
#pragma unroll
        for (int j = 0; j < 3; ++j) xv[j] = a.conv0 ? a.conv0[(b * a.D + ch) * 3 + j] : 0.0f;
      }
      const float4 w4 = r.cw[h];
      const float cb = r.cb[h];
      float uv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = fmaf(w4.w, xv[3 + j], fmaf(w4.z, xv[2 + j], fmaf(w4.y, xv[1 + j], fmaf(w4.x, xv[j], cb))));
        uv[j] = silu(v);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k)
        asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(o[k]) : "v"(uv[2 * k]), "v"(uv[2 * k + 1]));
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ut[(8 * g + j) * PITCH + c] = (uint16_t)(o[j >> 1] >> (16 * (j & 1)));
  }
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int ci = threadIdx.x + i * THREADS;
    if (ci < WCHUNKS) *reinterpret_cast<u32x4*>(&wt[(ci / (KC / 8)) * PITCH + 8 * (ci % (KC / 8))]) = r.wv[i];
  }
}

__global__ __launch_bounds__(THREADS) void conv_xproj_kernel(XprojArgs a) {
  __shared__ __attribute__((aligned(16))) Tiles tl;
  const int64_t tiles_per_row = (a.L + TT - 1) / TT;
  const int64_t b = blockIdx.x / tiles_per_row;
  const int64_t t0 = (blockIdx.x - b * tiles_per_row) * TT;
  const int m0 = blockIdx.y * ROWS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tb = wave & 3, mset = wave >> 2;
  const int nsteps = (int)((a.D + KC - 1) / KC);

  f32x16 acc[MB_PER_WAVE];
#pragma unroll
  for (int i = 0; i < MB_PER_WAVE; ++i) acc[i] = f32x16{};

  StepRegs r;
  load_step(a, b, t0, 0, m0, r);
  stage_step(a, b, t0, 0, r, tl.u[0], tl.w[0]);
  __syncthreads();
  const int frow = lane & 31, fk = 8 * (lane >> 5);
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    const bool more = s + 1 < nsteps;
    if (more) load_step(a, b, t0, (int64_t)(s + 1) * KC, m0, r);
#pragma unroll
    for (int ks = 0; ks < KC / 16; ++ks) {
      const bf16x8 bu = *reinterpret_cast<const bf16x8*>(&tl.u[cur][(32 * tb + frow) * PITCH + 16 * ks + fk]);
      bf16x8 aw[MB_PER_WAVE];  // rows past M are zero in the tile: their products are dropped at the end
#pragma unroll
      for (int i = 0; i < MB_PER_WAVE; ++i)
        aw[i] = *reinterpret_cast<const bf16x8*>(&tl.w[cur][(32 * (mset + 2 * i) + frow) * PITCH + 16 * ks + fk]);
#pragma unroll
      for (int i = 0; i < MB_PER_WAVE; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[i], bu, acc[i], 0, 0, 0);
    }
    if (more) stage_step(a, b, t0, (int64_t)(s + 1) * KC, r, tl.u[cur ^ 1], tl.w[cur ^ 1]);
    __syncthreads();
  }

  // acc[i] register j: row 32 blk + 8 (j / 4) + 4 (lane / 32) + j % 4, token 32 tb + lane % 32.
  const int64_t t = t0 + 32 * tb + (lane & 31);
  if (t >= a.L) return;
  const int64_t row_tok = b * a.L + t;  // one token row per lane: plain global stores
  uint16_t* o0 = static_cast<uint16_t*>(a.out0) + row_tok * a.R;
  uint16_t* o1 = static_cast<uint16_t*>(a.out1) + row_tok * a.N;
  uint16_t* o2 = static_cast<uint16_t*>(a.out2) + row_tok * a.N;
#pragma unroll
  for (int i = 0; i < MB_PER_WAVE; ++i) {
    const int blk = mset + 2 * i;
    if (m0 + 32 * blk >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const int m = m0 + 32 * blk + 8 * (j / 4) + 4 * (lane >> 5) + j % 4;  // m and m + 1
      uint32_t pk;
      asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(pk) : "v"(acc[i][j]), "v"(acc[i][j + 1]));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int mm = m + h;
        const unsigned short v = (unsigned short)(pk >> (16 * h));
        if (mm < a.R) o0[mm] = v;
        else if (mm < a.R + a.N) o1[mm - a.R] = v;
        else if (mm < a.M) o2[mm - a.R - a.N] = v;
      }
    }
  }
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }
bool overlaps(const void* p, int64_t np, const void* q, int64_t nq) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(q);
  return a0 < b0 + (uintptr_t)nq && b0 < a0 + (uintptr_t)np;
}

}  // namespace
}  // namespace ssm

extern "C" int ssm_conv_xproj(const ssm_dims* d, const ssm_params* p, const void* x, const float* conv0, const void* w,
                              int64_t rank, void* lowrank, void* Bm, void* Cm, void* stream) {
  using namespace ssm;
  if (!d || !p || !p->conv_w || !x || !w || !lowrank || !Bm || !Cm) return SSM_ERR_NULL;
  if (d->batch < 1 || d->seqlen < 1 || d->d_inner < 1 || d->d_conv != SSM_CONV_WIDTH || d->d_state < 1 ||
      d->d_state > SSM_MAX_STATE || rank < 1 || d->d_inner % 8 != 0 || d->seqlen % 8 != 0)
    return SSM_ERR_SHAPE;
  if (d->io_dtype != SSM_BF16) return SSM_ERR_DTYPE;
  if (rank > ((int64_t)1 << 20)) return SSM_ERR_SHAPE;
  const int64_t M = rank + 2 * d->d_state;
  // Per-row buffer views are 32-bit: a channel row of x, the whole of W and one token's row of
  // each output must stay below 2 GiB; the grid holds batch * ceil(L / 128) workgroups.
  int64_t rows, xbytes, tok, ob0, ob1;
  if (__builtin_mul_overflow(d->batch, d->d_inner, &rows) || __builtin_mul_overflow(rows, d->seqlen, &xbytes) ||
      __builtin_mul_overflow(xbytes, (int64_t)2, &xbytes) || __builtin_mul_overflow(d->batch, d->seqlen, &tok) ||
      __builtin_mul_overflow(tok, rank * 2, &ob0) || __builtin_mul_overflow(tok, d->d_state * 2, &ob1) ||
      d->seqlen * 2 >= ((int64_t)1 << 31) - 2 * TT || M * d->d_inner * 2 >= ((int64_t)1 << 31) ||
      d->batch > INT32_MAX / ((d->seqlen + TT - 1) / TT))
    return SSM_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(p->conv_w, 16) || (p->conv_b && !aligned(p->conv_b, 4)) ||
      (conv0 && !aligned(conv0, 4)) || !aligned(lowrank, 2) || !aligned(Bm, 2) || !aligned(Cm, 2))
    return SSM_ERR_ALIGN;
  const void* ins[3] = {x, w, conv0};
  const int64_t inb[3] = {xbytes, M * d->d_inner * 2, rows * 3 * 4};
  const void* outs[3] = {lowrank, Bm, Cm};
  const int64_t outb[3] = {ob0, ob1, ob1};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 3; ++i)
      if (ins[i] && overlaps(outs[o], outb[o], ins[i], inb[i])) return SSM_ERR_ALIAS;
    for (int q = o + 1; q < 3; ++q)
      if (overlaps(outs[o], outb[o], outs[q], outb[q])) return SSM_ERR_ALIAS;
  }
  XprojArgs a;
  memset(&a, 0, sizeof a);
  a.x = x;
  a.conv_w = p->conv_w;
  a.conv_b = p->conv_b;
  a.conv0 = conv0;
  a.w = w;
  a.out0 = lowrank;
  a.out1 = Bm;
  a.out2 = Cm;
  a.B = d->batch;
  a.L = d->seqlen;
  a.D = d->d_inner;
  a.M = (int)M;
  a.R = (int)rank;
  a.N = (int)d->d_state;
  const dim3 grid((unsigned)(d->batch * ((d->seqlen + TT - 1) / TT)), (unsigned)((M + ROWS - 1) / ROWS)),
      block(THREADS);
  (void)hipGetLastError();
  conv_xproj_kernel<<<grid, block, 0, static_cast<hipStream_t>(stream)>>>(a);
  return hipGetLastError() == hipSuccess ? SSM_OK : SSM_ERR_LAUNCH;
}
