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
//     reads its own channel row (one 16-byte load through a buffer view of the step's 64 rows,
//     plus the 12 bytes before it, or the cache at a row's start, for the conv history);
//   - the W rows of the step's 64 channels are staged as they are, [row][channel], by loads that
//     write LDS directly (no registers, no stores);
//   - wave w multiplies its 32-token block (w & 3) by the row blocks w >> 2, w >> 2 + 2, ... of
//     32 rows on the matrix cores: v_mfma_f32_32x32x16_bf16, fp32 accumulation, four per row
//     block per step.  Operand fragments are 16-byte LDS reads: lane l takes row l % 32 and
//     channels 8 (l / 32) .. + 7 of both tiles; the padded row pitch (144 bytes) keeps them
//     free of bank conflicts.  The products are unconditional (a guard per block made each product
//     wait for its operand read): rows past M feed only outputs that are not stored.
// The steps are software-pipelined so that the loads, the conv front and the products of
// different steps overlap instead of running in turn:
//   - x (with its conv weights) is loaded two steps ahead into one of two register sets, W one
//     step ahead straight into the other W tile;
//   - while a wave multiplies step s, it computes u of step s + 1 into the other u tile, a
//     quarter after each of the four 16-channel slices of products (the matrix cores run a
//     product while the vector units compute); one barrier per step.
// Loads are unconditional within a wave (indices clamped into the tensors; u past D is zeroed
// where it is made, and W past D or M holds copies of in-range weights that meet u = 0 or feed
// dropped rows), so no lane branches around a load; the step's conv weights are loaded and
// stored by the first wave alone (a wave-uniform branch: seven of eight waves issue no load for
// them).  The clamps, the cache history and the zeroing past D are compiled only into the general
// form of the loop, which runs in the first workgroup of each batch row (whose first group
// starts the row) and, when D is not a multiple of 64, in every workgroup; the others run a form
// whose x and W offsets are the same in every step (W's step offset is a scalar operand) and
// whose conv history is the 4 raw inputs before each group.  The sums are rounded to bf16 (nearest even) once,
// at the end, staged through LDS and written as whole 16-byte pieces of the output rows.
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
constexpr int WROW_SLOTS = PITCH * 2 / 16;  // 16-byte slots per W tile row: 8 of data, 1 of padding
constexpr int WPT = (ROWS * WROW_SLOTS + THREADS - 1) / THREADS;  // slots each thread loads per step
constexpr int WSLOTS = WPT * THREADS;         // slots per W tile (the last ones past the rows are spare)
constexpr int MB_PER_WAVE = MB / 2;        // row blocks per wave (two row-block sets)
constexpr int OPITCH = ROWS + 8;           // bf16 per token row of the output staging tile
static_assert(WROW_SLOTS * 16 == PITCH * 2, "a W tile row is a whole number of 16-byte slots");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x3 __attribute__((ext_vector_type(3), aligned(4)));
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

// The W tile of one step ([ROWS][PITCH] rows, then spare slots).  The two W tiles are separate
// LDS objects, so that the compiler can tell the tile being filled from memory apart from the one
// being read: it waits for the fill only where the filled tile is read (a single object of two
// tiles made it wait at the first fragment read of every step).
struct WTile {
  uint16_t w[WSLOTS * 8];
};
struct Tiles {
  uint16_t u[2][TT * PITCH];
  float c[2][5 * KC];  // conv weights of a step: [KC] float4 taps, then [KC] biases
};
constexpr int HALF_TT = TT / 2;
static_assert(sizeof(uint16_t) * HALF_TT * OPITCH <= sizeof(WTile), "half the output staging must fit in a W tile");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr int CPT = KC / 32;  // channels per thread (c and c + 32)

// One thread's x for one step: 8 tokens of channels c and c + 32 and the history before them:
// the 6 raw inputs before the group (bf16 pairs, of which the last 3 are used) or, for a row's
// first group, the 3 cached inputs (fp32).
struct XRegs {
  u32x4 xv[CPT];
  u32x3 xh[CPT];
};

// The conv taps and bias of one channel of a step, on their way to LDS.
struct WRegs {
  u32x4 cv;
  uint32_t cb;
};


// Every thread issues the same loads in every step (no load sits under a branch), so that the
// wait for a set loaded two steps ago leaves the later loads in flight.  HEAD: the workgroup's
// first group may start a row (t0 = 0); RAG: the step may hold channels past D.
template <bool HEAD, bool RAG>
__device__ __forceinline__ void load_x(const XprojArgs& a, int64_t b, int64_t t0, int64_t k0, XRegs& r) {
  const int g = threadIdx.x >> 5;
  const int64_t t = t0 + 8 * g;
  // L and t are multiples of 8: a group of 8 tokens is wholly inside or past the row end, and
  // the loads are naturally aligned.  Past the end the group reads the row's last 8 tokens.
  const int64_t tl = t < a.L ? t : a.L - 8;
  const bool head = t == 0 && a.conv0 != nullptr;  // history from the cache
  // the step's block of channel rows through a buffer view (uniform base, 32-bit lane offsets;
  // the offsets stay inside it, clamped as above)
  const int rows = !RAG ? KC : a.D - k0 < KC ? (int)(a.D - k0) : KC;
  const auto rx = rsrc(static_cast<const char*>(a.x) + (b * a.D + k0) * a.L * 2, (int64_t)rows * a.L * 2);
#pragma unroll
  for (int h = 0; h < CPT; ++h) {
    const int c = (threadIdx.x & 31) + 32 * h;
    const int cc = !RAG ? c : c < rows ? c : rows - 1;
    // raw values: channels past D give u = 0 in conv_piece, tokens past L only outputs that
    // are not stored
    r.xv[h] = __builtin_amdgcn_raw_buffer_load_b128(rx, (cc * (int)a.L + (int)tl) * 2, 0, 0);
    if constexpr (!HEAD) {
      // no group of this workgroup starts a row (t0 >= 128, so tl >= 120): the history is the
      // raw inputs before it (the last 3 of the 4 read are used)
      const u32x2 hv = __builtin_amdgcn_raw_buffer_load_b64(rx, (cc * (int)a.L + (int)tl - 4) * 2, 0, 0);
      r.xh[h][1] = hv[0];
      r.xh[h][2] = hv[1];
      continue;
    }
    // one load from one of two places (an address select, not a branch)
    const uintptr_t px = reinterpret_cast<uintptr_t>(static_cast<const char*>(a.x) + (b * a.D + k0) * a.L * 2) +
                         (uint32_t)((cc * (int)a.L + (tl >= 6 ? (int)tl - 6 : 0)) * 2);
    const uintptr_t pc = reinterpret_cast<uintptr_t>(a.conv0) + (uint64_t)((b * a.D + k0 + cc) * 12);
    r.xh[h] = *reinterpret_cast<const __attribute__((address_space(1))) u32x3*>(head ? pc : px);
  }
}

// W of step k0 (rows m0 ..) straight from memory into the tile wt (16-byte loads that write LDS
// directly: lane i of a wave's load fills slot base + i).  Slot j of the tile is row j / 9, chunk
// j % 9 (chunk 8 is the row's padding, and slots past the last row are spare: both take a copy of
// an in-range chunk).  Reads are clamped into W: rows past M hold copies of row M - 1 and feed only
// output rows that are never stored; chunks past D hold copies of the row's last in-range chunk,
// multiplied by u = 0 there.  A slot's byte offset is its row's and chunk's part (the same in every
// step, computed once: WSlots) plus 2 k0, capped at its row's last chunk: one add and one min per
// slot and step, with no branch (a branch between a fast and a clamped form made the compiler
// wait for this step's W before the conv front's first use of x).
struct WSlots {
  int off[WPT];  // (row * D + 8 * chunk) * 2 of this thread's slots, chunk 8 taken as 7
  int lim[WPT];  // (row * D + D - 8) * 2: the row's last in-range chunk
};

__device__ __forceinline__ WSlots w_slots(const XprojArgs& a, int m0) {
  WSlots ws;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    const int slot = i * THREADS + 64 * wave + lane;
    const int row = slot / WROW_SLOTS, q = slot - row * WROW_SLOTS;
    const int rr = m0 + row < a.M ? m0 + row : a.M - 1;
    ws.off[i] = (rr * (int)a.D + 8 * (q < 8 ? q : 7)) * 2;
    ws.lim[i] = (rr * (int)a.D + (int)a.D - 8) * 2;
  }
  return ws;
}

template <bool RAG>
__device__ __forceinline__ void dma_w(const XprojArgs& a, int64_t k0, const WSlots& ws, uint16_t* wt) {
  // 32-bit offsets: the caller keeps W below 2 GiB
  const auto rw = rsrc(a.w, (int64_t)a.M * a.D * 2);
  const int k2 = 2 * (int)k0;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int i = 0; i < WPT; ++i) {
    if constexpr (RAG) {
      const int o = ws.off[i] + k2 < ws.lim[i] ? ws.off[i] + k2 : ws.lim[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(wt + (i * THREADS + 64 * wave) * 8),
                                               16, o, 0, 0, 0);
    } else {
      // D a multiple of KC: every chunk of every step is in range (off + 2 k0 <= lim)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (__attribute__((address_space(3))) void*)(wt + (i * THREADS + 64 * wave) * 8),
                                               16, ws.off[i], k2, 0, 0);
    }
  }
}

// The conv weights of step kc: thread t reads channel kc + t % KC's taps (float4) and bias
// (clamped past D, and without a bias the taps are read again).
template <bool RAG>
__device__ __forceinline__ void load_cw(const XprojArgs& a, int64_t kc, WRegs& r) {
  const int last = (int)(a.D - 1 - kc);  // channels kc .. kc + last exist
  const int i = threadIdx.x % KC;
  const int ii = !RAG ? i : i <= last ? i : last;
  const auto rw = rsrc(a.conv_w + kc * 4, (int64_t)(last + 1) * 16);
  r.cv = __builtin_amdgcn_raw_buffer_load_b128(rw, ii * 16, 0, 0);
  const auto rb = a.conv_b ? rsrc(a.conv_b + kc, (int64_t)(last + 1) * 4) : rw;
  r.cb = __builtin_amdgcn_raw_buffer_load_b32(rb, ii * 4, 0, 0);
}

// Threads 0 .. KC - 1 store their channel's taps and bias ([KC] float4, then [KC] float).
template <bool RAG>
__device__ __forceinline__ void store_cw(const XprojArgs& a, int64_t kc, const WRegs& r, float* ct) {
  const int t = threadIdx.x;
  if (t < KC) {
    const bool ok = !RAG || t <= (int)(a.D - 1 - kc);
    *reinterpret_cast<u32x4*>(&ct[4 * t]) = ok ? r.cv : u32x4{0u, 0u, 0u, 0u};
    ct[4 * KC + t] = ok && a.conv_b ? __uint_as_float(r.cb) : 0.0f;
  }
}

// The conv taps and biases of this thread's two channels for one step.
struct ConvW {
  float4 w[CPT];
  float b[CPT];
};

__device__ __forceinline__ ConvW read_convw(const float* ct) {
  ConvW q;
#pragma unroll
  for (int h = 0; h < CPT; ++h) {
    const int c = (threadIdx.x & 31) + 32 * h;
    q.w[h] = *reinterpret_cast<const float4*>(&ct[4 * c]);
    q.b[h] = ct[4 * KC + c];
  }
  return q;
}

// u of tokens 4 HALF .. 4 HALF + 3 of this thread's channel H, bf16, into the transposed tile
// (nch: channels of the step below D).
template <int H, int HALF, bool HEAD, bool RAG>
__device__ __forceinline__ void conv_piece(const XRegs& r, const ConvW& q, bool head, bool cache, int nch,
                                           uint16_t* ut) {
  const int g = threadIdx.x >> 5;
  const int c = (threadIdx.x & 31) + 32 * H;
  float xv[7];  // raw inputs at window positions 4 HALF .. 4 HALF + 6 (positions 0..2 precede the group)
  if (HALF == 0) {
    // a row's first group (head) takes the cached inputs (zero without a cache); the others
    // tokens t - 3 .. t - 1: the high half of the second pair and the third pair
    if constexpr (HEAD) {
      xv[0] = head ? (cache ? __uint_as_float(r.xh[H][0]) : 0.0f) : __uint_as_float(r.xh[H][1] & 0xFFFF0000u);
      xv[1] = head ? (cache ? __uint_as_float(r.xh[H][1]) : 0.0f) : __uint_as_float(r.xh[H][2] << 16);
      xv[2] = head ? (cache ? __uint_as_float(r.xh[H][2]) : 0.0f) : __uint_as_float(r.xh[H][2] & 0xFFFF0000u);
    } else {
      xv[0] = __uint_as_float(r.xh[H][1] & 0xFFFF0000u);
      xv[1] = __uint_as_float(r.xh[H][2] << 16);
      xv[2] = __uint_as_float(r.xh[H][2] & 0xFFFF0000u);
    }
    xv[3] = __uint_as_float(r.xv[H][0] << 16);
    xv[4] = __uint_as_float(r.xv[H][0] & 0xFFFF0000u);
    xv[5] = __uint_as_float(r.xv[H][1] << 16);
    xv[6] = __uint_as_float(r.xv[H][1] & 0xFFFF0000u);
  } else {
    xv[0] = __uint_as_float(r.xv[H][0] & 0xFFFF0000u);
    xv[1] = __uint_as_float(r.xv[H][1] << 16);
    xv[2] = __uint_as_float(r.xv[H][1] & 0xFFFF0000u);
    xv[3] = __uint_as_float(r.xv[H][2] << 16);
    xv[4] = __uint_as_float(r.xv[H][2] & 0xFFFF0000u);
    xv[5] = __uint_as_float(r.xv[H][3] << 16);
    xv[6] = __uint_as_float(r.xv[H][3] & 0xFFFF0000u);
  }
  const float4 w4 = q.w[H];
  const float cb = q.b[H];
  f32x2 uv[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float v = fmaf(w4.w, xv[3 + j], fmaf(w4.z, xv[2 + j], fmaf(w4.y, xv[1 + j], fmaf(w4.x, xv[j], cb))));
    uv[j >> 1][j & 1] = !RAG || c < nch ? silu(v) : 0.0f;  // channels past D: exactly zero
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {  // round to bf16, nearest even (v_cvt_pk_bf16_f32)
    const uint32_t o = __builtin_bit_cast(uint32_t, __builtin_convertvector(uv[k], bf16x2));
    ut[(8 * g + 4 * HALF + 2 * k) * PITCH + c] = (uint16_t)o;
    ut[(8 * g + 4 * HALF + 2 * k + 1) * PITCH + c] = (uint16_t)(o >> 16);
  }
}

// The products of one step on the tiles ut / wt, with u of the next step (nch channels below D)
// computed into nu from X and the conv weights ct.  Per 16-channel slice: the operand fragments
// of the next slice are read first, then the slice's five products are issued one at a time with
// a quarter of the conv front's arithmetic between them (the matrix cores run a product while
// the vector units compute), then that quarter's u is written.
template <bool HEAD, bool RAG>
__device__ __forceinline__ void step_products(f32x16 (&acc)[MB_PER_WAVE], const uint16_t* ut, const uint16_t* wt,
                                              int tb, int mset, const XRegs& X, bool head, bool cache, int nch,
                                              const float* ct, uint16_t* nu) {
  const int lane = threadIdx.x & 63;
  const int frow = lane & 31, fk = 8 * (lane >> 5);
  bf16x8 bu[2], aw[2][MB_PER_WAVE];  // rows past M feed only outputs that are dropped
  auto frags = [&](int ks, int f) {
    bu[f] = *reinterpret_cast<const bf16x8*>(&ut[(32 * tb + frow) * PITCH + 16 * ks + fk]);
#pragma unroll
    for (int i = 0; i < MB_PER_WAVE; ++i)
      aw[f][i] = *reinterpret_cast<const bf16x8*>(&wt[(32 * (mset + 2 * i) + frow) * PITCH + 16 * ks + fk]);
  };
  const ConvW q = read_convw(ct);
  frags(0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < KC / 16; ++ks) {
    const int f = ks & 1;
    if (ks + 1 < KC / 16) frags(ks + 1, f ^ 1);
#pragma unroll
    for (int i = 0; i < MB_PER_WAVE; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aw[f][i], bu[f], acc[i], 0, 0, 0);
    if (ks == 0) conv_piece<0, 0, HEAD, RAG>(X, q, head, cache, nch, nu);
    if (ks == 1) conv_piece<0, 1, HEAD, RAG>(X, q, head, cache, nch, nu);
    if (ks == 2) conv_piece<1, 0, HEAD, RAG>(X, q, head, cache, nch, nu);
    if (ks == 3) conv_piece<1, 1, HEAD, RAG>(X, q, head, cache, nch, nu);
    // order within the slice: next fragments, then product / arithmetic / product ...
    if (ks + 1 < KC / 16) __builtin_amdgcn_sched_group_barrier(0x100, MB_PER_WAVE + 1, 0);
#pragma unroll
    for (int i = 0; i < MB_PER_WAVE; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One step of the pipeline on tiles P: products of step s; u of step s + 1 from XN (loaded two
// steps ago) with conv weights c[P ^ 1]; loads of W for step s + 1 (stored into w[P ^ 1] at the
// end), the conv weights of step s + 2 (into c[P], free since u of step s was made) and x of
// step s + 2 into XL.  All of it runs in every step, past the last step on repeated data into
// tiles that are no longer read: no load or wait then depends on a branch.
template <int P, bool HEAD, bool RAG>
__device__ __forceinline__ void pipe_step(const XprojArgs& a, Tiles& tl, WTile& w0, WTile& w1,
                                          f32x16 (&acc)[MB_PER_WAVE], int64_t b,
                                          int64_t t0, int m0, int tb, int mset, bool head, int s, int nsteps,
                                          const WSlots& ws, WRegs& W, XRegs& XL, const XRegs& XN) {
  const bool next = s + 1 < nsteps, after = s + 2 < nsteps;
  const int64_t kn = (int64_t)(next ? s + 1 : s) * KC;
  const int64_t ka = (int64_t)(after ? s + 2 : nsteps - 1) * KC;
  // issue order: what this step stores at its end first, x last (its wait is two steps away)
  dma_w<RAG>(a, kn, ws, P ? w0.w : w1.w);
  __builtin_amdgcn_sched_barrier(0);  // the tile loads first: the wait at the barrier is for them alone
  // only the first wave stores the conv weights: the others issue no load for them
  const bool cw_wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
  if (cw_wave) load_cw<RAG>(a, ka, W);
  load_x<HEAD, RAG>(a, b, t0, ka, XL);
  const int nch = a.D - kn < KC ? (int)(a.D - kn) : KC;
  step_products<HEAD, RAG>(acc, tl.u[P], P ? w1.w : w0.w, tb, mset, XN, head, a.conv0 != nullptr, nch, tl.c[P ^ 1], tl.u[P ^ 1]);
  if (cw_wave) store_cw<RAG>(a, ka, W, tl.c[P]);
  __syncthreads();
}

template <bool HEAD, bool RAG>
__device__ __forceinline__ void main_loop(const XprojArgs& a, Tiles& tl, WTile& w0, WTile& w1,
                                          f32x16 (&acc)[MB_PER_WAVE], int64_t b,
                                          int64_t t0, int m0, int tb, int mset) {
  const int nsteps = (int)((a.D + KC - 1) / KC);
  const bool head = t0 == 0 && (threadIdx.x >> 5) == 0;  // this thread's group starts a row
  const bool cache = a.conv0 != nullptr;
  XRegs X0, X1;
  WRegs W;
  const WSlots ws = w_slots(a, m0);
  dma_w<RAG>(a, 0, ws, w0.w);
  load_cw<RAG>(a, 0, W);
  load_x<HEAD, RAG>(a, b, t0, 0, X0);
  load_x<HEAD, RAG>(a, b, t0, nsteps > 1 ? KC : 0, X1);
  store_cw<RAG>(a, 0, W, tl.c[0]);
  if (nsteps > 1) {
    load_cw<RAG>(a, KC, W);
    store_cw<RAG>(a, KC, W, tl.c[1]);
  }
  __syncthreads();
  const int nch0 = a.D < KC ? (int)a.D : KC;
  const ConvW q0 = read_convw(tl.c[0]);
  conv_piece<0, 0, HEAD, RAG>(X0, q0, head, cache, nch0, tl.u[0]);
  conv_piece<0, 1, HEAD, RAG>(X0, q0, head, cache, nch0, tl.u[0]);
  conv_piece<1, 0, HEAD, RAG>(X0, q0, head, cache, nch0, tl.u[0]);
  conv_piece<1, 1, HEAD, RAG>(X0, q0, head, cache, nch0, tl.u[0]);
  __syncthreads();
  // Two steps per trip, so that each register set and tile has a fixed role in each half.
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    pipe_step<0, HEAD, RAG>(a, tl, w0, w1, acc, b, t0, m0, tb, mset, head, s, nsteps, ws, W, X0, X1);
    pipe_step<1, HEAD, RAG>(a, tl, w0, w1, acc, b, t0, m0, tb, mset, head, s + 1, nsteps, ws, W, X1, X0);
  }
  if (s < nsteps) pipe_step<0, HEAD, RAG>(a, tl, w0, w1, acc, b, t0, m0, tb, mset, head, s, nsteps, ws, W, X0, X1);
}

// Copy rows [lo, hi) of the stacked output (tensor `out`, width hi - lo) held in the staging
// tiles for this workgroup's ntok tokens (tokens 0..63 in ot0, 64..127 in ot1): V = 8 moves whole
// 16-byte pieces (each token's run starts 16-byte aligned and is a multiple of 8 long), V = 1
// single elements.
template <int V>
__device__ __forceinline__ void copy_rows(const uint16_t* ot0, const uint16_t* ot1, uint16_t* out, int64_t tok0,
                                          int ntok, int m0, int lo, int hi) {
  const int a0 = lo > m0 ? lo : m0, a1 = hi < m0 + ROWS ? hi : m0 + ROWS;
  if (a0 >= a1) return;
  const int width = hi - lo, run = (a1 - a0) / V;
  const int total = ntok * run;
  for (int e = threadIdx.x; e < total; e += THREADS) {
    const int tok = e / run, col = V * (e - tok * run);
    const uint16_t* src = &(tok < HALF_TT ? ot0 : ot1)[(tok % HALF_TT) * OPITCH + (a0 - m0) + col];
    uint16_t* dst = out + (tok0 + tok) * width + (a0 - lo) + col;
    if (V == 8)
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    else
      *dst = *src;
  }
}

__device__ __forceinline__ bool vec_ok(const void* out, int m0, int lo, int hi) {
  const int a0 = lo > m0 ? lo : m0, a1 = hi < m0 + ROWS ? hi : m0 + ROWS;
  return ((hi - lo) % 8 == 0) && ((a0 - lo) % 8 == 0) && ((a1 - a0) % 8 == 0) && ((a0 - m0) % 8 == 0) &&
         (reinterpret_cast<uintptr_t>(out) & 15) == 0;
}

__global__ __launch_bounds__(THREADS) void conv_xproj_kernel(XprojArgs a) {
  __shared__ __attribute__((aligned(16))) Tiles tl;
  __shared__ __attribute__((aligned(16))) WTile w0;
  __shared__ __attribute__((aligned(16))) WTile w1;
  const int64_t tiles_per_row = (a.L + TT - 1) / TT;
  const int64_t b = blockIdx.x / tiles_per_row;
  const int64_t t0 = (blockIdx.x - b * tiles_per_row) * TT;
  const int m0 = blockIdx.y * ROWS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tb = wave & 3, mset = wave >> 2;

  f32x16 acc[MB_PER_WAVE];
#pragma unroll
  for (int i = 0; i < MB_PER_WAVE; ++i) acc[i] = f32x16{};
  // The general form (a row's first tokens, channels past D in the last step) only where it is
  // needed: the first workgroup of each row, and every workgroup when D is not a multiple of KC.
  if (t0 == 0 || a.D % KC != 0) {
    if (t0 == 0) main_loop<true, true>(a, tl, w0, w1, acc, b, t0, m0, tb, mset);
    else main_loop<false, true>(a, tl, w0, w1, acc, b, t0, m0, tb, mset);
  } else {
    main_loop<false, false>(a, tl, w0, w1, acc, b, t0, m0, tb, mset);
  }

  // Stage the sums, rounded to bf16, as [token][row] in the W tiles (the last barrier of the loop
  // has freed them; tokens 0..63 in w0, 64..127 in w1): acc[i] register j is row
  // 32 blk + 8 (j / 4) + 4 (lane / 32) + j % 4 of token 32 tb + lane % 32, and registers j, j + 1
  // are adjacent rows.
  uint16_t* ot = tb < 2 ? w0.w : w1.w;  // uniform over the wave
  const int tok = 32 * (tb & 1) + (lane & 31);
#pragma unroll
  for (int i = 0; i < MB_PER_WAVE; ++i) {
    const int blk = mset + 2 * i;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const int m = 32 * blk + 8 * (j / 4) + 4 * (lane >> 5) + j % 4;
      const f32x2 pr = {acc[i][j], acc[i][j + 1]};
      *reinterpret_cast<uint32_t*>(&ot[tok * OPITCH + m]) = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
    }
  }
  __syncthreads();
  const int ntok = (int)((a.L - t0) < TT ? (a.L - t0) : TT);
  const int64_t tok0 = b * a.L + t0;
  uint16_t* outs[3] = {static_cast<uint16_t*>(a.out0), static_cast<uint16_t*>(a.out1),
                       static_cast<uint16_t*>(a.out2)};
  const int lo[3] = {0, a.R, a.R + a.N}, hi[3] = {a.R, a.R + a.N, a.M};
#pragma unroll
  for (int o = 0; o < 3; ++o) {
    if (vec_ok(outs[o], m0, lo[o], hi[o]))
      copy_rows<8>(w0.w, w1.w, outs[o], tok0, ntok, m0, lo[o], hi[o]);
    else
      copy_rows<1>(w0.w, w1.w, outs[o], tok0, ntok, m0, lo[o], hi[o]);
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
  // Buffer views and lane offsets are 32-bit: 64 channel rows of x and the whole of W must stay
  // below 2 GiB (seqlen below 2^24); the grid holds batch * ceil(L / 128) workgroups.
  int64_t rows, xbytes, tok, ob0, ob1;
  if (__builtin_mul_overflow(d->batch, d->d_inner, &rows) || __builtin_mul_overflow(rows, d->seqlen, &xbytes) ||
      __builtin_mul_overflow(xbytes, (int64_t)2, &xbytes) || __builtin_mul_overflow(d->batch, d->seqlen, &tok) ||
      __builtin_mul_overflow(tok, rank * 2, &ob0) || __builtin_mul_overflow(tok, d->d_state * 2, &ob1) ||
      d->seqlen * 2 * KC >= ((int64_t)1 << 31) || M * d->d_inner * 2 >= ((int64_t)1 << 31) ||
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
