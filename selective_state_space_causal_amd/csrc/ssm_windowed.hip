// ssm_windowed.hip -- prefill with one wave per (batch, channel) and the wave's lanes
// spread over time.
//
// The recurrence h_t = a_t * h_{t-1} + b_t (a_t = exp(delta_t * A), b_t = delta_t * u_t * B_t)
// is channel-local ("Scaling State-Space Models on Multiple GPUs with Tensor Parallelism",
// euno.news summary of arXiv 2602.21144, Methodology item 2), so a wave owns one channel
// and walks its sequence in windows of 64 * K tokens:
//   1. lane i takes tokens [t0 + i*K, t0 + (i+1)*K): loads x / dt / z with one 16-byte
//      vector load each, runs the conv + SiLU + softplus front end in registers (the
//      three previous raw inputs come from lane i-1 through a DPP wave shift);
//   2. per group of 4 states, each lane reduces its K tokens to one affine pair
//      (P, H) = (prod a_t, state reached from zero), keeping every a_t and b_t in
//      registers;
//   3. a Kogge-Stone scan of the pairs across the 64 lanes with DPP (row_shr 1/2/4/8,
//      row_bcast 15/31) gives each lane the state entering its tokens, seeded with the
//      carry of the previous window; lane 63's total becomes the next carry;
//   4. each lane replays its K tokens from that state with the stored a_t / b_t (no second
//      exp) and accumulates y_t = C_t . h_t.
// B and C are shared by every channel of a batch row, so the waves of a workgroup (W
// channels of one batch row) stage each window's B / C once in LDS as fp32, in a padded
// layout that keeps the 16-byte LDS reads free of bank conflicts.  The next window's
// inputs are prefetched into registers while the current one is computed.
#include "ssm_device.h"
#include "ssm_internal.h"

namespace ssm {
namespace {

constexpr int NS = 16;              // d_state handled by this kernel
constexpr int K = 8;                // tokens per lane per window
constexpr int WAVE = 64;
constexpr int WIN = WAVE * K;       // tokens per window
constexpr int W = 8;                // waves (channels) per workgroup
constexpr int THREADS = W * WAVE;
constexpr int G = 4;                // states per replay group
constexpr int LANE_STRIDE = K * NS + 4;  // floats per lane block in LDS (+4: conflict-free b128)

// GFX9 DPP control: each lane reads lane - 1 of the whole wave (lane 0 has no source).
constexpr int DPP_WAVE_SHR1 = 0x138;

// Value of `src` from the lane selected by CTRL; `old` where that lane does not exist or
// the row is masked off.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp(float old, float src) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, ROW_MASK, 0xf, false));
}

// Inclusive scan of four states' affine pairs (P, H) (the map h -> P h + H of this lane's
// tokens) across the 64 lanes, composing each lane's map after the earlier lanes' maps:
// four steps inside each row of 16 lanes (row_shr 1, 2, 4, 8), then row 0's total into
// row 1 and row 2's into row 3 (row_bcast 15), then rows 0-1 into rows 2 and 3
// (row_bcast 31).  Each step is H += H_src * P; P *= P_src with the DPP source folded into
// the VALU op; a lane without a source (or in a masked-off row) is not written, which is
// the identity (1, 0).  Then, with the window's entry state `carry` (uniform):
//   hin   = state entering this lane's tokens = (lane i-1's composed map)(carry),
//   carry = state after the window = (lane 63's composed map)(carry).
// The four states are interleaved, so every DPP source was written at least eight
// instructions earlier; the leading s_nop covers values written just before the block.
#define SSM_SCAN_STEP(CTRL)                                       \
  "v_fmac_f32_dpp %[H0], %[H0], %[P0] " CTRL " bank_mask:0xf\n"   \
  "v_fmac_f32_dpp %[H1], %[H1], %[P1] " CTRL " bank_mask:0xf\n"   \
  "v_fmac_f32_dpp %[H2], %[H2], %[P2] " CTRL " bank_mask:0xf\n"   \
  "v_fmac_f32_dpp %[H3], %[H3], %[P3] " CTRL " bank_mask:0xf\n"   \
  "v_mul_f32_dpp %[P0], %[P0], %[P0] " CTRL " bank_mask:0xf\n"    \
  "v_mul_f32_dpp %[P1], %[P1], %[P1] " CTRL " bank_mask:0xf\n"    \
  "v_mul_f32_dpp %[P2], %[P2], %[P2] " CTRL " bank_mask:0xf\n"    \
  "v_mul_f32_dpp %[P3], %[P3], %[P3] " CTRL " bank_mask:0xf\n"

__device__ __forceinline__ void scan4(float (&P)[4], float (&H)[4], float (&carry)[4], float (&hin)[4]) {
  float e0, e1, e2, e3;
  int s0, s1, s2, s3;
  asm volatile(
      "s_nop 1\n"
      SSM_SCAN_STEP("row_shr:1 row_mask:0xf")
      SSM_SCAN_STEP("row_shr:2 row_mask:0xf")
      SSM_SCAN_STEP("row_shr:4 row_mask:0xf")
      SSM_SCAN_STEP("row_shr:8 row_mask:0xf")
      SSM_SCAN_STEP("row_bcast:15 row_mask:0xa")
      SSM_SCAN_STEP("row_bcast:31 row_mask:0xc")
      "v_fma_f32 %[e0], %[P0], %[c0], %[H0]\n"
      "v_fma_f32 %[e1], %[P1], %[c1], %[H1]\n"
      "v_fma_f32 %[e2], %[P2], %[c2], %[H2]\n"
      "v_fma_f32 %[e3], %[P3], %[c3], %[H3]\n"
      "v_mov_b32 %[i0], %[c0]\n"
      "v_mov_b32 %[i1], %[c1]\n"
      "v_mov_b32 %[i2], %[c2]\n"
      "v_mov_b32 %[i3], %[c3]\n"
      "v_mov_b32_dpp %[i0], %[e0] wave_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b32_dpp %[i1], %[e1] wave_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b32_dpp %[i2], %[e2] wave_shr:1 row_mask:0xf bank_mask:0xf\n"
      "v_mov_b32_dpp %[i3], %[e3] wave_shr:1 row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_readlane_b32 %[s0], %[e0], 63\n"
      "v_readlane_b32 %[s1], %[e1], 63\n"
      "v_readlane_b32 %[s2], %[e2], 63\n"
      "v_readlane_b32 %[s3], %[e3], 63\n"
      "s_nop 1\n"
      : [H0] "+v"(H[0]), [H1] "+v"(H[1]), [H2] "+v"(H[2]), [H3] "+v"(H[3]), [P0] "+v"(P[0]), [P1] "+v"(P[1]),
        [P2] "+v"(P[2]), [P3] "+v"(P[3]), [e0] "=&v"(e0), [e1] "=&v"(e1), [e2] "=&v"(e2), [e3] "=&v"(e3),
        [i0] "=&v"(hin[0]), [i1] "=&v"(hin[1]), [i2] "=&v"(hin[2]), [i3] "=&v"(hin[3]), [s0] "=&s"(s0),
        [s1] "=&s"(s1), [s2] "=&s"(s2), [s3] "=&s"(s3)
      : [c0] "s"(carry[0]), [c1] "s"(carry[1]), [c2] "s"(carry[2]), [c3] "s"(carry[3]));
  carry[0] = __int_as_float(s0);
  carry[1] = __int_as_float(s1);
  carry[2] = __int_as_float(s2);
  carry[3] = __int_as_float(s3);
}
#undef SSM_SCAN_STEP

__device__ __forceinline__ float lane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

struct Tile {
  float B[WAVE * LANE_STRIDE];
  float C[WAVE * LANE_STRIDE];
};

// K consecutive io values of one channel row starting at token t (zero past L).
template <typename IO, bool ALIGNED>
__device__ __forceinline__ void load_block(const IO* __restrict__ row, int64_t t, int64_t L, IO (&v)[K]) {
  if (ALIGNED && t + K <= L) {
    const uint4* p = reinterpret_cast<const uint4*>(row + t);
    uint4 u[K * sizeof(IO) / 16];
#pragma unroll
    for (int i = 0; i < (int)(K * sizeof(IO) / 16); ++i) u[i] = p[i];
    __builtin_memcpy(v, u, sizeof(u));
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j) v[j] = (t + j < L) ? row[t + j] : IO{};
  }
}

template <typename IO, bool ALIGNED>
__device__ __forceinline__ void store_block(IO* __restrict__ row, int64_t t, int64_t L, const IO (&v)[K]) {
  if (ALIGNED && t + K <= L) {
    uint4 u[K * sizeof(IO) / 16];
    __builtin_memcpy(u, v, sizeof(u));
    uint4* p = reinterpret_cast<uint4*>(row + t);
#pragma unroll
    for (int i = 0; i < (int)(K * sizeof(IO) / 16); ++i) p[i] = u[i];
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (t + j < L) row[t + j] = v[j];
  }
}

// Window B / C staging: the tile of one io tensor is WIN * NS values, moved in 16-byte
// chunks, PER_THREAD chunks per thread of the workgroup.
template <typename IO>
struct TileChunks {
  static constexpr int EPC = 16 / sizeof(IO);          // io elements per chunk
  static constexpr int CHUNKS = WIN * NS / EPC;        // chunks per tensor per window
  static constexpr int PER_THREAD = CHUNKS / THREADS;
  uint4 b[PER_THREAD], c[PER_THREAD];
};

template <typename IO>
__device__ __forceinline__ void tile_fetch(TileChunks<IO>& tc, const IO* __restrict__ Bm, const IO* __restrict__ Cm,
                                           int64_t t0, int64_t L) {
  using T = TileChunks<IO>;
#pragma unroll
  for (int r = 0; r < T::PER_THREAD; ++r) {
    const int ci = threadIdx.x + r * THREADS;
    const int token = ci * T::EPC / NS;
    const int s0 = (ci * T::EPC) % NS;
    const int64_t tt = t0 + token;
    if (tt < L) {
      tc.b[r] = *reinterpret_cast<const uint4*>(Bm + tt * NS + s0);
      tc.c[r] = *reinterpret_cast<const uint4*>(Cm + tt * NS + s0);
    } else {
      tc.b[r] = make_uint4(0, 0, 0, 0);
      tc.c[r] = make_uint4(0, 0, 0, 0);
    }
  }
}

template <typename IO>
__device__ __forceinline__ void widen(const uint4& u, float (&f)[16 / sizeof(IO)]) {
  IO v[16 / sizeof(IO)];
  __builtin_memcpy(v, &u, 16);
#pragma unroll
  for (int e = 0; e < (int)(16 / sizeof(IO)); ++e) f[e] = to_f32(v[e]);
}

template <typename IO>
__device__ __forceinline__ void tile_store(Tile& tile, const TileChunks<IO>& tc) {
  using T = TileChunks<IO>;
#pragma unroll
  for (int r = 0; r < T::PER_THREAD; ++r) {
    const int ci = threadIdx.x + r * THREADS;
    const int token = ci * T::EPC / NS;
    const int s0 = (ci * T::EPC) % NS;
    const int off = (token / K) * LANE_STRIDE + (token % K) * NS + s0;
    float fb[T::EPC], fc[T::EPC];
    widen<IO>(tc.b[r], fb);
    widen<IO>(tc.c[r], fc);
#pragma unroll
    for (int e = 0; e < T::EPC; e += 4) {
      *reinterpret_cast<float4*>(&tile.B[off + e]) = make_float4(fb[e], fb[e + 1], fb[e + 2], fb[e + 3]);
      *reinterpret_cast<float4*>(&tile.C[off + e]) = make_float4(fc[e], fc[e + 1], fc[e + 2], fc[e + 3]);
    }
  }
}

template <typename IO, bool ALIGNED>
__global__ __launch_bounds__(THREADS) void prefill_windowed(ScanArgs a) {
  __shared__ Tile tile;
  const int lane = threadIdx.x & (WAVE - 1);
  const int wave = threadIdx.x / WAVE;
  const int64_t groups = (a.D + W - 1) / W;
  const int64_t b = blockIdx.x / groups;
  const int64_t c = (blockIdx.x - b * groups) * W + wave;
  const bool active = c < a.D;  // a ragged last group: idle waves still stage tiles and meet barriers
  const int64_t L = a.L;
  const int64_t row = b * a.D + (active ? c : 0);

  const IO* __restrict__ Bm = static_cast<const IO*>(a.Bm) + b * L * NS;
  const IO* __restrict__ Cm = static_cast<const IO*>(a.Cm) + b * L * NS;
  const IO* __restrict__ xr = static_cast<const IO*>(a.x) + row * L;
  const IO* __restrict__ dtr = static_cast<const IO*>(a.dt) + row * L;
  const IO* __restrict__ zr = a.z ? static_cast<const IO*>(a.z) + row * L : nullptr;
  IO* __restrict__ yr = static_cast<IO*>(a.y) + row * L;

  // Channel constants.
  const int64_t cc = active ? c : 0;
  const float w0 = a.conv_w[cc * 4 + 0], w1 = a.conv_w[cc * 4 + 1], w2 = a.conv_w[cc * 4 + 2],
              w3 = a.conv_w[cc * 4 + 3];
  const float cb = a.conv_b ? a.conv_b[cc] : 0.0f;
  const float dtb = a.dt_bias[cc], dsk = a.Dskip[cc];
  float A2[NS], carry[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    A2[n] = a.A[cc * NS + n] * kLog2e;
    carry[n] = a.h0 ? a.h0[row * NS + n] : 0.0f;
  }
  float hist0 = 0.0f, hist1 = 0.0f, hist2 = 0.0f;  // raw x[t0-3], x[t0-2], x[t0-1]
  if (a.conv0) {
    hist0 = a.conv0[row * 3 + 0];
    hist1 = a.conv0[row * 3 + 1];
    hist2 = a.conv0[row * 3 + 2];
  }
  const float init0 = hist0, init1 = hist1, init2 = hist2;

  const int64_t nwin = (L + WIN - 1) / WIN;
  TileChunks<IO> pf;
  IO px[K], pdt[K], pz[K];
#pragma unroll
  for (int j = 0; j < K; ++j) pz[j] = IO{};
  tile_fetch<IO>(pf, Bm, Cm, 0, L);
  load_block<IO, ALIGNED>(xr, (int64_t)lane * K, L, px);
  load_block<IO, ALIGNED>(dtr, (int64_t)lane * K, L, pdt);
  if (zr) load_block<IO, ALIGNED>(zr, (int64_t)lane * K, L, pz);

  for (int64_t w = 0; w < nwin; ++w) {
    const int64_t t0 = w * WIN;
    const int64_t tl = t0 + (int64_t)lane * K;  // this lane's first token
    __syncthreads();  // every wave is done reading the previous tile
    tile_store<IO>(tile, pf);
    __syncthreads();
    IO cx[K], cdt[K], cz[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
      cx[j] = px[j];
      cdt[j] = pdt[j];
      cz[j] = pz[j];
    }
    if (w + 1 < nwin) {  // prefetch the next window while this one is computed
      tile_fetch<IO>(pf, Bm, Cm, t0 + WIN, L);
      load_block<IO, ALIGNED>(xr, tl + WIN, L, px);
      load_block<IO, ALIGNED>(dtr, tl + WIN, L, pdt);
      if (zr) load_block<IO, ALIGNED>(zr, tl + WIN, L, pz);
    }
    if (!active) continue;

    // ---- front end: conv window, SiLU, softplus, gate ----
    float xv[K];
#pragma unroll
    for (int j = 0; j < K; ++j) xv[j] = to_f32(cx[j]);
    const float xm3 = dpp<DPP_WAVE_SHR1, 0xf>(hist0, xv[K - 3]);
    const float xm2 = dpp<DPP_WAVE_SHR1, 0xf>(hist1, xv[K - 2]);
    const float xm1 = dpp<DPP_WAVE_SHR1, 0xf>(hist2, xv[K - 1]);
    hist0 = lane63(xv[K - 3]);
    hist1 = lane63(xv[K - 2]);
    hist2 = lane63(xv[K - 1]);

    float dl[K], du[K], yv[K], gt[K];
    float dsum = 0.0f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const float s3 = j >= 3 ? xv[j - 3] : (j == 0 ? xm3 : (j == 1 ? xm2 : xm1));
      const float s2 = j >= 2 ? xv[j - 2] : (j == 0 ? xm2 : xm1);
      const float s1 = j >= 1 ? xv[j - 1] : xm1;
      const float v = cb + w0 * s3 + w1 * s2 + w2 * s1 + w3 * xv[j];
      const float u = silu(v);
      const bool valid = tl + j < L;
      const float d = valid ? softplus(to_f32(cdt[j]) + dtb) : 0.0f;  // delta = 0: identity step
      dl[j] = d;
      du[j] = d * u;
      yv[j] = dsk * u;
      gt[j] = zr ? silu(to_f32(cz[j])) : 1.0f;
      dsum += d;
    }

    // ---- state groups: local pairs, lane scan, replay ----
    const float* tb = &tile.B[lane * LANE_STRIDE];
    const float* tcp = &tile.C[lane * LANE_STRIDE];
#pragma unroll
    for (int q0 = 0; q0 < NS; q0 += G) {
      float av[K][G], bv[K][G], P[G], H[G];
#pragma unroll
      for (int q = 0; q < G; ++q) {
        P[q] = hw_exp2(A2[q0 + q] * dsum);  // prod_j exp(delta_j A) over this lane's tokens
        H[q] = 0.0f;
      }
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const float4 Bq = *reinterpret_cast<const float4*>(tb + j * NS + q0);
        const float bq[4] = {Bq.x, Bq.y, Bq.z, Bq.w};
#pragma unroll
        for (int q = 0; q < G; ++q) {
          av[j][q] = hw_exp2(dl[j] * A2[q0 + q]);
          bv[j][q] = du[j] * bq[q];
          H[q] = fmaf(av[j][q], H[q], bv[j][q]);
        }
      }
      float hc[G], cg[G];
#pragma unroll
      for (int q = 0; q < G; ++q) cg[q] = carry[q0 + q];
      scan4(P, H, cg, hc);
#pragma unroll
      for (int q = 0; q < G; ++q) carry[q0 + q] = cg[q];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const float4 Cq = *reinterpret_cast<const float4*>(tcp + j * NS + q0);
        const float cq[4] = {Cq.x, Cq.y, Cq.z, Cq.w};
#pragma unroll
        for (int q = 0; q < G; ++q) {
          hc[q] = fmaf(av[j][q], hc[q], bv[j][q]);
          yv[j] = fmaf(cq[q], hc[q], yv[j]);
        }
      }
    }

    IO out[K];
#pragma unroll
    for (int j = 0; j < K; ++j) out[j] = from_f32<IO>(yv[j] * gt[j]);
    store_block<IO, ALIGNED>(yr, tl, L, out);
  }

  if (active && lane == 0) {
#pragma unroll
    for (int n = 0; n < NS; ++n) a.h_out[row * NS + n] = carry[n];
    const float init[3] = {init0, init1, init2};
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int64_t t = L - 3 + j;  // raw input xi[L-3+j]; history below zero
      a.conv_out[row * 3 + j] = t >= 0 ? to_f32(xr[t]) : init[t + 3];
    }
  }
}

}  // namespace

bool windowed_supported(const ScanArgs& a) { return a.N == NS; }

hipError_t launch_windowed(const ScanArgs& a, hipStream_t s) {
  const int64_t groups = (a.D + W - 1) / W;
  const dim3 grid((unsigned)(a.B * groups)), block(THREADS);
  if (a.bf16) {
    if (a.L % 8 == 0) prefill_windowed<bf16_t, true><<<grid, block, 0, s>>>(a);
    else prefill_windowed<bf16_t, false><<<grid, block, 0, s>>>(a);
  } else {
    if (a.L % 4 == 0) prefill_windowed<float, true><<<grid, block, 0, s>>>(a);
    else prefill_windowed<float, false><<<grid, block, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace ssm
