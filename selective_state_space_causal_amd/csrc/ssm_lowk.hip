// ssm_lowk.hip -- ssm_proj (include/ssm_proj.h) for a small inner dimension: the token-major-in,
// channel-major-out kinds, out[b, m, t] = sum_k W[m, k] in[b, t, k], with K a multiple of 16 up to
// 256 -- the step-size projection, whose K is the step input's rank ("Scaling State-Space Models
// on Multiple GPUs with Tensor Parallelism", euno.news summary of arXiv 2602.21144, Methodology
// item 1: a rank's slice of the mixer's projections).
//
// With K this small each output element needs few products, so the call is bound by writing the
// channel-major output (M x L values, against L x K of input), not by the matrix cores.  Each wave
// keeps the weights of its 64 channels (two blocks of 32) in registers for the whole call (K / 2
// VGPRs), and a workgroup of 8 waves (512 channels) walks a contiguous range of 64-token tiles:
// a tile of the input ([64 tokens][K], bf16) is loaded once into LDS, double-buffered (the next
// tile's loads are in flight while the current one is multiplied), and every wave multiplies it by
// its weights on the matrix cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation; per tile 2 token
// blocks x 2 channel blocks x K / 16 products).  The input tile is the product's first operand and
// the weights its second, so that each lane holds runs of 4 consecutive tokens of one channel;
// rounded to bf16 (nearest even) they are staged in the wave's own LDS region as [64 channels]
// [64 tokens] and stored as 16-byte pieces, 8 lanes to a row: each store instruction writes whole
// 128-byte lines of 8 output rows.  (Stored straight from the accumulators, 8 bytes per lane, an
// instruction touched 32 rows and a row got half a line per tile: 70 us for the 7B-class layer's
// step-size projection, against 60 us for the library GEMM.)  Tokens are flattened over the batch
// rows (a tile may span two of them; each 8-token piece lies in one, found by a multiply-shift
// division).  The workgroups of one token range (one per group of 512 channels) are given ids that
// land on one XCD, so that they share its L2 copy of the input tiles (the input was fetched past L2
// once per channel group before: 69 MB against 25 MB).  Loads past the last token or channel are
// clamped into the tensors; their products feed only outputs that are not stored.
#include <stdint.h>

#include "ssm_internal.h"
#include "ssm_lowk.h"

namespace ssm {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kChPerWave = 64;
constexpr int kChPerBlock = kWaves * kChPerWave;
constexpr int kTok = 64;        // tokens per tile (two blocks of 32)
constexpr int kMaxKS = 16;      // K / 16 at most (K <= 256)
constexpr int kTargetBlocks = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct LowkArgs {
  const uint16_t* in;  // [T, K], T = batch x seqlen (token-major)
  const uint16_t* w;   // [M, K]
  uint16_t* out;       // [batch, M, L]
  int64_t L, T;
  uint64_t l_magic;    // bt / L = (bt * l_magic) >> l_shift for bt < 2^30
  int l_shift;
  int M, ntiles, per;  // per: tiles per workgroup (a contiguous range)
  int gx;              // channel groups
};

template <int KS>
__global__ __launch_bounds__(kThreads) void lowk_kernel(LowkArgs a) {
  constexpr int K = 16 * KS;
  constexpr int PITCH = K + 8;           // bf16 per LDS tile row: 16-byte fragment reads of 16 rows hit distinct banks
  constexpr int PIECES = kTok * K / 8;   // 16-byte pieces per input tile
  constexpr int PPT = (PIECES + kThreads - 1) / kThreads;
  constexpr int SPITCH = kTok + 8;       // bf16 per row of a wave's output staging ([64 channels][64 tokens])
  __shared__ __attribute__((aligned(16))) uint16_t tile[2][kTok * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t stage[kWaves][kChPerWave * SPITCH];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Workgroup id -> (channel group gx, token range gy): consecutive ids go to the 8 XCDs in turn,
  // so the channel groups of one token range are given ids of one XCD, and share its L2 copy of
  // the input tiles.
  const int id = blockIdx.x, xcd = id & 7, slot = id >> 3;
  const int gxi = slot % a.gx, gyi = (slot / a.gx) * 8 + xcd;
  const int c0 = gxi * kChPerBlock + wave * kChPerWave;  // the wave's first channel
  const bool active = c0 < a.M;                                   // uniform over the wave

  // Weight fragments: block j, product s: W[c0 + 32 j + lane % 32][16 s + 8 (lane / 32) .. + 7].
  bf16x8 wf[2][KS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = min(c0 + 32 * j + (lane & 31), a.M - 1);
    const uint16_t* wr = a.w + (int64_t)c * K + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < KS; ++s) wf[j][s] = *reinterpret_cast<const bf16x8*>(wr + 16 * s);
  }
  // Wait for them here, once: their first use inside the loop made the compiler wait on the
  // memory counter there in every trip, and so also for the next tile's loads issued before it.
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(wf[j][s]));

  const int first = gyi * a.per;
  const int last = min(first + a.per, a.ntiles);
  u32x4 pre[PPT];
  auto load_tile = [&](int it) {
    const int64_t t0 = (int64_t)it * kTok;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = threadIdx.x + i * kThreads;
      if (PIECES % kThreads == 0 || p < PIECES) {
        const int row = p / (K / 8), ch = p - row * (K / 8);
        const int64_t bt = min(t0 + row, a.T - 1);
        pre[i] = *reinterpret_cast<const u32x4*>(a.in + bt * K + 8 * ch);
      }
    }
  };
  auto store_tile = [&](uint16_t* buf) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = threadIdx.x + i * kThreads;
      if (PIECES % kThreads == 0 || p < PIECES) {
        const int row = p / (K / 8), ch = p - row * (K / 8);
        *reinterpret_cast<u32x4*>(buf + row * PITCH + 8 * ch) = pre[i];
      }
    }
  };

  if (first < last) {
    load_tile(first);
    store_tile(tile[0]);
  }
  __syncthreads();
  uint16_t* const st = stage[wave];
  int buf = 0;
  for (int it = first; it < last; ++it) {
    if (it + 1 < last) load_tile(it + 1);
    if (active) {
      f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};  // [token block][channel block]
      const uint16_t* tr = tile[buf] + (lane & 31) * PITCH + 8 * (lane >> 5);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const bf16x8 af = *reinterpret_cast<const bf16x8*>(tr + 32 * tb * PITCH + 16 * s);
          acc[tb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wf[0][s], acc[tb][0], 0, 0, 0);
          acc[tb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, wf[1][s], acc[tb][1], 0, 0, 0);
        }
      }
      // The next tile into LDS before the output stores: waiting for its loads then does not also
      // wait for this tile's stores.
      if (it + 1 < last) store_tile(tile[buf ^ 1]);
      // acc[tb][j] register 4 q + r is token 32 tb + 8 q + 4 (lane / 32) + r of the tile, channel
      // 32 j + lane % 32 of the wave: rounded to bf16, staged as [channel][token] in the wave's own
      // region (no other wave reads it), 4 consecutive tokens per 8-byte write ...
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x2 lo = {acc[tb][j][4 * q], acc[tb][j][4 * q + 1]};
            const f32x2 hi = {acc[tb][j][4 * q + 2], acc[tb][j][4 * q + 3]};
            const u32x2 v = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                             __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2))};
            *reinterpret_cast<u32x2*>(st + (32 * j + (lane & 31)) * SPITCH + 32 * tb + 8 * q + 4 * (lane >> 5)) = v;
          }
      // ... then read back as 16-byte pieces of 8 tokens, 8 lanes to a channel row, so that each
      // store fills whole 128-byte lines of 8 rows.
#pragma unroll
      for (int i = 0; i < kChPerWave * kTok / 8 / 64; ++i) {
        const int p = lane + 64 * i, row = p >> 3, col = 8 * (p & 7);
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + row * SPITCH + col);
        const int c = c0 + row;
        const int64_t bt = (int64_t)it * kTok + col;  // a multiple of 8, as L is: one batch row
        if (c < a.M && bt < a.T) {
          const int64_t b = (int64_t)(((uint64_t)bt * a.l_magic) >> a.l_shift);
          const int64_t t = bt - b * a.L;
          *reinterpret_cast<u32x4*>(a.out + (b * a.M + c) * a.L + t) = v;
        }
      }
    } else if (it + 1 < last) {
      store_tile(tile[buf ^ 1]);
    }
    __syncthreads();
    buf ^= 1;
  }
}

template <int KS>
hipError_t launch(const LowkArgs& a, int gx, int gy, hipStream_t s) {
  lowk_kernel<KS><<<dim3((unsigned)(gx * gy)), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace

bool lowk_fits(int64_t batch, int64_t seqlen, int64_t in_features, int64_t out_features, bool bf16_io,
               bool bf16_out) {
  return bf16_io && bf16_out && in_features % 16 == 0 && in_features <= 16 * kMaxKS && seqlen % 8 == 0 &&
         seqlen <= ((int64_t)1 << 24) && batch * seqlen < ((int64_t)1 << 30) && out_features < ((int64_t)1 << 30);
}

bool lowk(int64_t batch, int64_t seqlen, int64_t in_features, int64_t out_features, const void* in, const void* w,
          void* out, hipStream_t stream) {
  LowkArgs a;
  a.in = static_cast<const uint16_t*>(in);
  a.w = static_cast<const uint16_t*>(w);
  a.out = static_cast<uint16_t*>(out);
  a.L = seqlen;
  a.T = batch * seqlen;
  div_magic(seqlen, &a.l_magic, &a.l_shift);
  a.M = (int)out_features;
  a.ntiles = (int)((a.T + kTok - 1) / kTok);
  const int gx = (int)((out_features + kChPerBlock - 1) / kChPerBlock);
  // about kTargetBlocks workgroups in all (one per CU), each a contiguous range of tiles
  const int want = (kTargetBlocks + gx - 1) / gx;
  a.per = (a.ntiles + want - 1) / want;
  const int gy = ((a.ntiles + a.per - 1) / a.per + 7) / 8 * 8;  // a multiple of 8 (ranges past the end are empty)
  a.gx = gx;
  (void)hipGetLastError();
  hipError_t e;
  switch (in_features / 16) {
    case 1: e = launch<1>(a, gx, gy, stream); break;
    case 2: e = launch<2>(a, gx, gy, stream); break;
    case 3: e = launch<3>(a, gx, gy, stream); break;
    case 4: e = launch<4>(a, gx, gy, stream); break;
    case 5: e = launch<5>(a, gx, gy, stream); break;
    case 6: e = launch<6>(a, gx, gy, stream); break;
    case 7: e = launch<7>(a, gx, gy, stream); break;
    case 8: e = launch<8>(a, gx, gy, stream); break;
    case 9: e = launch<9>(a, gx, gy, stream); break;
    case 10: e = launch<10>(a, gx, gy, stream); break;
    case 11: e = launch<11>(a, gx, gy, stream); break;
    case 12: e = launch<12>(a, gx, gy, stream); break;
    case 13: e = launch<13>(a, gx, gy, stream); break;
    case 14: e = launch<14>(a, gx, gy, stream); break;
    case 15: e = launch<15>(a, gx, gy, stream); break;
    case 16: e = launch<16>(a, gx, gy, stream); break;
    default: return false;
  }
  return e == hipSuccess;
}

}  // namespace ssm
