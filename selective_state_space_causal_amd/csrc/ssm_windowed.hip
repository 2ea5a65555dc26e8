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
//   2. per group of 8 or 4 states (the launch shapes below), each lane reduces its K tokens
//      to one affine pair (P, H) = (prod a_t, state reached from zero), keeping every a_t
//      and b_t in registers;
//   3. a Kogge-Stone scan of the pairs across the 64 lanes with DPP (row_shr 1/2/4/8,
//      row_bcast 15/31) gives each lane the state entering its tokens; the carry of the
//      previous window enters through lane 0's first token, and lane 63's total becomes the
//      next carry;
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
// Launch shapes (waves per workgroup W = channels per workgroup, states per replay group G).
// Per channel the arithmetic is the same in every shape -- same windows, same per-state
// operations in the same order -- so every shape gives bit-identical results, and the choice
// may follow the channel count.  A workgroup of any shape fills one CU (registers and the
// two LDS tiles), so a launch runs in rounds of one workgroup per CU:
//   W 8,  G 8: two waves per SIMD, eight independent state chains per pass; 249 VGPRs;
//   W 12, G 4: three waves per SIMD; 168 VGPRs; a round takes ~1.40x as long as W 8's for
//              1.5x the channels;
//   W 16, G 2: four waves per SIMD; at most 128 VGPRs; a round ~1.84x W 8's for 2x the channels;
//   W 8,  G 4: fp32 io (its wider prefetch registers would spill with more).
// The wider bf16 shapes need 16-byte aligned rows (their unaligned forms would spill).  For
// bf16 io the launch takes the shape with the fewest round-weighted units,
// ceil(workgroups / CUs) x round time: the wider shapes pay off when they need fewer rounds
// (mamba130m's 6144 channels: 3 rounds of W 8 against 2 of W 12).
struct ShapeCost {
  int w;
  float round_time;  // relative to W 8, G 8; measured on MI355X, bf16 io
};
constexpr ShapeCost kShapes[] = {{8, 1.0f}, {12, 1.40f}, {16, 1.84f}};
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
// the identity (1, 0).  The window's entry state was already folded into lane 0's first
// token (seed_carry), so after the scan H is the state after each lane's tokens, and the
// last step needs no P.  Then:
//   hin   = state entering this lane's tokens = H of lane i-1, and 0 for lane 0 (its tokens
//           carry the entry state themselves; bound_ctrl:0 is this assembler's spelling of
//           the zero-fill bit for lanes without a source),
//   carry = state after the window = H of lane 63.
// The four states are interleaved, so every DPP source was written at least three
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
#define SSM_SCAN_LAST(CTRL)                                       \
  "v_fmac_f32_dpp %[H0], %[H0], %[P0] " CTRL " bank_mask:0xf\n"   \
  "v_fmac_f32_dpp %[H1], %[H1], %[P1] " CTRL " bank_mask:0xf\n"   \
  "v_fmac_f32_dpp %[H2], %[H2], %[P2] " CTRL " bank_mask:0xf\n"   \
  "v_fmac_f32_dpp %[H3], %[H3], %[P3] " CTRL " bank_mask:0xf\n"

__device__ __forceinline__ void scan4(float (&P)[4], float (&H)[4], float (&carry)[4], float (&hin)[4]) {
  int s0, s1, s2, s3;
  asm volatile(
      "s_nop 1\n"
      SSM_SCAN_STEP("row_shr:1 row_mask:0xf")
      SSM_SCAN_STEP("row_shr:2 row_mask:0xf")
      SSM_SCAN_STEP("row_shr:4 row_mask:0xf")
      SSM_SCAN_STEP("row_shr:8 row_mask:0xf")
      SSM_SCAN_STEP("row_bcast:15 row_mask:0xa")
      SSM_SCAN_LAST("row_bcast:31 row_mask:0xc")
      "s_nop 1\n"
      "v_mov_b32_dpp %[i0], %[H0] wave_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:0\n"
      "v_mov_b32_dpp %[i1], %[H1] wave_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:0\n"
      "v_mov_b32_dpp %[i2], %[H2] wave_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:0\n"
      "v_mov_b32_dpp %[i3], %[H3] wave_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:0\n"
      "v_readlane_b32 %[s0], %[H0], 63\n"
      "v_readlane_b32 %[s1], %[H1], 63\n"
      "v_readlane_b32 %[s2], %[H2], 63\n"
      "v_readlane_b32 %[s3], %[H3], 63\n"
      "s_nop 1\n"
      : [H0] "+v"(H[0]), [H1] "+v"(H[1]), [H2] "+v"(H[2]), [H3] "+v"(H[3]), [P0] "+v"(P[0]), [P1] "+v"(P[1]),
        [P2] "+v"(P[2]), [P3] "+v"(P[3]), [i0] "=&v"(hin[0]), [i1] "=&v"(hin[1]), [i2] "=&v"(hin[2]),
        [i3] "=&v"(hin[3]), [s0] "=&s"(s0), [s1] "=&s"(s1), [s2] "=&s"(s2), [s3] "=&s"(s3));
  carry[0] = __int_as_float(s0);
  carry[1] = __int_as_float(s1);
  carry[2] = __int_as_float(s2);
  carry[3] = __int_as_float(s3);
}

// The same scan over two interleaved states (the 2-state groups of the 16-channel shape).
// Each DPP source is written at least one instruction before it is read; the s_nop 1 lines
// cover the places where it is the instruction right before.
#define SSM_SCAN2_STEP(CTRL)                                      \
  "v_fmac_f32_dpp %[H0], %[H0], %[P0] " CTRL " bank_mask:0xf\n"   \
  "v_fmac_f32_dpp %[H1], %[H1], %[P1] " CTRL " bank_mask:0xf\n"   \
  "v_mul_f32_dpp %[P0], %[P0], %[P0] " CTRL " bank_mask:0xf\n"    \
  "v_mul_f32_dpp %[P1], %[P1], %[P1] " CTRL " bank_mask:0xf\n"

__device__ __forceinline__ void scan2(float (&P)[2], float (&H)[2], float (&carry)[2], float (&hin)[2]) {
  int s0, s1;
  asm volatile(
      "s_nop 1\n"
      SSM_SCAN2_STEP("row_shr:1 row_mask:0xf")
      SSM_SCAN2_STEP("row_shr:2 row_mask:0xf")
      SSM_SCAN2_STEP("row_shr:4 row_mask:0xf")
      SSM_SCAN2_STEP("row_shr:8 row_mask:0xf")
      SSM_SCAN2_STEP("row_bcast:15 row_mask:0xa")
      "v_fmac_f32_dpp %[H0], %[H0], %[P0] row_bcast:31 row_mask:0xc bank_mask:0xf\n"
      "v_fmac_f32_dpp %[H1], %[H1], %[P1] row_bcast:31 row_mask:0xc bank_mask:0xf\n"
      "s_nop 1\n"
      "v_mov_b32_dpp %[i0], %[H0] wave_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:0\n"
      "v_mov_b32_dpp %[i1], %[H1] wave_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:0\n"
      "v_readlane_b32 %[s0], %[H0], 63\n"
      "v_readlane_b32 %[s1], %[H1], 63\n"
      "s_nop 1\n"
      : [H0] "+v"(H[0]), [H1] "+v"(H[1]), [P0] "+v"(P[0]), [P1] "+v"(P[1]), [i0] "=&v"(hin[0]),
        [i1] "=&v"(hin[1]), [s0] "=&s"(s0), [s1] "=&s"(s1));
  carry[0] = __int_as_float(s0);
  carry[1] = __int_as_float(s1);
}
#undef SSM_SCAN2_STEP
#undef SSM_SCAN_LAST
#undef SSM_SCAN_STEP

// Fold the window's entry state into lane 0's first token: b_0 += a_0 * carry on lane 0 only
// (exec narrowed to lane 0 and restored inside the block; lane 0 stays off if it was off), so
// the lane scan and the replay carry it with no further term.  A DPP instruction needs five
// wait states after an exec write; the next one (the lane scan) comes after the seven fold
// FMAs per state that depend on this block's results.
#define SSM_SEED(I) "v_fmac_f32 %[b" #I "], %[c" #I "], %[a" #I "]\n"
__device__ __forceinline__ void seed4(float* b, const float* a, const float* c) {
  uint64_t save;
  asm volatile("s_mov_b64 %[sv], exec\n"
               "s_and_b64 exec, %[sv], 1\n"
               SSM_SEED(0) SSM_SEED(1) SSM_SEED(2) SSM_SEED(3)
               "s_mov_b64 exec, %[sv]\n"
               : [b0] "+v"(b[0]), [b1] "+v"(b[1]), [b2] "+v"(b[2]), [b3] "+v"(b[3]), [sv] "=&s"(save)
               : [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]), [c0] "s"(c[0]), [c1] "s"(c[1]),
                 [c2] "s"(c[2]), [c3] "s"(c[3]));
}
__device__ __forceinline__ void seed2(float* b, const float* a, const float* c) {
  uint64_t save;
  asm volatile("s_mov_b64 %[sv], exec\n"
               "s_and_b64 exec, %[sv], 1\n"
               SSM_SEED(0) SSM_SEED(1)
               "s_mov_b64 exec, %[sv]\n"
               : [b0] "+v"(b[0]), [b1] "+v"(b[1]), [sv] "=&s"(save)
               : [a0] "v"(a[0]), [a1] "v"(a[1]), [c0] "s"(c[0]), [c1] "s"(c[1]));
}
#undef SSM_SEED

template <int G>
__device__ __forceinline__ void seed_carry(float (&b0)[G], const float (&a0)[G], const float (&carry)[G]) {
  if constexpr (G == 2) {
    seed2(b0, a0, carry);
  } else {
#pragma unroll
    for (int g = 0; g < G; g += 4) seed4(&b0[g], &a0[g], &carry[g]);
  }
}

// Scan G interleaved states (G = 2, or a multiple of 4).
template <int G>
__device__ __forceinline__ void scan_group(float (&P)[G], float (&H)[G], float (&carry)[G], float (&hin)[G]) {
  if constexpr (G == 2) {
    scan2(P, H, carry, hin);
  } else {
    static_assert(G % 4 == 0, "state groups of 2 or a multiple of 4");
#pragma unroll
    for (int g = 0; g < G; g += 4)
      scan4(*reinterpret_cast<float(*)[4]>(&P[g]), *reinterpret_cast<float(*)[4]>(&H[g]),
            *reinterpret_cast<float(*)[4]>(&carry[g]), *reinterpret_cast<float(*)[4]>(&hin[g]));
  }
}

// G consecutive fp32 states of one token from the LDS tile (16-byte reads; 8-byte for G = 2).
template <int G>
__device__ __forceinline__ void tile_states(const float* p, float (&v)[G]) {
  if constexpr (G == 2) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x;
    v[1] = t.y;
  } else {
#pragma unroll
    for (int g = 0; g < G; g += 4) {
      const float4 t = *reinterpret_cast<const float4*>(p + g);
      v[g] = t.x;
      v[g + 1] = t.y;
      v[g + 2] = t.z;
      v[g + 3] = t.w;
    }
  }
}

// A scheduling fence for LDS reads only: the tile reads issued before it stay before the
// arithmetic after it (vector and scalar ALU work may still move across it).
__device__ __forceinline__ void keep_lds_reads_here() { __builtin_amdgcn_sched_barrier(0x6); }

__device__ __forceinline__ float lane63(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

struct Tile {
  float B[WAVE * LANE_STRIDE];
  float C[WAVE * LANE_STRIDE];
};

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw-buffer view of one tensor row: loads past `bytes` return zeros and stores past it are
// dropped by the hardware, so ragged ends need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// View of a row of `elems` elements from element `from` on, for one window: the window's offset
// is in the descriptor's base (scalar arithmetic), so every access of the window addresses it
// through its per-lane voffset alone, which the range check covers, and the view ends where the
// row ends (an empty view when `from` is past it: loads read zeros, stores are dropped).
// Rows hold fewer than 2^31 bytes (windowed_supported), so the counts are 32-bit scalars.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window_rsrc(const T* row, int elems, int from) {
  const int left = elems - from;
  return row_rsrc(row + from, left > 0 ? left * (int)sizeof(T) : 0);
}

// Unpack io words into fp32: bf16 pairs are (low, high) halves of a dword.
template <typename IO>
__device__ __forceinline__ float unpack(const uint32_t* w, int j) {
  if constexpr (sizeof(IO) == 2)
    return __uint_as_float((j & 1) ? (w[j >> 1] & 0xFFFF0000u) : (w[j >> 1] << 16));
  else
    return __uint_as_float(w[j]);
}

// Two fp32 values -> two bf16 (round to nearest even) packed in a dword, first in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  uint32_t r;
  asm("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(r) : "v"(lo), "v"(hi));
  return r;
}

// Cache policy of the per-channel streams (x, dt, z read once; y written once): non-temporal.
// A prefill streams ~400 MB of them through the caches; with the default policy they evict
// the data the next calls keep reusing (a decode step right after a slice7b prefill took
// 3.26 us instead of 2.0 us; 2.68 us with this policy), and the prefill itself is no slower.
// B / C keep the default: every channel of a batch row rereads them.
constexpr int STREAM = 2;

// K io values of a lane as dwords: 16-byte loads when rows are 16-byte aligned, element loads
// otherwise; past the row end the buffer returns zeros.
template <typename IO, bool ALIGNED>
struct Lanes {
  static constexpr int DW = K * (int)sizeof(IO) / 4;
  uint32_t w[DW];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, int voff) {
    if constexpr (ALIGNED) {
#pragma unroll
      for (int i = 0; i < DW; i += 4) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 4 * i, 0, STREAM);
        w[i] = v[0];
        w[i + 1] = v[1];
        w[i + 2] = v[2];
        w[i + 3] = v[3];
      }
    } else if constexpr (sizeof(IO) == 2) {
#pragma unroll
      for (int i = 0; i < DW; ++i) {
        const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, voff + 4 * i, 0, STREAM);
        const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, voff + 4 * i + 2, 0, STREAM);
        w[i] = lo | (hi << 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < DW; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, voff + 4 * i, 0, STREAM);
    }
  }
};

// Store the lane's first `nvalid` outputs (all K as vector stores when the lane is whole).
template <typename IO, bool ALIGNED>
__device__ __forceinline__ void store_lanes(__amdgpu_buffer_rsrc_t r, int voff, const float (&v)[K], int nvalid) {
  if (nvalid < K) {
    if (nvalid > 0) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        if (j < nvalid) {
          if constexpr (sizeof(IO) == 2)
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_bf16x2(v[j], 0.0f) & 0xFFFFu), r,
                                                  voff + 2 * j, 0, STREAM);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[j]), r, voff + 4 * j, 0, STREAM);
        }
      }
    }
    return;
  }
  if constexpr (sizeof(IO) == 2) {
    uint32_t w[K / 2];
#pragma unroll
    for (int i = 0; i < K / 2; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    if constexpr (ALIGNED) {
      const u32x4 v4 = {w[0], w[1], w[2], w[3]};
      __builtin_amdgcn_raw_buffer_store_b128(v4, r, voff, 0, STREAM);
    } else {
#pragma unroll
      for (int i = 0; i < K / 2; ++i) {
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(w[i] & 0xFFFFu), r, voff + 4 * i, 0, STREAM);
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(w[i] >> 16), r, voff + 4 * i + 2, 0, STREAM);
      }
    }
  } else {
    if constexpr (ALIGNED) {
#pragma unroll
      for (int i = 0; i < K; i += 4) {
        const u32x4 v4 = {__float_as_uint(v[i]), __float_as_uint(v[i + 1]), __float_as_uint(v[i + 2]),
                          __float_as_uint(v[i + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(v4, r, voff + 4 * i, 0, STREAM);
      }
    } else {
#pragma unroll
      for (int i = 0; i < K; ++i) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[i]), r, voff + 4 * i, 0, STREAM);
    }
  }
}

// Window B / C staging: one io tensor's tile is WIN * NS values, moved as 16-byte chunks
// (a batch row of B or C is L * 16 io values, a multiple of 16 bytes, so a chunk is either
// wholly inside the row or wholly past its end and then reads as zeros).
template <typename IO, int THREADS>
struct TileChunks {
  static constexpr int EPC = 16 / sizeof(IO);          // io elements per chunk
  static constexpr int CHUNKS = WIN * NS / EPC;        // chunks per tensor per window
  static constexpr int PER_THREAD = (CHUNKS + THREADS - 1) / THREADS;
  uint32_t b[PER_THREAD][4], c[PER_THREAD][4];

  __device__ __forceinline__ void fetch(__amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rc) {
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int voff = (threadIdx.x + r * THREADS) * 16;
      const auto vb = __builtin_amdgcn_raw_buffer_load_b128(rb, voff, 0, 0);
      const auto vc = __builtin_amdgcn_raw_buffer_load_b128(rc, voff, 0, 0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        b[r][e] = vb[e];
        c[r][e] = vc[e];
      }
    }
  }

  __device__ __forceinline__ void store(Tile& tile) const {
#pragma unroll
    for (int r = 0; r < PER_THREAD; ++r) {
      const int ci = threadIdx.x + r * THREADS;
      if (CHUNKS % THREADS != 0 && ci >= CHUNKS) break;  // fetched (harmless) but not staged
      const int token = ci * EPC / NS;
      const int s0 = (ci * EPC) % NS;
      const int off = (token / K) * LANE_STRIDE + (token % K) * NS + s0;
#pragma unroll
      for (int e = 0; e < EPC; e += 4) {
        float4 fb, fc;
        fb.x = unpack<IO>(b[r], e);
        fb.y = unpack<IO>(b[r], e + 1);
        fb.z = unpack<IO>(b[r], e + 2);
        fb.w = unpack<IO>(b[r], e + 3);
        fc.x = unpack<IO>(c[r], e);
        fc.y = unpack<IO>(c[r], e + 1);
        fc.z = unpack<IO>(c[r], e + 2);
        fc.w = unpack<IO>(c[r], e + 3);
        *reinterpret_cast<float4*>(&tile.B[off + e]) = fb;
        *reinterpret_cast<float4*>(&tile.C[off + e]) = fc;
      }
    }
  }
};

template <typename IO, bool ALIGNED, int W, int G>
__global__ __launch_bounds__(W * WAVE) void prefill_windowed(ScanArgs a) {
  constexpr int THREADS = W * WAVE;
  __shared__ Tile tiles[2];  // window w reads tiles[w & 1] while window w + 1's goes into the other
  constexpr int ES = sizeof(IO);
  const int lane = threadIdx.x & (WAVE - 1);
  // Wave-uniform by construction; saying so keeps the row descriptors below in SGPRs (a
  // descriptor the compiler cannot prove uniform costs a readfirstlane loop per access).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  const int64_t groups = (a.D + W - 1) / W;
  const int64_t b = blockIdx.x / groups;
  const int64_t c = (blockIdx.x - b * groups) * W + wave;
  const bool active = c < a.D;  // a ragged last group: idle waves still stage tiles and meet barriers
  const int64_t L = a.L;                 // row stride of x, dt, z, y and B / C
  const int64_t cc = active ? c : 0;
  const int64_t row = b * a.D + cc;
  int64_t crow;                          // cache (h / conv) row
  if (!cache_row(a, b, cc, crow)) return;  // a skipped batch row: the whole workgroup leaves together
  const int64_t Lb = row_len(a, b);      // tokens to run for this batch row

  // Rows of the channel's streams and of the batch row's B / C; each window reads and writes
  // them through window_rsrc views.  An idle wave's y view is empty, so it stores nothing.
  const bool gate = a.z != nullptr;
  const IO* xrow = static_cast<const IO*>(a.x) + row * L;
  const IO* dtrow = static_cast<const IO*>(a.dt) + row * L;
  const IO* zrow = gate ? static_cast<const IO*>(a.z) + row * L : xrow;
  IO* yrow = static_cast<IO*>(a.y) + row * L;
  const int Li = (int)L;
  const int y_elems = active ? Li : 0;
  // B / C are viewed up to the row's own length only: a 16-byte chunk holds half a token (a
  // quarter for fp32), so the range check reads the tokens past the end as zeros, whatever
  // the tensors hold there (a ragged row's padding may hold anything, NaN included).
  const IO* Brow = static_cast<const IO*>(a.Bm) + b * L * NS;
  const IO* Crow = static_cast<const IO*>(a.Cm) + b * L * NS;
  const int bc_elems = (int)Lb * NS;

  // Channel constants.
  const float w0 = a.conv_w[cc * 4 + 0], w1 = a.conv_w[cc * 4 + 1], w2 = a.conv_w[cc * 4 + 2],
              w3 = a.conv_w[cc * 4 + 3];
  const float cb = a.conv_b ? a.conv_b[cc] : 0.0f;
  const float dtb = a.dt_bias[cc], dsk = a.Dskip[cc];
  float A2[NS], carry[NS];
#pragma unroll
  for (int n = 0; n < NS; ++n) {
    A2[n] = a.A[cc * NS + n] * kLog2e;
    carry[n] = a.h0 ? a.h0[crow * NS + n] : 0.0f;
  }
  float hist0 = 0.0f, hist1 = 0.0f, hist2 = 0.0f;  // raw x[t0-3], x[t0-2], x[t0-1]
  if (a.conv0) {
    hist0 = a.conv0[crow * 3 + 0];
    hist1 = a.conv0[crow * 3 + 1];
    hist2 = a.conv0[crow * 3 + 2];
  }
  const float init0 = hist0, init1 = hist1, init2 = hist2;

  const int nwin = (int)((Lb + WIN - 1) / WIN);
  const int voff = lane * K * ES;  // this lane's byte offset inside a window
  TileChunks<IO, THREADS> pf;
  Lanes<IO, ALIGNED> px, pdt, pz;
  pf.fetch(window_rsrc(Brow, bc_elems, 0), window_rsrc(Crow, bc_elems, 0));
  px.load(window_rsrc(xrow, Li, 0), voff);
  pdt.load(window_rsrc(dtrow, Li, 0), voff);
  if (gate) pz.load(window_rsrc(zrow, Li, 0), voff);

  pf.store(tiles[0]);
  for (int w = 0; w < nwin; ++w) {
    const int t0 = w * WIN;
    // One barrier per window: window w's tile (written at the end of window w-1) is visible,
    // and every wave is done reading tiles[(w+1) & 1] (window w-1's), which is refilled below.
    __syncthreads();
    const Tile& tile = tiles[w & 1];
    // The next window's inputs are prefetched while this one is computed.  With two waves per
    // SIMD (8-wave workgroups) x, dt and z are loaded at the window's start, into a second set of
    // registers; with three or four waves per SIMD x and dt are loaded right after the front end
    // has consumed this window's, and z after the gate, into the same registers (12 fewer
    // copies per window: 0.9-1.6% faster there, but 5% slower with two waves per SIMD, whose
    // loads issued mid-window are not covered by other waves' work).  Past the last window the
    // views are empty and those loads return zeros.
    constexpr bool kLateLoads = W > 8;
    const bool more = w + 1 < nwin;
    const int t1 = t0 + WIN;
    Lanes<IO, ALIGNED> cx, cdt, cz;
    if constexpr (!kLateLoads) {
      cx = px;
      cdt = pdt;
      cz = pz;
    }
    const Lanes<IO, ALIGNED>& ux = kLateLoads ? px : cx;
    const Lanes<IO, ALIGNED>& udt = kLateLoads ? pdt : cdt;
    const Lanes<IO, ALIGNED>& uz = kLateLoads ? pz : cz;
    if (more) {
      pf.fetch(window_rsrc(Brow, bc_elems, t1 * NS), window_rsrc(Crow, bc_elems, t1 * NS));
      if constexpr (!kLateLoads) {
        px.load(window_rsrc(xrow, Li, t1), voff);
        pdt.load(window_rsrc(dtrow, Li, t1), voff);
        if (gate) pz.load(window_rsrc(zrow, Li, t1), voff);
      }
    }
    if (!active) {
      if constexpr (kLateLoads) {
        px.load(window_rsrc(xrow, Li, t1), voff);
        pdt.load(window_rsrc(dtrow, Li, t1), voff);
        if (gate) pz.load(window_rsrc(zrow, Li, t1), voff);
      }
      if (more) pf.store(tiles[(w + 1) & 1]);
      continue;
    }

    // ---- front end: conv window, SiLU, softplus ----
    const int64_t left = Lb - t0;  // >= 1, uniform
    const int rem = left < WIN ? (int)left : WIN;
    const int nvalid = rem - lane * K < 0 ? 0 : (rem - lane * K > K ? K : rem - lane * K);
    float xv[K];
#pragma unroll
    for (int j = 0; j < K; ++j) xv[j] = unpack<IO>(ux.w, j);
    const float xm3 = dpp<DPP_WAVE_SHR1, 0xf>(hist0, xv[K - 3]);
    const float xm2 = dpp<DPP_WAVE_SHR1, 0xf>(hist1, xv[K - 2]);
    const float xm1 = dpp<DPP_WAVE_SHR1, 0xf>(hist2, xv[K - 1]);
    hist0 = lane63(xv[K - 3]);
    hist1 = lane63(xv[K - 2]);
    hist2 = lane63(xv[K - 1]);

    float dl[K], du[K], yv[K];
    float dsum;
    // Past the row end the step is the identity: delta is exactly 0 (softplus(-inf)) and so is
    // the drive delta * u, selected rather than multiplied, since u there is made of whatever
    // the tensors hold past the row (NaN and infinities included).  The tile's B there is
    // zero too (read through the B / C views, which end at the row's length).  Only a window that reaches past the end needs this per-token
    // selection (a uniform branch picks it).
    auto front = [&](auto masked) {
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const bool pad = decltype(masked)::value && j >= nvalid;
        const float s3 = j >= 3 ? xv[j - 3] : (j == 0 ? xm3 : (j == 1 ? xm2 : xm1));
        const float s2 = j >= 2 ? xv[j - 2] : (j == 0 ? xm2 : xm1);
        const float s1 = j >= 1 ? xv[j - 1] : xm1;
        const float v = fmaf(w3, xv[j], fmaf(w2, s1, fmaf(w1, s2, fmaf(w0, s3, cb))));
        const float u = silu(v);
        const float arg = unpack<IO>(udt.w, j) + dtb;
        const float d = softplus(pad ? -__builtin_inff() : arg);
        dl[j] = d;
        du[j] = pad ? 0.0f : d * u;
        yv[j] = dsk * u;
        dsum = j == 0 ? d : dsum + d;
      }
    };
    // With two waves per SIMD (8-state groups) the front end, too, runs at raised priority:
    // measured 2% faster there, and ~0.5% slower with three or four waves.
    if constexpr (G == 8) __builtin_amdgcn_s_setprio(1);
    if (rem == WIN) front(std::integral_constant<bool, false>{});
    else front(std::integral_constant<bool, true>{});
    if constexpr (G == 8) __builtin_amdgcn_s_setprio(0);
    if constexpr (kLateLoads) {
      px.load(window_rsrc(xrow, Li, t1), voff);
      pdt.load(window_rsrc(dtrow, Li, t1), voff);
    }

    // ---- state groups: local pairs, lane scan, replay ----
    const float* tb = &tile.B[lane * LANE_STRIDE];
    const float* tcp = &tile.C[lane * LANE_STRIDE];
#pragma unroll
    for (int q0 = 0; q0 < NS; q0 += G) {
      float av[K][G], bv[K][G], P[G], H[G];
#pragma unroll
      for (int q = 0; q < G; ++q) P[q] = hw_exp2(A2[q0 + q] * dsum);  // prod_j exp(delta_j A) over this lane's tokens
      float hc[G], cg[G];
#pragma unroll
      for (int q = 0; q < G; ++q) cg[q] = carry[q0 + q];
      // The fold reads each token's B one token ahead (bn), so that each tile read has a token's
      // work before its first use, and computes each decay's argument before its exponential,
      // so that no exponential waits on the multiply just before it (against reading and using
      // in the same token: 375 -> 359 us on slice7b, with the replay's read-ahead below).  With
      // 8-state groups (two waves per SIMD, which reach the fold together) or 2-state groups,
      // all arguments of the group come first (after its first B read), then all its exponentials,
      // then the drives and pair updates token by token: the two waves' transcendentals run back
      // to back and their plain work pairs up afterwards (slice7b 359 -> 350 us, 16-channel shape
      // -1%); with 4-state groups that ordering was 0.3-1% slower, so the arguments and
      // exponentials stay with their token there.
      constexpr bool kExpBurst = G != 4;
      float bn[G];
      tile_states<G>(tb + q0, bn);
      if constexpr (kExpBurst) {
#pragma unroll
        for (int j = 0; j < K; ++j)
#pragma unroll
          for (int q = 0; q < G; ++q) av[j][q] = dl[j] * A2[q0 + q];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < K; ++j)
#pragma unroll
          for (int q = 0; q < G; ++q) av[j][q] = hw_exp2(av[j][q]);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < K; ++j) {
        float bq[G];
#pragma unroll
        for (int q = 0; q < G; ++q) bq[q] = bn[q];
        if (j + 1 < K) tile_states<G>(tb + (j + 1) * NS + q0, bn);
        keep_lds_reads_here();
        if constexpr (!kExpBurst) {
#pragma unroll
          for (int q = 0; q < G; ++q) av[j][q] = dl[j] * A2[q0 + q];
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int q = 0; q < G; ++q) {
          if constexpr (!kExpBurst) av[j][q] = hw_exp2(av[j][q]);
          bv[j][q] = du[j] * bq[q];
        }
        if (j == 0) seed_carry<G>(bv[0], av[0], cg);
        // The first token's pair is its own drive (the state reached from zero).
#pragma unroll
        for (int q = 0; q < G; ++q) H[q] = j == 0 ? bv[0][q] : fmaf(av[j][q], H[q], bv[j][q]);
      }
      // The replay's first C read goes out before the lane scan, which hides its latency.
      float cn[G];
      tile_states<G>(tcp + q0, cn);
      // The lane scan is a chain of dependent DPP steps; raising the wave's issue priority for it
      // lets the other waves of the SIMD fill the gaps with their (independent) fold and replay
      // work instead of the reverse (3-4% faster with three or four waves per SIMD).
      __builtin_amdgcn_s_setprio(2);
      scan_group<G>(P, H, cg, hc);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int q = 0; q < G; ++q) carry[q0 + q] = cg[q];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        float cq[G];
#pragma unroll
        for (int q = 0; q < G; ++q) cq[q] = cn[q];
        if (j + 1 < K) tile_states<G>(tcp + (j + 1) * NS + q0, cn);
        keep_lds_reads_here();
#pragma unroll
        for (int q = 0; q < G; ++q) {
          hc[q] = fmaf(av[j][q], hc[q], bv[j][q]);
          yv[j] = fmaf(cq[q], hc[q], yv[j]);
        }
      }
    }

    if (gate) {
#pragma unroll
      for (int j = 0; j < K; ++j) yv[j] *= silu(unpack<IO>(uz.w, j));
    }
    if constexpr (kLateLoads) {
      if (gate) pz.load(window_rsrc(zrow, Li, t1), voff);
    }
    if (more) pf.store(tiles[(w + 1) & 1]);
    store_lanes<IO, ALIGNED>(window_rsrc(yrow, y_elems, t0), voff, yv, nvalid);
  }

  if (active && lane == 0) {
#pragma unroll
    for (int n = 0; n < NS; ++n) a.h_out[crow * NS + n] = carry[n];
    const float init[3] = {init0, init1, init2};
    const IO* xr = static_cast<const IO*>(a.x) + row * L;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int64_t t = Lb - 3 + j;  // raw input xi[Lb-3+j]; history below zero
      a.conv_out[crow * 3 + j] = t >= 0 ? to_f32(xr[t]) : init[t + 3];
    }
  }
}

}  // namespace

// Buffer offsets are 32-bit: a batch row of B / C (L * 16 io values) must stay below 2 GiB.
bool windowed_supported(const ScanArgs& a) {
  const int64_t es = a.bf16 ? 2 : 4;
  return a.N == NS && a.L * NS * es < ((int64_t)1 << 31) - WIN * NS * es;
}

template <typename IO, bool ALIGNED, int W, int G>
void launch_shape(const ScanArgs& a, hipStream_t s) {
  const int64_t groups = (a.D + W - 1) / W;
  const dim3 grid((unsigned)(a.B * groups)), block(W * WAVE);
  prefill_windowed<IO, ALIGNED, W, G><<<grid, block, 0, s>>>(a);
}

// The bf16 workgroup width for this launch (see the shape table above).
int bf16_width(const ScanArgs& a) {
  if (a.L % 8 != 0) return 8;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 8;
  int best = 8;
  double best_cost = 0.0;
  for (const ShapeCost& sh : kShapes) {
    const int64_t wgs = a.B * ((a.D + sh.w - 1) / sh.w);
    const double cost = (double)((wgs + cus - 1) / cus) * sh.round_time;
    if (sh.w == 8 || cost < best_cost) {
      best = sh.w;
      best_cost = cost;
    }
  }
  return best;
}

hipError_t launch_windowed(const ScanArgs& a, hipStream_t s) {
  if (a.bf16) {
    switch (bf16_width(a)) {  // 12 and 16 only for aligned rows
      case 16: launch_shape<bf16_t, true, 16, 2>(a, s); break;
      case 12: launch_shape<bf16_t, true, 12, 4>(a, s); break;
      default:
        if (a.L % 8 == 0) launch_shape<bf16_t, true, 8, 8>(a, s);
        else launch_shape<bf16_t, false, 8, 8>(a, s);
    }
  } else if (a.L % 4 == 0) {
    launch_shape<float, true, 8, 4>(a, s);
  } else {
    launch_shape<float, false, 8, 4>(a, s);
  }
  return hipGetLastError();
}

}  // namespace ssm
