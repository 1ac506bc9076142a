// Decode path of the W4A16 linear layer (small M): weights streamed from HBM
// once with 16-byte loads, dequantised in registers, multiplied on the gfx950
// matrix cores, fp32 accumulation.
//
// This is the generation-stage kernel of "TinyChat: Efficient and Lightweight
// Chatbot with AWQ" (section "Speed Benchmarks": INT4 weights with a W4A16 GPU
// kernel; latency reported per generated token). Decode reads every weight
// once per token, so the kernel is bound by HBM bandwidth: the work per
// weight must stay far below the vector ALU budget (about 2.5 lane-operations
// per weight at 8 TB/s on 256 CUs at 2.4 GHz).
//
// Design
//   * A workgroup owns one 16-column tile of the device layout; its WAVES
//     waves split the K range, taking the 128-row tiles in turn (wave w reads
//     tiles w, w + WAVES, ...), so a workgroup streams WAVES consecutive KiB at
//     a time. One 64-lane 16-byte load brings a whole 1 KiB tile.
//   * Lane l holds column l%16 and rows 8(l/16) + 32j .. +7 (j = 0..3) of a
//     tile: exactly the B operand of v_mfma_f32_16x16x32_f16 for the four
//     32-row blocks of the tile. The activation rows form the A operand (rows
//     beyond M are zero), so one MFMA covers 16 rows of x at no extra cost:
//     the same kernel serves M = 1..16 per 16-row tile, up to four tiles.
//   * Per word: 1 shift, 4 mask-and-or, 4 packed fp16 subtractions give the
//     exact (q - z) as fp16 (0.6 VALU operations per weight). The per-group
//     scale is applied once per group to the fp32 MFMA result.
//   * Activations, scales and zero points are read with raw buffer loads:
//     rows >= M and columns >= N get an out-of-range offset and read as zero,
//     so the loop has no branches. All loads of a tile are issued together,
//     DEPTH tiles ahead; the loop body is branch-free, so the in-order
//     vector-memory counter lets each wave wait only for the tile it consumes.
//     Past a wave's last tile the prefetch index is clamped (a cache hit) and
//     the consumed result is scaled by zero.
//   * A ragged last tile (K not a multiple of 128) is handled after the loop
//     with explicit row masks.
//   * The waves' fp32 results are summed through LDS and stored as fp16.
//   * Workgroup ids are remapped so neighbouring tiles run on the same XCD and
//     share its L2 for scales, zero points and activations.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

// Groups per 128-row tile: GPT = 4 (G = 32), 2 (G = 64), 1 (G = 128) or
// 0 (G a larger multiple of 128: several tiles per group).
template <int MT, int GPT>
struct Bundle {
  u4 wq;             // one 16-byte slice of the tile: 4 words
  u4 xa[MT][4];      // A operand: 8 fp16 of x per 32-row block and 16-row tile
  uint32_t s[GPT > 0 ? GPT : 1];   // scale bits per group in the tile
  uint32_t zw[GPT > 0 ? GPT : 1];  // packed zero-point word per group
};

struct DecodeCtx {
  rsrc_t rx, rs, rz;
  const u4* qcol;       // first 16-byte slice of this lane in the column tile
  uint32_t xoff[4];     // per 16-row tile: byte offset of (row, 8h) or kOOB
  uint32_t soff, zoff;  // byte offsets of this lane's scale / zero word, or kOOB
  uint32_t srow, zrow;  // bytes per group row of scales / zeros
  int tpg;              // 128-row tiles per group (GPT == 0)
};

template <int MT, int GPT>
__device__ __forceinline__ void load_bundle(Bundle<MT, GPT>& b, const DecodeCtx& c, int kt) {
  b.wq = c.qcol[(int64_t)kt * 64];
  constexpr int NG = GPT > 0 ? GPT : 1;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const uint32_t g = GPT == 0 ? (uint32_t)kt / (uint32_t)c.tpg : (uint32_t)(kt * GPT + gi);
    b.s[gi] = __builtin_amdgcn_raw_buffer_load_b16(c.rs, c.soff + g * c.srow, 0, 0);
    b.zw[gi] = __builtin_amdgcn_raw_buffer_load_b32(c.rz, c.zoff + g * c.zrow, 0, 0);
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b.xa[mt][j] = __builtin_bit_cast(
          u4, __builtin_amdgcn_raw_buffer_load_b128(c.rx, c.xoff[mt] + 256u * (uint32_t)kt + 64u * j, 0, 0));
}

template <int MT, int GPT>
__device__ __forceinline__ void consume_bundle(const Bundle<MT, GPT>& b, f4 (&acc)[MT], int col, float valid) {
  constexpr int NG = GPT > 0 ? GPT : 1;
  constexpr int JPG = 4 / NG;  // 32-row blocks per group inside the tile
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const ZeroConst zc = zero_const(zero_nibble(b.zw[gi], col));
    f4 accg[MT];
#pragma unroll
    for (int jj = 0; jj < JPG; ++jj) {
      const int j = gi * JPG + jj;
      const h8 bw = decode_diff(b.wq[j], zc);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        accg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, b.xa[mt][j]), bw,
                                                          jj == 0 ? f4{0.f, 0.f, 0.f, 0.f} : accg[mt], 0, 0, 0);
    }
    const float sf = valid * (float)__builtin_bit_cast(_Float16, (uint16_t)b.s[gi]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] += sf * accg[mt];
  }
}

template <int MT, int GPT, int WAVES, int DEPTH>
__global__ __launch_bounds__(64 * WAVES) void decode_kernel(const uint16_t* __restrict__ x,
                                                            const u4* __restrict__ qw,
                                                            const uint16_t* __restrict__ scales,
                                                            const uint32_t* __restrict__ zeros,
                                                            uint16_t* __restrict__ y, int M, int K, int N, int G,
                                                            int KT) {
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int h = lane >> 4;
  const int col = 16 * t + (lane & 15);
  const int groups = K / G;

  DecodeCtx c;
  c.rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  c.rs = make_rsrc(scales, (uint32_t)groups * (uint32_t)N * 2u);
  c.rz = make_rsrc(zeros, (uint32_t)groups * (uint32_t)(N / 8) * 4u);
  c.qcol = qw + (int64_t)t * KT * 64 + lane;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int row = 16 * mt + (lane & 15);
    c.xoff[mt] = row < M ? (uint32_t)(row * K + 8 * h) * 2u : kOOB;
  }
  c.soff = col < N ? (uint32_t)col * 2u : kOOB;
  c.zoff = col < N ? (uint32_t)(col >> 3) * 4u : kOOB;
  c.srow = (uint32_t)N * 2u;
  c.zrow = (uint32_t)(N / 8) * 4u;
  c.tpg = G / 128;

  const int KTF = K / 128;  // full 128-row tiles
  const int n_my = KTF > w ? (KTF - w + WAVES - 1) / WAVES : 0;
  const int last = w + WAVES * (n_my - 1);

  f4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f4{0.f, 0.f, 0.f, 0.f};

  if (n_my > 0) {
    Bundle<MT, GPT> buf[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) load_bundle<MT, GPT>(buf[d], c, min(w + WAVES * d, last));
    const int rounds = (n_my + DEPTH - 1) / DEPTH;
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int i = r * DEPTH + d;
        consume_bundle<MT, GPT>(buf[d], acc, col, i < n_my ? 1.f : 0.f);
        load_bundle<MT, GPT>(buf[d], c, min(w + WAVES * (i + DEPTH), last));
      }
    }
  }

  // Ragged last tile: rows K .. 128*KT-1 are padding. Its activation loads
  // are masked per 32-row block; padding blocks also read zero scales and
  // zero points (their group index is out of range), so they add nothing.
  if (KTF < KT && w == (KTF % WAVES)) {
    Bundle<MT, GPT> b;
    load_bundle<MT, GPT>(b, c, KTF);
    const int valid_blocks = (K - 128 * KTF) / 32;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j >= valid_blocks) b.xa[mt][j] = u4{0u, 0u, 0u, 0u};
    consume_bundle<MT, GPT>(b, acc, col, 1.f);
  }

  // Sum the waves' partial tiles. Lane l, register r of 16-row tile mt holds
  // output row 16mt + 4(l/16) + r, column 16t + l%16.
  if constexpr (WAVES > 1) {
    constexpr int OUTS = MT * 4 * 64;
    __shared__ float red[WAVES][OUTS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[w][(mt * 4 + r) * 64 + lane] = acc[mt][r];
    __syncthreads();
    for (int o = threadIdx.x; o < OUTS; o += 64 * WAVES) {
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) v += red[ww][o];
      const int ol = o & 63, mr = o >> 6;
      const int row = 16 * (mr >> 2) + 4 * (ol >> 4) + (mr & 3);
      const int cc = 16 * t + (ol & 15);
      if (row < M && cc < N) y[(int64_t)row * N + cc] = __builtin_bit_cast(uint16_t, (_Float16)v);
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mt + 4 * h + r;
        const float v = acc[mt][r];
        if (row < M && col < N) y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
  }
}

template <int MT, int GPT, int WAVES>
static hipError_t launch_decode_t(const LinearArgs& a, const Launch& L) {
  constexpr int DEPTH = MT == 1 ? 4 : (MT == 2 ? 3 : 2);
  const int KT = (a.K + 127) / 128;
  const int NT = (a.N + 15) / 16;
  return launch_kernel(decode_kernel<MT, GPT, WAVES, DEPTH>, dim3((unsigned)NT), dim3(64 * WAVES), L, a.x,
                       reinterpret_cast<const u4*>(a.qw), a.scales, a.zeros, a.y, a.M, a.K, a.N, a.G, KT);
}

template <int MT, int GPT>
static hipError_t launch_decode_w(const LinearArgs& a, int waves, const Launch& L) {
  switch (waves) {
    case 1: return launch_decode_t<MT, GPT, 1>(a, L);
    case 2: return launch_decode_t<MT, GPT, 2>(a, L);
    case 4: return launch_decode_t<MT, GPT, 4>(a, L);
    case 8: return launch_decode_t<MT, GPT, 8>(a, L);
    case 16: return launch_decode_t<MT, GPT, 16>(a, L);
  }
  return hipErrorInvalidValue;
}

template <int MT>
static hipError_t launch_decode_g(const LinearArgs& a, int waves, const Launch& L) {
  if (a.G == 32) return launch_decode_w<MT, 4>(a, waves, L);
  if (a.G == 64) return launch_decode_w<MT, 2>(a, waves, L);
  if (a.G == 128) return launch_decode_w<MT, 1>(a, waves, L);
  return launch_decode_w<MT, 0>(a, waves, L);
}

hipError_t launch_decode(const LinearArgs& a, int waves, const Launch& L) {
  if (a.M <= 16) return launch_decode_g<1>(a, waves, L);
  if (a.M <= 32) return launch_decode_g<2>(a, waves, L);
  if (a.M <= 64) return launch_decode_g<4>(a, waves, L);
  return hipErrorInvalidValue;
}

}  // namespace awq
