// Decode path of the W4A16 linear layer (small M): weights streamed from HBM
// once with 16-byte loads, dequantised in registers, multiplied on the gfx950
// matrix cores, fp32 accumulation.
//
// This is the generation-stage kernel of "TinyChat: Efficient and Lightweight
// Chatbot with AWQ" (section "Speed Benchmarks": INT4 weights with a W4A16 GPU
// kernel; latency reported per generated token). Decode reads every weight
// once per token, so the kernel is bound by HBM bandwidth and by the number
// of memory requests: each 128-row weight tile must cost one 16-byte load per
// lane and little vector-ALU work (the budget is about 2.5 lane-operations per
// weight at 8 TB/s on 256 CUs at 2.4 GHz).
//
// Design
//   * A workgroup owns TPW 16-column tiles of the device layout; its WAVES
//     waves split the K range, taking the 128-row bands in turn (wave w reads
//     bands w, w + WAVES, ...). Tiles of one band are adjacent in memory, so
//     at any moment the workgroups read a contiguous stretch of the matrix.
//     One 64-lane 16-byte load brings a whole 1 KiB tile.
//   * Lane l holds column l%16 and rows 8(l/16) + 32j .. +7 (j = 0..3) of a
//     tile: exactly the B operand of v_mfma_f32_16x16x32_f16 for the four
//     32-row blocks of the tile. The activation rows form the A operand, so
//     one MFMA covers 16 rows of x at no extra cost.
//   * Per word: 1 shift, 4 mask-and-or (v_and_or_b32), 4 packed fp16
//     subtractions give the exact (q - z) as fp16. The per-group scale is
//     applied once per group to the fp32 MFMA result.
//   * Staged variant (M <= 16 and the activations fit in LDS): at the start
//     each workgroup copies the activation rows into LDS; the loop reads the
//     A operand from there. Each band's scale and packed zero word are loaded
//     into registers right before the band's weights, DEPTH bands ahead, so
//     they arrive in order with the weights (measured: staging them up front
//     made every workgroup wait several microseconds for them behind the
//     whole chip's weight stream).
//   * Streamed variant (larger M or K): activations, scales and zero points
//     are read per tile with raw buffer loads.
//   * Rows >= M and columns >= N read as zero (out-of-range buffer offsets) or
//     are never stored, so loops have no data-dependent branches; past a
//     wave's last tile the prefetch index is clamped and the result is scaled
//     by zero. A ragged last band (K not a multiple of 128) runs through the
//     loop like the others: its activations past K are zero (zero padding of
//     the staged rows; out-of-range loads in the streamed variant), and its
//     padding rows hold code 0 with the last group's (finite) scale.
//   * The waves' fp32 results are summed through LDS in a fixed order and
//     stored as fp16. Workgroup ids are remapped so neighbouring tiles run on
//     the same XCD.
#include <algorithm>

#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

// Groups per 128-row band: GPT = 4 (G = 32), 2 (G = 64), 1 (G = 128) or 0 (G a
// larger multiple of 128: several bands per group).
template <int GPT>
struct GroupsPerBand {
  static constexpr int NG = GPT > 0 ? GPT : 1;  // group entries per band
  static constexpr int JPG = 4 / NG;            // 32-row blocks per group entry
  __device__ static __forceinline__ uint32_t group(int kt, int gi, int tpg) {
    return GPT == 0 ? (uint32_t)kt / (uint32_t)tpg : (uint32_t)(kt * GPT + gi);
  }
};

// Weights are read exactly once per call: non-temporal loads stream them
// past the caches.
__device__ __forceinline__ u4 load_weights(const u4* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ float scale_of(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// ---------------------------------------------------------------------------
// Staged variant
// ---------------------------------------------------------------------------

struct StagedLayout {
  uint32_t x_row;        // bytes per staged activation row (K zero-padded to whole bands, + 16)
  uint32_t x_chunks;     // 16-byte chunks per staged row
  uint32_t scratch_off;  // per-thread 16-byte slots for masked staging stores
};

// Weights of one band for TPW column tiles and their groups' scale bits and
// packed zero words (lane l: column l % 16 of each tile).
template <int TPW, int NG>
struct BandBuf {
  u4 wq[TPW];
  uint32_t s[TPW][NG];
  uint32_t zw[TPW][NG];
};

// TM: 1 = one 16-column tile per workgroup, 2 = two adjacent tiles, 3 = the
// gated epilogue: tile t of the first half of the columns (gate) and tile t
// of the second half (up) in one workgroup, the first WAVES/2 waves on the
// gate tile and the others on the up tile (each wave holds one tile, so the
// register footprint is that of TM = 1), stored as y[m, n] = silu(gate) * up.
template <int TM, int GPT, int WAVES, int DEPTH, int S>
__device__ __forceinline__ void decode_staged_body(const uint16_t* __restrict__ x, const u4* __restrict__ qw,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint32_t* __restrict__ zeros, uint16_t* __restrict__ y,
                                                   int M, int K, int N, int G, int NT, StagedLayout lay) {
  using GB = GroupsPerBand<GPT>;
  constexpr int TPW = TM == 2 ? 2 : 1;
  constexpr bool GATED = TM == 3;
  static_assert(!GATED || WAVES % 2 == 0, "gated: an even number of waves");
  constexpr int WK = GATED ? WAVES / 2 : WAVES;  // waves that split one tile's K range
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int NTH = 64 * WAVES;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // gated: waves WK.. take the up tile, NT/2 tiles after the gate tile
  const int w = GATED ? wid % WK : wid;
  const int t0 = GATED ? wg + (wid >= WK ? NT / 2 : 0) : wg * TPW;
  const int h = lane >> 4;
  const int groups = K / G;
  const int tpg = G / 128;
  const int KT = (K + 127) / 128;

  const rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const rsrc_t rs = make_rsrc(scales, (uint32_t)groups * (uint32_t)N * 2u);
  const rsrc_t rz = make_rsrc(zeros, (uint32_t)groups * (uint32_t)(N / 8) * 4u);

  // 1. Staging loads (activations), issued first: they come from L2 and are
  //    waited for before the weight stream is.
  const uint32_t x_total = (uint32_t)M * lay.x_chunks;
  u4 xv[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const uint32_t e = threadIdx.x + i * NTH;
    const uint32_t row = e / lay.x_chunks, cc = e - row * lay.x_chunks;
    const bool ok = e < x_total && cc * 8u < (uint32_t)K;
    xv[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? (row * K + cc * 8u) * 2u : kOOB, 0, 0));
  }

  // 2. Weight prefetch: per band, the scale and zero word of each of the
  //    lane's columns, then one 16-byte load per lane per tile, DEPTH bands
  //    ahead. The band index is clamped to the wave's last band (band 0 when
  //    it has none, which always exists), so the prefetch is unconditional
  //    and the waits before the staging stores cover only the staging loads.
  //    Offsets are below 2^31, so setting bit 31 makes a masked load read
  //    zero; group indices are clamped to the last group (a ragged band's
  //    missing groups are then never used with nonzero weight).
  const int n_my = KT > w ? (KT - w + WK - 1) / WK : 0;
  const int last = max(w + WK * (n_my - 1), 0);
  const u4* qcol[TPW];
  uint32_t soff[TPW], zoff[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int ti = t0 + tt;
    qcol[tt] = qw + (int64_t)min(ti, NT - 1) * 64 + lane;
    const uint32_t col = 16u * ti + (lane & 15u);
    const uint32_t bad = (uint32_t)!(col < (uint32_t)N) << 31;
    soff[tt] = (col * 2u) | bad;
    zoff[tt] = ((col >> 3) * 4u) | bad;
  }
  const int64_t band = (int64_t)NT * 64;
  const uint32_t srow = (uint32_t)N * 2u, zrow = (uint32_t)(N / 8) * 4u;
  // Two groups per band (G = 64): lanes 0..31 load the first group's scale
  // and zero word, lanes 32..63 (the same columns) the second's; a swap of
  // the two half-waves at use gives every lane both (one load each instead
  // of two).
  constexpr int NL = GPT == 2 ? 1 : GB::NG;  // scale/zero entries loaded per band
  auto load_band = [&](BandBuf<TPW, NL>& b, int kt) {
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
#pragma unroll
      for (int gi = 0; gi < NL; ++gi) {
        const uint32_t g = GPT == 2 ? min((uint32_t)(2 * kt) + (uint32_t)(lane >> 5), (uint32_t)groups - 1u)
                                    : min(GB::group(kt, gi, tpg), (uint32_t)groups - 1u);
        b.s[tt][gi] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff[tt] + g * srow, 0, 0);
        b.zw[tt][gi] = __builtin_amdgcn_raw_buffer_load_b32(rz, zoff[tt] + g * zrow, 0, 0);
      }
      b.wq[tt] = load_weights(qcol[tt] + kt * band);
    }
  };
  BandBuf<TPW, NL> buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_band(buf[d], min(w + WK * d, last));

  // 3. Staging stores (masked ones go to this thread's scratch slot) and barrier.
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const uint32_t e = threadIdx.x + i * NTH;
    const uint32_t row = e / lay.x_chunks, cc = e - row * lay.x_chunks;
    const uint32_t xa = e < x_total ? row * lay.x_row + cc * 16u : lay.scratch_off + threadIdx.x * 16u;
    *reinterpret_cast<u4*>(smem + xa) = xv[i];
  }
  __syncthreads();

  // 4. Main loop over full bands.
  const DecodeConsts kc = decode_consts();
  const int rowc = min(lane & 15, M - 1);  // rows >= M read row M-1; never stored
  const char* xrow = smem + rowc * lay.x_row + 16 * h;
  f4 acc[TPW];
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) acc[tt] = f4{0.f, 0.f, 0.f, 0.f};

  const int lcol = lane & 15;  // column within a tile (16-column tiles start at multiples of 8)
  auto consume = [&](const BandBuf<TPW, NL>& b, int kt, float valid) {
    h8 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *reinterpret_cast<const h8*>(xrow + 256 * kt + 64 * j);
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
      uint32_t sv[GB::NG], zv[GB::NG];
      if constexpr (GPT == 2) {
        const auto sp = __builtin_amdgcn_permlane32_swap(b.s[tt][0], b.s[tt][0], false, false);
        const auto zp = __builtin_amdgcn_permlane32_swap(b.zw[tt][0], b.zw[tt][0], false, false);
        sv[0] = sp[0], sv[1] = sp[1], zv[0] = zp[0], zv[1] = zp[1];
      } else {
#pragma unroll
        for (int gi = 0; gi < GB::NG; ++gi) sv[gi] = b.s[tt][gi], zv[gi] = b.zw[tt][gi];
      }
#pragma unroll
      for (int gi = 0; gi < GB::NG; ++gi) {
        const ZeroConst zc = zero_const(zero_nibble(zv[gi], lcol));
        f4 accg;
#pragma unroll
        for (int jj = 0; jj < GB::JPG; ++jj) {
          const int j = gi * GB::JPG + jj;
          accg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], decode_diff_vk(b.wq[tt][j], zc, kc),
                                                        jj == 0 ? f4{0.f, 0.f, 0.f, 0.f} : accg, 0, 0, 0);
        }
        acc[tt] += (valid * scale_of(sv[gi])) * accg;
      }
    }
  };

  // Unconditional loop: a wave without bands runs one round scaled by zero on
  // band 0 (a branch around the loop would let the compiler sink the weight
  // prefetch below the barrier).
  const int rounds = max((n_my + DEPTH - 1) / DEPTH, 1);
  for (int r = 0; r < rounds - 1; ++r) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int i = r * DEPTH + d;
      consume(buf[d], w + WK * i, 1.f);
      load_band(buf[d], min(w + WK * (i + DEPTH), last));
    }
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    const int i = (rounds - 1) * DEPTH + d;
    consume(buf[d], min(w + WK * i, last), i < n_my ? 1.f : 0.f);
  }

  // 5. Sum the waves' results through LDS (the staging area is reused) and
  //    store. Lane l, register r of tile tt holds output row 4(l/16) + r,
  //    column 16(t0 + tt) + l%16.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[((wid * TPW + tt) * 4 + r) * 64 + lane] = acc[tt][r];
  __syncthreads();
  if constexpr (GATED) {
    // gate: waves 0 .. WK-1, up: waves WK .. WAVES-1, same (row, column) at the same offset
    const int NO = N / 2;
    for (int o = threadIdx.x; o < 256; o += NTH) {
      float vg = 0.f, vu = 0.f;
#pragma unroll
      for (int ww = 0; ww < WK; ++ww) vg += red[ww * 256 + o], vu += red[(WK + ww) * 256 + o];
      const int ol = o & 63, r = o >> 6;
      const int row = 4 * (ol >> 4) + r;
      const int cc = 16 * wg + (ol & 15);
      if (row < M && cc < NO) y[(int64_t)row * NO + cc] = __builtin_bit_cast(uint16_t, (_Float16)(vg / (1.f + expf(-vg)) * vu));
    }
  } else {
    for (int o = threadIdx.x; o < TPW * 256; o += NTH) {
      float v = 0.f;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) v += red[ww * TPW * 256 + o];
      const int ol = o & 63, r = (o >> 6) & 3, tt = o >> 8;
      const int row = 4 * (ol >> 4) + r;
      const int cc = 16 * (t0 + tt) + (ol & 15);
      if (row < M && cc < N) y[(int64_t)row * N + cc] = __builtin_bit_cast(uint16_t, (_Float16)v);
    }
  }
}

template <int TM, int GPT, int WAVES, int DEPTH, int S>
__global__ __launch_bounds__(64 * WAVES) void decode_staged_kernel(const uint16_t* __restrict__ x,
                                                                   const u4* __restrict__ qw,
                                                                   const uint16_t* __restrict__ scales,
                                                                   const uint32_t* __restrict__ zeros,
                                                                   uint16_t* __restrict__ y, int M, int K, int N,
                                                                   int G, int NT, StagedLayout lay) {
  decode_staged_body<TM, GPT, WAVES, DEPTH, S>(x, qw, scales, zeros, y, M, K, N, G, NT, lay);
}

// The same kernel held to 64 VGPRs, i.e. eight waves per SIMD, so that four
// 8-wave (or two 16-wave) workgroups fit on a CU; used only for the
// instantiations that compile without spills (see launch_staged_s).
template <int TM, int GPT, int WAVES, int DEPTH, int S>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(8))) void decode_staged_kernel_o8(
    const uint16_t* __restrict__ x, const u4* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint32_t* __restrict__ zeros, uint16_t* __restrict__ y, int M, int K, int N, int G, int NT,
    StagedLayout lay) {
  decode_staged_body<TM, GPT, WAVES, DEPTH, S>(x, qw, scales, zeros, y, M, K, N, G, NT, lay);
}

// ---------------------------------------------------------------------------
// Streamed variant
// ---------------------------------------------------------------------------

template <int MT, int GPT, int TW>
struct Bundle {
  u4 wq[TW];                                // one 16-byte slice of each tile: 4 words
  u4 xa[MT][4];                             // A operand per 32-row block and 16-row tile
  uint32_t s[TW][GroupsPerBand<GPT>::NG];   // scale bits per tile and group entry
  uint32_t zw[TW][GroupsPerBand<GPT>::NG];  // packed zero-point word per tile and group entry
};

template <int TW>
struct StreamCtx {
  rsrc_t rx, rs, rz;
  const u4* qcol[TW];       // this lane's slice of each column tile in band 0
  int64_t band;             // u4 stride between bands
  uint32_t xoff[4];         // per 16-row tile: byte offset of (row, 8h) or kOOB
  uint32_t soff[TW], zoff[TW];  // byte offsets of this lane's scale / zero word, or kOOB
  uint32_t srow, zrow;      // bytes per group row of scales / zeros
  int tpg;
  int K;
};

template <int MT, int GPT, int TW>
__device__ __forceinline__ void load_bundle(Bundle<MT, GPT, TW>& b, const StreamCtx<TW>& c, int kt) {
  using GB = GroupsPerBand<GPT>;
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) {
    b.wq[tt] = load_weights(c.qcol[tt] + kt * c.band);
#pragma unroll
    for (int gi = 0; gi < GB::NG; ++gi) {
      const uint32_t g = GB::group(kt, gi, c.tpg);
      b.s[tt][gi] = __builtin_amdgcn_raw_buffer_load_b16(c.rs, c.soff[tt] + g * c.srow, 0, 0);
      b.zw[tt][gi] = __builtin_amdgcn_raw_buffer_load_b32(c.rz, c.zoff[tt] + g * c.zrow, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // 32-row blocks past K (in a ragged last band) read zero activations
    const bool blk = 128 * kt + 32 * j < c.K;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      b.xa[mt][j] = __builtin_bit_cast(
          u4, __builtin_amdgcn_raw_buffer_load_b128(c.rx, blk ? c.xoff[mt] + 256u * (uint32_t)kt + 64u * j : kOOB,
                                                    0, 0));
  }
}

// The activation fragments of a band are loaded once and used for all TW
// column tiles of the workgroup.
template <int MT, int GPT, int TW>
__device__ __forceinline__ void consume_bundle(const Bundle<MT, GPT, TW>& b, f4 (&acc)[TW][MT], int col,
                                               float valid, const DecodeConsts& kc) {
  using GB = GroupsPerBand<GPT>;
#pragma unroll
  for (int tt = 0; tt < TW; ++tt)
#pragma unroll
    for (int gi = 0; gi < GB::NG; ++gi) {
      const ZeroConst zc = zero_const(zero_nibble(b.zw[tt][gi], col));
      f4 accg[MT];
#pragma unroll
      for (int jj = 0; jj < GB::JPG; ++jj) {
        const int j = gi * GB::JPG + jj;
        const h8 bw = decode_diff_vk(b.wq[tt][j], zc, kc);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          accg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, b.xa[mt][j]), bw,
                                                            jj == 0 ? f4{0.f, 0.f, 0.f, 0.f} : accg[mt], 0, 0, 0);
      }
      const float sf = valid * scale_of(b.s[tt][gi]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[tt][mt] += sf * accg[mt];
    }
}

// TW: 16-column tiles per workgroup (adjacent), each wave covering all of
// them for its bands, so the activations it loads serve TW tiles. GATED (TW =
// 2 or 4): TW/2 adjacent tiles of the gate half and the same tiles of the up
// half, stored as y[m, n] = silu(gate) * up ([M, N/2]).
// K split (part != nullptr): work id u = split * n_groups + group covers the
// bands [split * kps, (split + 1) * kps) of its column group and stores its
// fp32 sums at part[split][row][column] (gated: the gate sums at the output's
// column, the up sums N/2 further); a second kernel adds the splits in order.
// Work ids of one split are adjacent, so the workgroups that run together on
// one XCD share that split's activation slice in L2.
template <int MT, int GPT, int WAVES, int DEPTH, int TW, bool GATED = false>
__global__ __launch_bounds__(64 * WAVES) void decode_stream_kernel(const uint16_t* __restrict__ x,
                                                                   const u4* __restrict__ qw,
                                                                   const uint16_t* __restrict__ scales,
                                                                   const uint32_t* __restrict__ zeros,
                                                                   uint16_t* __restrict__ y, int M, int K, int N,
                                                                   int G, int NT, float* __restrict__ part,
                                                                   int n_groups, int kps) {
  static_assert(!GATED || TW == 2 || TW == 4, "gated: gate tiles and as many up tiles");
  constexpr int TH = GATED ? TW / 2 : TW;  // gate tiles (gated) or tiles per workgroup
  const int u = xcd_remap(blockIdx.x, gridDim.x);
  const int split = u / n_groups;
  const int t0 = (u - split * n_groups) * TH;
  // column tile of the workgroup's tile tt: the up tiles lie NT/2 after the gate tiles
  auto tile_of = [&](int tt) { return GATED && tt >= TH ? NT / 2 + t0 + (tt - TH) : t0 + tt; };
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 4;
  const int groups = K / G;
  const int KT = (K + 127) / 128;

  StreamCtx<TW> c;
  c.rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  c.rs = make_rsrc(scales, (uint32_t)groups * (uint32_t)N * 2u);
  c.rz = make_rsrc(zeros, (uint32_t)groups * (uint32_t)(N / 8) * 4u);
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) {
    // tiles past the last one read the last tile's weights (never stored)
    c.qcol[tt] = qw + (int64_t)min(tile_of(tt), NT - 1) * 64 + lane;
    const int col = 16 * tile_of(tt) + (lane & 15);
    c.soff[tt] = col < N ? (uint32_t)col * 2u : kOOB;
    c.zoff[tt] = col < N ? (uint32_t)(col >> 3) * 4u : kOOB;
  }
  c.band = (int64_t)NT * 64;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int row = 16 * mt + (lane & 15);
    c.xoff[mt] = row < M ? (uint32_t)(row * K + 8 * h) * 2u : kOOB;
  }
  c.srow = (uint32_t)N * 2u;
  c.zrow = (uint32_t)(N / 8) * 4u;
  c.tpg = G / 128;
  c.K = K;
  const DecodeConsts kc = decode_consts();
  const int lcol = lane & 15;

  // this workgroup's bands [kt0, kt1), never empty; wave w takes kt0 + w,
  // kt0 + w + WAVES, ...
  const int kt0 = split * kps, kt1 = min(KT, kt0 + kps);
  const int n_my = kt1 - kt0 > w ? (kt1 - kt0 - w + WAVES - 1) / WAVES : 0;
  const int last = kt0 + max(w + WAVES * (n_my - 1), 0);

  f4 acc[TW][MT];
#pragma unroll
  for (int tt = 0; tt < TW; ++tt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[tt][mt] = f4{0.f, 0.f, 0.f, 0.f};

  Bundle<MT, GPT, TW> buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) load_bundle<MT, GPT, TW>(buf[d], c, min(kt0 + w + WAVES * d, last));
  const int rounds = max((n_my + DEPTH - 1) / DEPTH, 1);
  for (int r = 0; r < rounds - 1; ++r) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int i = r * DEPTH + d;
      consume_bundle<MT, GPT, TW>(buf[d], acc, lcol, 1.f, kc);
      load_bundle<MT, GPT, TW>(buf[d], c, min(kt0 + w + WAVES * (i + DEPTH), last));
    }
  }
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    const int i = (rounds - 1) * DEPTH + d;
    consume_bundle<MT, GPT, TW>(buf[d], acc, lcol, i < n_my ? 1.f : 0.f, kc);
  }

  // Sum the waves' partial tiles, one column tile at a time. Lane l,
  // register r of 16-row tile mt holds output row 16mt + 4(l/16) + r,
  // column 16(t0 + tt) + l%16.
  if constexpr (GATED) {
    // per gate tile: its sums and the up tile's, then silu(gate) * up
    constexpr int OUTS = MT * 4 * 64;
    constexpr int PER = (OUTS + 64 * WAVES - 1) / (64 * WAVES);  // outputs per thread
    __shared__ float red[WAVES][OUTS];
    const int NO = N / 2;
#pragma unroll
    for (int pt = 0; pt < TH; ++pt) {
      float v[2][PER];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if (pt || hf) __syncthreads();  // the previous sums have been read
        const int tt = pt + hf * TH;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[w][(mt * 4 + r) * 64 + lane] = acc[tt][mt][r];
        __syncthreads();
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int o = threadIdx.x + i * 64 * WAVES;
          float a = 0.f;
          if (o < OUTS) {
#pragma unroll
            for (int ww = 0; ww < WAVES; ++ww) a += red[ww][o];
          }
          v[hf][i] = a;
        }
      }
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int o = threadIdx.x + i * 64 * WAVES;
        const int ol = o & 63, mr = o >> 6;
        const int row = 16 * (mr >> 2) + 4 * (ol >> 4) + (mr & 3);
        const int cc = 16 * (t0 + pt) + (ol & 15);
        const float g = v[0][i], up = v[1][i];
        if (o < OUTS && row < M && cc < NO) {
          if (part) {
            float* pr = part + ((int64_t)split * M + row) * N;
            pr[cc] = g;
            pr[NO + cc] = up;
          } else {
            y[(int64_t)row * NO + cc] = __builtin_bit_cast(uint16_t, (_Float16)(g / (1.f + expf(-g)) * up));
          }
        }
      }
    }
  } else if constexpr (WAVES > 1) {
    constexpr int OUTS = MT * 4 * 64;
    __shared__ float red[WAVES][OUTS];
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      if (tt) __syncthreads();  // the previous tile's sums have been read
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[w][(mt * 4 + r) * 64 + lane] = acc[tt][mt][r];
      __syncthreads();
      for (int o = threadIdx.x; o < OUTS; o += 64 * WAVES) {
        float v = 0.f;
#pragma unroll
        for (int ww = 0; ww < WAVES; ++ww) v += red[ww][o];
        const int ol = o & 63, mr = o >> 6;
        const int row = 16 * (mr >> 2) + 4 * (ol >> 4) + (mr & 3);
        const int cc = 16 * (t0 + tt) + (ol & 15);
        if (row < M && cc < N) {
          if (part)
            part[((int64_t)split * M + row) * N + cc] = v;
          else
            y[(int64_t)row * N + cc] = __builtin_bit_cast(uint16_t, (_Float16)v);
        }
      }
    }
  } else {
#pragma unroll
    for (int tt = 0; tt < TW; ++tt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * h + r;
          const int col = 16 * (t0 + tt) + lcol;
          const float v = acc[tt][mt][r];
          if (row < M && col < N) {
            if (part)
              part[((int64_t)split * M + row) * N + col] = v;
            else
              y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)v);
          }
        }
  }
}


// ---------------------------------------------------------------------------
// Slab variant (batched rows: every wave of the workgroup on the same bands)
// ---------------------------------------------------------------------------

// The streamed variant loads each band's activation rows once per wave, so
// with M rows they cost M/4 times the bytes of a one-tile band. Here the
// workgroup's waves each own TW adjacent column tiles and walk the same
// 128-row bands together; the activation rows of kSlabBands bands (a slab)
// are copied global -> registers -> LDS once per workgroup and every wave
// reads its MFMA A operand from there, so one activation load serves
// kSlabWaves * TW tiles. Two slab buffers alternate, one barrier per slab;
// the next slab's loads are issued before the current slab's products and
// stored to LDS after them. Weights, scales and zero points come per band
// into registers, kSlabBands bands ahead. A K split over workgroups works as
// in the streamed variant (part != nullptr: fp32 sums at
// part[split][row][column], then the fixed-order reduction kernel). Whole
// groups per band only (G a multiple of 128). GATED (TW = 2 or 4): each wave
// holds TW/2 adjacent tiles of the gate half and the same tiles of the up
// half and stores y[m, n] = silu(gate) * up ([M, N/2]); with a K split the
// gate and up sums go to their global columns and the reduction applies the
// epilogue.
constexpr int kSlabWaves = 8;
constexpr int kSlabBands = 2;

// LDS byte offset of 16-byte chunk `c` of staged activation row `r` (rows of
// kSlabBands * 16 chunks; the chunk index is XOR-swizzled by the row so that
// the 16 rows one MFMA operand read touches spread over the banks).
__device__ __forceinline__ uint32_t slab_off(uint32_t r, uint32_t c) {
  return (r * (kSlabBands * 16) + (c ^ (r & 15))) * 16;
}

template <int TW>
struct SlabBand {
  u4 wq[TW];
  uint32_t s[TW];
  uint32_t zw[TW];
};

template <int MT, int GPT, int TW, bool GATED = false>
__global__ __launch_bounds__(64 * kSlabWaves) void decode_slab_kernel(const uint16_t* __restrict__ x,
                                                                      const u4* __restrict__ qw,
                                                                      const uint16_t* __restrict__ scales,
                                                                      const uint32_t* __restrict__ zeros,
                                                                      uint16_t* __restrict__ y, int M, int K, int N,
                                                                      int G, int NT, float* __restrict__ part,
                                                                      int n_groups, int kps) {
  static_assert(GPT == 0 || GPT == 1, "one group entry per band");
  static_assert(!GATED || TW == 2 || TW == 4, "gated: gate tiles and as many up tiles");
  constexpr int TH = GATED ? TW / 2 : TW;  // gate tiles (gated) or tiles per wave
  static_assert(kSlabBands == 2, "the loop consumes a slab as two bands in the two weight buffers");
  constexpr int NTH = 64 * kSlabWaves;
  constexpr int CPR = kSlabBands * 16;  // 16-byte chunks per staged row
  constexpr int PER = 16 * MT * CPR / NTH;  // staging chunks per thread
  static_assert(PER * NTH == 16 * MT * CPR, "whole chunks per thread");
  __shared__ __attribute__((aligned(16))) char slab[2][16 * MT * CPR * 16];

  const int u = xcd_remap(blockIdx.x, gridDim.x);
  const int split = u / n_groups;
  const int grp = u - split * n_groups;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 4;
  const int lcol = lane & 15;
  const int t0 = (grp * kSlabWaves + w) * TH;  // the wave's first (gate) column tile
  const int NO = N / 2;                         // gated: output columns
  // column tile of the wave's tile tt: the up tiles lie NT/2 after the gate tiles
  auto tile_of = [&](int tt) { return GATED && tt >= TH ? NT / 2 + t0 + (tt - TH) : t0 + tt; };
  // the tile's column exists (gated: its output column)
  auto col_ok = [&](int tt) { return GATED ? 16 * (t0 + tt % TH) + lcol < NO : 16 * (t0 + tt) + lcol < N; };
  const int groups = K / G;
  const int tpg = G / 128;
  const int KT = (K + 127) / 128;
  const int kt0 = split * kps;
  const int nb = min(KT, kt0 + kps) - kt0;  // bands of this split, >= 1
  const int last = kt0 + nb - 1;
  const int nslab = (nb + kSlabBands - 1) / kSlabBands;

  const rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const rsrc_t rs = make_rsrc(scales, (uint32_t)groups * (uint32_t)N * 2u);
  const rsrc_t rz = make_rsrc(zeros, (uint32_t)groups * (uint32_t)(N / 8) * 4u);
  const u4* qcol[TW];
  uint32_t soff[TW], zoff[TW];
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) {
    // tiles past the last one read the last tile's weights (never stored)
    qcol[tt] = qw + (int64_t)min(tile_of(tt), NT - 1) * 64 + lane;
    const int col = 16 * tile_of(tt) + lcol;
    soff[tt] = col_ok(tt) ? (uint32_t)col * 2u : kOOB;
    zoff[tt] = col_ok(tt) ? (uint32_t)(col >> 3) * 4u : kOOB;
  }
  const int64_t band = (int64_t)NT * 64;
  const uint32_t srow = (uint32_t)N * 2u, zrow = (uint32_t)(N / 8) * 4u;
  auto load_band = [&](SlabBand<TW>& b, int kt) {
    const uint32_t g = GroupsPerBand<GPT>::group(kt, 0, tpg);
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      b.s[tt] = __builtin_amdgcn_raw_buffer_load_b16(rs, soff[tt] + g * srow, 0, 0);
      b.zw[tt] = __builtin_amdgcn_raw_buffer_load_b32(rz, zoff[tt] + g * zrow, 0, 0);
      b.wq[tt] = load_weights(qcol[tt] + kt * band);
    }
  };
  // Staging chunk p = i * NTH + tid sits at LDS row p / CPR, position p % CPR,
  // and holds global chunk (position ^ (row & 15)) of that row of the slab;
  // rows past M and columns past K read zero.
  auto load_slab = [&](u4 (&v)[PER], int s) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t p = (uint32_t)(i * NTH) + threadIdx.x;
      const uint32_t r = p / CPR, pos = p % CPR;
      const uint32_t kc = 128u * (uint32_t)(kt0 + kSlabBands * s) + 8u * (pos ^ (r & 15u));
      const bool ok = r < (uint32_t)M && kc < (uint32_t)K;
      v[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? (r * (uint32_t)K + kc) * 2u : kOOB,
                                                                            0, 0));
    }
  };
  auto store_slab = [&](const u4 (&v)[PER], int buf) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t p = (uint32_t)(i * NTH) + threadIdx.x;
      *reinterpret_cast<u4*>(slab[buf] + p * 16u) = v[i];
    }
  };

  const DecodeConsts kc = decode_consts();
  f4 acc[TW][MT];
#pragma unroll
  for (int tt = 0; tt < TW; ++tt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[tt][mt] = f4{0.f, 0.f, 0.f, 0.f};

  // Band bi of the slab in buffer `buf`: A operand from LDS (lane l: row
  // 16 mt + l % 16, rows 32 j + 8 (l / 16) .. +7 of the band), shared by the
  // wave's TW tiles.
  auto consume = [&](const SlabBand<TW>& b, int buf, int bi, float valid) {
    h8 a[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a[mt][j] = *reinterpret_cast<const h8*>(slab[buf] +
                                                slab_off((uint32_t)(16 * mt + lcol), (uint32_t)(16 * bi + 4 * j + h)));
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      const ZeroConst zc = zero_const(zero_nibble(b.zw[tt], lcol));
      f4 accg[MT];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const h8 bw = decode_diff_vk(b.wq[tt][j], zc, kc);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          accg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][j], bw, j == 0 ? f4{0.f, 0.f, 0.f, 0.f} : accg[mt],
                                                            0, 0, 0);
      }
      const float sf = valid * scale_of(b.s[tt]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[tt][mt] += sf * accg[mt];
    }
  };

  // Prologue: slab 0's loads, the first two bands' weights, slab 0 to LDS.
  SlabBand<TW> b0, b1;
  {
    u4 v[PER];
    load_slab(v, 0);
    load_band(b0, kt0);
    load_band(b1, min(kt0 + 1, last));
    store_slab(v, 0);
  }
  __syncthreads();
  // Every wave runs the same slabs, so the barriers match; bands past the
  // split's last one are multiplied by zero (their weights are the last
  // band's, their activations finite or zero).
  for (int s = 0; s < nslab; ++s) {
    const int buf = s & 1;
    const bool more = s + 1 < nslab;
    u4 v[PER];
    if (more) load_slab(v, s + 1);
    consume(b0, buf, 0, 1.f);
    load_band(b0, min(kt0 + kSlabBands * s + 2, last));
    consume(b1, buf, 1, kSlabBands * s + 1 < nb ? 1.f : 0.f);
    load_band(b1, min(kt0 + kSlabBands * s + 3, last));
    if (more) store_slab(v, buf ^ 1);
    __syncthreads();
  }

  // Each wave holds whole sums (over the split's bands) of its own tiles.
  // Lane l, register r of row tile mt: row 16 mt + 4 (l / 16) + r, column
  // 16 (t0 + tt) + l % 16 (gated: output column; the up sums in tile tt + TH).
  if constexpr (GATED) {
#pragma unroll
    for (int pt = 0; pt < TH; ++pt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * h + r;
          const int oc = 16 * (t0 + pt) + lcol;
          const float g = acc[pt][mt][r], up = acc[TH + pt][mt][r];
          if (row < M && oc < NO) {
            if (part) {
              float* pr = part + ((int64_t)split * M + row) * N;
              pr[oc] = g;
              pr[NO + oc] = up;
            } else {
              y[(int64_t)row * NO + oc] = __builtin_bit_cast(uint16_t, (_Float16)(g / (1.f + expf(-g)) * up));
            }
          }
        }
    return;
  }
#pragma unroll
  for (int tt = 0; tt < TW; ++tt)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mt + 4 * h + r;
        const int col = 16 * (t0 + tt) + lcol;
        if (row < M && col < N) {
          if (part)
            part[((int64_t)split * M + row) * N + col] = acc[tt][mt][r];
          else
            y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)acc[tt][mt][r]);
        }
      }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

namespace {

constexpr int kStagedDepth = 4;

struct StagedSizes {
  StagedLayout lay;
  size_t lds;
  int S;  // staging iterations per thread (power of two, <= 8; 0 = too many)
};

StagedSizes staged_sizes(int M, int K, int G, int waves, int tpw) {
  StagedSizes z;
  const int nth = 64 * waves;
  // rows padded with zeros to whole 128-row bands, plus one 16-byte chunk
  const uint32_t kp = (uint32_t)((K + 127) / 128 * 128);
  z.lay.x_chunks = kp / 8 + 1;
  z.lay.x_row = z.lay.x_chunks * 16;
  z.lay.scratch_off = (uint32_t)M * z.lay.x_row;
  const size_t lds = z.lay.scratch_off + (size_t)nth * 16;
  const size_t red = (size_t)waves * tpw * 256 * 4;
  z.lds = lds > red ? lds : red;
  const int64_t items = (int64_t)M * z.lay.x_chunks;
  const int64_t per = (items + nth - 1) / nth;
  z.S = per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= 8 ? 8 : 0;
  return z;
}

template <typename F>
hipError_t allow_lds(F kernel, size_t lds) {
  if (lds <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds);
}

template <int TM, int WAVES, typename F>
hipError_t launch_staged_k(F k, const LinearArgs& a, const StagedSizes& z, const Launch& L) {
  const int NT = (a.N + 15) / 16;
  hipError_t e = allow_lds(k, z.lds);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(TM == 1 ? NT : TM == 2 ? (NT + 1) / 2 : NT / 2);
  return launch_kernel(k, dim3(grid), dim3(64 * WAVES), z.lds, L, a.x, reinterpret_cast<const u4*>(a.qw), a.scales,
                       a.zeros, a.y, a.M, a.K, a.N, a.G, NT, z.lay);
}

template <int TM, int GPT, int WAVES, int S>
hipError_t launch_staged_s(const LinearArgs& a, const StagedSizes& z, const Launch& L) {
  // Five bands per wave (e.g. K = 4544, 36 bands over 8 waves): all five in
  // flight at once (measured on the Falcon-7B layers at group 64: QKV 6.9 ->
  // 6.0 us), with the 64-VGPR build set aside (it would spill).
  const int per_wave = ((a.K + 127) / 128 + WAVES - 1) / WAVES;
  if constexpr (TM == 1) {
    if (per_wave == 5)
      return launch_staged_k<TM, WAVES>(decode_staged_kernel<TM, GPT, WAVES, 5, S>, a, z, L);
  }
  // Twelve or more bands per wave at two groups per band (G = 64): six in
  // flight (the Falcon-7B down projection, 18176 x 4544, 18 bands per wave:
  // 16.0-16.4 against 16.5-17.0 us with four; nine gain nothing).
  if constexpr (TM == 1 && GPT == 2) {
    if (per_wave >= 12)
      return launch_staged_k<TM, WAVES>(decode_staged_kernel<TM, GPT, WAVES, 6, S>, a, z, L);
  }
  // the 64-VGPR build only where it compiles without spills: one group per
  // band, at most two 16-byte staging loads per thread, four or more waves
  if constexpr (TM != 2 && GPT == 1 && S <= 2 && WAVES >= 4)
    return launch_staged_k<TM, WAVES>(decode_staged_kernel_o8<TM, GPT, WAVES, kStagedDepth, S>, a, z, L);
  else
    return launch_staged_k<TM, WAVES>(decode_staged_kernel<TM, GPT, WAVES, kStagedDepth, S>, a, z, L);
}

template <int TM, int GPT, int WAVES>
hipError_t launch_staged_w(const LinearArgs& a, const StagedSizes& z, const Launch& L) {
  switch (z.S) {
    case 1: return launch_staged_s<TM, GPT, WAVES, 1>(a, z, L);
    case 2: return launch_staged_s<TM, GPT, WAVES, 2>(a, z, L);
    case 4: return launch_staged_s<TM, GPT, WAVES, 4>(a, z, L);
    case 8: return launch_staged_s<TM, GPT, WAVES, 8>(a, z, L);
  }
  return hipErrorInvalidValue;
}

template <int TM, int GPT>
hipError_t launch_staged_g(const LinearArgs& a, int waves, const StagedSizes& z, const Launch& L) {
  switch (waves) {
    case 2: return launch_staged_w<TM, GPT, 2>(a, z, L);
    case 4: return launch_staged_w<TM, GPT, 4>(a, z, L);
    case 8: return launch_staged_w<TM, GPT, 8>(a, z, L);
    case 16: return launch_staged_w<TM, GPT, 16>(a, z, L);
  }
  return hipErrorInvalidValue;
}

template <int TM>
hipError_t launch_staged_t(const LinearArgs& a, int waves, const StagedSizes& z, const Launch& L) {
  if (a.G == 32) return launch_staged_g<TM, 4>(a, waves, z, L);
  if (a.G == 64) return launch_staged_g<TM, 2>(a, waves, z, L);
  if (a.G == 128) return launch_staged_g<TM, 1>(a, waves, z, L);
  return launch_staged_g<TM, 0>(a, waves, z, L);
}

// A split of the K range into `splits` ranges of whole bands (every range
// non-empty): bands per range, and the number of ranges that gives.
struct KSplit {
  int kps, splits;
};
KSplit k_split(int K, int splits) {
  const int KT = (K + 127) / 128;
  const int s = splits < 1 ? 1 : (splits > KT ? KT : splits);
  const int kps = (KT + s - 1) / s;
  return KSplit{kps, (KT + kps - 1) / kps};
}

// With splits > 1 the kernel writes fp32 partials to ws[split][M][N] and the
// prefill path's fixed-order reduction adds them (and applies the gated
// epilogue); `L.start` is recorded at the first kernel, `L.stop` at the last.
template <typename F>
hipError_t launch_stream_split(F k, int groups, int waves, const LinearArgs& a, int splits, float* ws, bool gated,
                               const Launch& L) {
  const int NT = (a.N + 15) / 16;
  const KSplit ks = k_split(a.K, splits);
  float* part = ks.splits > 1 ? ws : nullptr;
  if (ks.splits > 1 && !ws) return hipErrorInvalidValue;
  const Launch first{L.stream, L.start, part ? nullptr : L.stop};
  hipError_t e = launch_kernel(k, dim3((unsigned)(groups * ks.splits)), dim3(64 * waves), 0, first, a.x,
                               reinterpret_cast<const u4*>(a.qw), a.scales, a.zeros, a.y, a.M, a.K, a.N, a.G, NT,
                               part, groups, ks.kps);
  if (e != hipSuccess || !part) return e;
  return launch_prefill_reduce(part, a.y, a.M, a.N, ks.splits, gated, Launch{L.stream, nullptr, L.stop});
}

template <int MT, int GPT, int WAVES, int TW>
hipError_t launch_stream_k(const LinearArgs& a, int splits, float* ws, const Launch& L) {
  // bands in flight per wave: fewer when a band carries more registers
  constexpr int DEPTH = TW == 1 ? (MT == 1 ? 4 : (MT == 2 ? 3 : 2)) : 2;
  const int NT = (a.N + 15) / 16;
  return launch_stream_split(decode_stream_kernel<MT, GPT, WAVES, DEPTH, TW>, (NT + TW - 1) / TW, WAVES, a, splits,
                             ws, false, L);
}

template <int MT, int GPT, int WAVES, int TW>
hipError_t launch_stream_gated_k(const LinearArgs& a, int splits, float* ws, const Launch& L) {
  const int NT = (a.N + 15) / 16;
  if ((NT / 2) % (TW / 2)) return hipErrorInvalidValue;  // whole groups of gate tiles
  return launch_stream_split(decode_stream_kernel<MT, GPT, WAVES, 2, TW, true>, NT / TW, WAVES, a, splits, ws, true,
                             L);
}

template <int MT, int GPT>
hipError_t launch_stream_gated(const LinearArgs& a, int waves, int tw, int splits, float* ws, const Launch& L) {
  if (waves == 4 && tw == 2) return launch_stream_gated_k<MT, GPT, 4, 2>(a, splits, ws, L);
  if (waves == 4 && tw == 4) return launch_stream_gated_k<MT, GPT, 4, 4>(a, splits, ws, L);
  if (waves == 8 && tw == 2) return launch_stream_gated_k<MT, GPT, 8, 2>(a, splits, ws, L);
  if (waves == 8 && tw == 4) return launch_stream_gated_k<MT, GPT, 8, 4>(a, splits, ws, L);
  return hipErrorInvalidValue;
}

template <int MT>
hipError_t launch_stream_gated_g(const LinearArgs& a, int waves, int tw, int splits, float* ws, const Launch& L) {
  if (a.G == 32) return launch_stream_gated<MT, 4>(a, waves, tw, splits, ws, L);
  if (a.G == 64) return launch_stream_gated<MT, 2>(a, waves, tw, splits, ws, L);
  if (a.G == 128) return launch_stream_gated<MT, 1>(a, waves, tw, splits, ws, L);
  return launch_stream_gated<MT, 0>(a, waves, tw, splits, ws, L);
}

template <int MT, int GPT, int WAVES>
hipError_t launch_stream_t(const LinearArgs& a, int tw, int splits, float* ws, const Launch& L) {
  if constexpr (MT <= 2 && (WAVES == 4 || WAVES == 8)) {
    if (tw == 2) return launch_stream_k<MT, GPT, WAVES, 2>(a, splits, ws, L);
    if (tw == 4) return launch_stream_k<MT, GPT, WAVES, 4>(a, splits, ws, L);
  }
  if (tw != 1) return hipErrorInvalidValue;
  return launch_stream_k<MT, GPT, WAVES, 1>(a, splits, ws, L);
}

template <int MT, int GPT>
hipError_t launch_stream_w(const LinearArgs& a, int waves, int tw, int splits, float* ws, const Launch& L) {
  switch (waves) {
    case 1: return launch_stream_t<MT, GPT, 1>(a, tw, splits, ws, L);
    case 2: return launch_stream_t<MT, GPT, 2>(a, tw, splits, ws, L);
    case 4: return launch_stream_t<MT, GPT, 4>(a, tw, splits, ws, L);
    case 8: return launch_stream_t<MT, GPT, 8>(a, tw, splits, ws, L);
    case 16: return launch_stream_t<MT, GPT, 16>(a, tw, splits, ws, L);
  }
  return hipErrorInvalidValue;
}

template <int MT>
hipError_t launch_stream_g(const LinearArgs& a, int waves, int tw, int splits, float* ws, const Launch& L) {
  if (a.G == 32) return launch_stream_w<MT, 4>(a, waves, tw, splits, ws, L);
  if (a.G == 64) return launch_stream_w<MT, 2>(a, waves, tw, splits, ws, L);
  if (a.G == 128) return launch_stream_w<MT, 1>(a, waves, tw, splits, ws, L);
  return launch_stream_w<MT, 0>(a, waves, tw, splits, ws, L);
}

template <int MT, int GPT>
hipError_t launch_slab_t(const LinearArgs& a, int tw, int splits, float* ws, bool gated, const Launch& L) {
  const int NT = (a.N + 15) / 16;
  if (gated) {
    // N % 32 == 0: each half is whole tiles
    if (a.N % 32) return hipErrorInvalidValue;
    const int per_group = kSlabWaves * (tw / 2);
    const int groups = (NT / 2 + per_group - 1) / per_group;
    if (tw == 2)
      return launch_stream_split(decode_slab_kernel<MT, GPT, 2, true>, groups, kSlabWaves, a, splits, ws, true, L);
    if (tw == 4)
      return launch_stream_split(decode_slab_kernel<MT, GPT, 4, true>, groups, kSlabWaves, a, splits, ws, true, L);
    return hipErrorInvalidValue;
  }
  const int per_group = kSlabWaves * tw;
  const int groups = (NT + per_group - 1) / per_group;
  if (tw == 1) return launch_stream_split(decode_slab_kernel<MT, GPT, 1>, groups, kSlabWaves, a, splits, ws, false, L);
  if (tw == 2) return launch_stream_split(decode_slab_kernel<MT, GPT, 2>, groups, kSlabWaves, a, splits, ws, false, L);
  if (tw == 4) return launch_stream_split(decode_slab_kernel<MT, GPT, 4>, groups, kSlabWaves, a, splits, ws, false, L);
  return hipErrorInvalidValue;
}

template <int MT>
hipError_t launch_slab_g(const LinearArgs& a, int tw, int splits, float* ws, bool gated, const Launch& L) {
  if (a.G == 128) return launch_slab_t<MT, 1>(a, tw, splits, ws, gated, L);
  if (a.G % 128 == 0) return launch_slab_t<MT, 0>(a, tw, splits, ws, gated, L);
  return hipErrorInvalidValue;
}

}  // namespace

int decode_splits(int K, int splits) { return k_split(K, splits).splits; }

bool decode_staged_fits(int M, int K, int G, int waves, int tpw) {
  if (M > 16 || waves < 2 || (tpw != 1 && tpw != 2)) return false;
  const StagedSizes z = staged_sizes(M, K, G, waves, tpw);
  return z.S > 0 && z.lds <= (size_t)kDecodeLdsBytes;
}

hipError_t launch_decode(const LinearArgs& a, const DecodeConfig& cfg, const Launch& L) {
  if (cfg.gated) {
    // gate and up tiles paired in one workgroup
    if (a.N % 32) return hipErrorInvalidValue;
    if (cfg.slab) {
      if (cfg.waves != kSlabWaves) return hipErrorInvalidValue;
      if (a.M <= 16) return launch_slab_g<1>(a, cfg.tpw, cfg.splits, cfg.ws, true, L);
      if (a.M <= 32) return launch_slab_g<2>(a, cfg.tpw, cfg.splits, cfg.ws, true, L);
      return hipErrorInvalidValue;
    }
    if (!cfg.staged) {
      if (a.M <= 16) return launch_stream_gated_g<1>(a, cfg.waves, cfg.tpw, cfg.splits, cfg.ws, L);
      if (a.M <= 32) return launch_stream_gated_g<2>(a, cfg.waves, cfg.tpw, cfg.splits, cfg.ws, L);
      return hipErrorInvalidValue;
    }
    if (cfg.waves < 2 || !decode_staged_fits(a.M, a.K, a.G, cfg.waves, 1)) return hipErrorInvalidValue;
    return launch_staged_t<3>(a, cfg.waves, staged_sizes(a.M, a.K, a.G, cfg.waves, 1), L);
  }
  if (cfg.staged) {
    if (!decode_staged_fits(a.M, a.K, a.G, cfg.waves, cfg.tpw)) return hipErrorInvalidValue;
    const StagedSizes z = staged_sizes(a.M, a.K, a.G, cfg.waves, cfg.tpw);
    if (cfg.tpw == 2) return launch_staged_t<2>(a, cfg.waves, z, L);
    return launch_staged_t<1>(a, cfg.waves, z, L);
  }
  if (cfg.slab) {
    if (cfg.waves != kSlabWaves) return hipErrorInvalidValue;
    if (a.M <= 16) return launch_slab_g<1>(a, cfg.tpw, cfg.splits, cfg.ws, false, L);
    if (a.M <= 32) return launch_slab_g<2>(a, cfg.tpw, cfg.splits, cfg.ws, false, L);
    return hipErrorInvalidValue;
  }
  if (a.M <= 16) return launch_stream_g<1>(a, cfg.waves, cfg.tpw, cfg.splits, cfg.ws, L);
  if (a.M <= 32) return launch_stream_g<2>(a, cfg.waves, cfg.tpw, cfg.splits, cfg.ws, L);
  if (a.M <= 64) return launch_stream_g<4>(a, cfg.waves, cfg.tpw, cfg.splits, cfg.ws, L);
  return hipErrorInvalidValue;
}

}  // namespace awq
