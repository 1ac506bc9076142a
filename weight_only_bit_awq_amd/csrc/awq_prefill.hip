// Prefill path of the W4A16 linear layer (large M): a dequantise-then-MFMA
// fp16 GEMM with fp32 accumulation.
//
// At prefill sizes (hundreds to thousands of activation rows, as in the
// context stage of "TinyChat: Efficient and Lightweight Chatbot with AWQ",
// section "New Optimization of Context Stage") every weight is reused by many
// rows, so the layer is a dense contraction bound by the matrix cores. Each
// packed weight is decoded to its exact fp16 value (q - z) * s once per wave
// that uses it and fed to v_mfma_f32_16x16x32_f16. In the 256 x 256 tile
// every wave owns two column tiles for all 256 rows, so each weight is
// decoded once per workgroup (the vector-ALU work per MFMA is what limits
// this kernel; the price is twice the activation reads from LDS).
//
// Structure (per workgroup: WM x WN waves, each wave MTW x NTW tiles of 16x16
// outputs; K advances KS rows per step):
//   * Activations: the BM x KS fp16 slab of a step is copied from global
//     memory straight into LDS by buffer loads with the LDS bit (no register
//     round trip), one step ahead, into two alternating buffers. The 16-byte
//     chunks of a slab row are XOR-swizzled by the row index, so the 16-byte
//     fragment reads of 16 consecutive rows hit distinct banks; the swizzle is
//     applied on the global side because such a load always writes lane l's
//     16 bytes at LDS offset 16*l.
//   * Scales and packed zero words of the workgroup's columns for the step's
//     groups ride along the same way (one dword per thread each).
//   * Weights: each wave reads the packed words of its own columns straight
//     from global memory into registers (KS/128 of the lane's 16-byte slice
//     of a 128-row tile per column tile); tiles of one 128-row band are
//     adjacent in the device layout, so these reads are contiguous.
//   * Software pipeline inside a step: iteration (substep, column tile)
//     issues that tile's MFMAs for all of the wave's row tiles, decodes the
//     next tile's words in between (about two VALU instructions per MFMA,
//     which the matrix core's issue gaps absorb), and carries an even share
//     of the next stage's loads (the next step's weight words first, into a
//     second register set, then activations, scales and zero points). A row
//     tile's A fragment for the next substep is read from LDS right after its
//     last MFMA in this one.
//   * One barrier per step; rows past M and K past the end read zero
//     through the buffers' range checks; columns past N get zero scales, so
//     their outputs are zero, and are never stored.
//   * Split-K (for layers with fewer output tiles than the chip has
//     workgroup slots): workgroup (split, tile) covers a contiguous range of
//     K steps and writes fp32 partial sums to ws[split][M][N]; a second
//     kernel adds the splits in a fixed order and rounds once to fp16, so the
//     result does not depend on scheduling.
#include <atomic>
#include <cmath>

#include "awq_device.h"
#include "awq_launch.h"

// Device memory for callers that cannot allocate (awq_linear_noalloc): the
// fp32 split-K partial sums live in this array, one copy per GPU the library
// is loaded on, held until the process ends. Host code never passes its name
// to a kernel (on the host it is only a stand-in for the device symbol); it
// uses the device address from hipGetSymbolAddress, taken once per device.
static __device__ __align__(256) float scratch[awq::kNoAllocScratchBytes / sizeof(float)];

namespace awq {

typedef uint32_t u2 __attribute__((ext_vector_type(2)));

template <int WM, int WN, int MTW, int NTW, int KS, int GS>
struct PrefillCfg {
  static constexpr int NW = WM * WN;
  static constexpr int NTH = 64 * NW;
  static constexpr int BM = 16 * MTW * WM;
  static constexpr int BN = 16 * NTW * WN;
  static constexpr int KB = KS / 32;            // MFMA k-blocks per step
  static constexpr int CPR = KS / 8;            // 16-byte chunks per slab row
  static constexpr int A_BYTES = BM * KS * 2;   // one activation slab
  static constexpr int A_DMA = BM * CPR / NTH;  // 16-byte loads per thread per step
  static constexpr int SC_OFF = A_BYTES;        // NTH dwords of scales (GS rows x BN)
  static constexpr int ZW_OFF = A_BYTES + NTH * 4;  // NTH dwords of zero words (GS rows x BN/8)
  static constexpr int STAGE = A_BYTES + 2 * NTH * 4;
  static constexpr int LDS_BYTES = 2 * STAGE;
  static_assert(KS == 64 || KS == 128, "step of 64 or 128 rows");
  static_assert((BM * CPR) % NTH == 0, "activation slab must split evenly over the threads");
  static_assert(GS * BN / 2 <= NTH && GS * BN / 8 <= NTH, "scale and zero rows exceed one dword per thread");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Weight words of one lane and column tile for one step: KS/32 words.
template <int KB>
struct WeightWords;
template <>
struct WeightWords<2> {
  typedef u2 T;
  static __device__ __forceinline__ T load(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  }
};
template <>
struct WeightWords<4> {
  typedef u4 T;
  static __device__ __forceinline__ T load(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  }
};

// Byte offset of 16-byte chunk `chunk` of slab row `row` (rows of CPR chunks).
template <int CPR>
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) {
  return row * (16u * CPR) + ((chunk ^ (row % CPR)) << 4);
}

// EPI = true: gated epilogue. The workgroup's BN logical columns are BN/2
// gate columns g0 .. g0+BN/2-1 followed by the matching up columns N/2 + g0 ..;
// each wave holds NTW/2 gate tiles and the NTW/2 up tiles of the same
// columns, so silu(gate) * up is formed in registers and y is [M, N/2]
// (with split-K the fp32 partials go to the workspace at their global
// columns and the reduction applies the epilogue).
template <int WM, int WN, int MTW, int NTW, int KS, int GS, bool EPI>
__global__ __launch_bounds__(64 * WM * WN) void prefill_kernel(const uint16_t* __restrict__ x,
                                                               const uint32_t* __restrict__ qw,
                                                               const uint16_t* __restrict__ scales,
                                                               const uint32_t* __restrict__ zeros,
                                                               uint16_t* __restrict__ y, float* __restrict__ ws, int M,
                                                               int K, int N, int G, int NT, int n_mtiles, int n_tiles,
                                                               int split_steps, uint32_t qw_bytes) {
  using C = PrefillCfg<WM, WN, MTW, NTW, KS, GS>;
  using WW = WeightWords<C::KB>;
  typedef typename WW::T wvec;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int u = xcd_remap(blockIdx.x, gridDim.x);
  const int split = u / n_tiles;
  const int tile = u - split * n_tiles;
  // column tiles fastest: the workgroups that run together on one XCD share
  // one activation slab (measured 1-1.5% faster than rows fastest)
  const int n_ntiles = n_tiles / n_mtiles;
  const int mtile = tile / n_ntiles;
  const int ntile = tile % n_ntiles;
  const int m0 = mtile * C::BM;
  const int n0 = ntile * C::BN;  // plain: first global column of the workgroup
  const int NO = N / 2;           // gated: columns per half
  const int g0 = ntile * (C::BN / 2);  // gated: first gate column of the workgroup
  // logical column c of the workgroup tile -> global column, and whether it exists
  auto gcol = [&](int c) { return EPI ? (c < C::BN / 2 ? g0 + c : NO + g0 + (c - C::BN / 2)) : n0 + c; };
  auto gvalid = [&](int c) { return EPI ? g0 + (c % (C::BN / 2)) < NO : n0 + c < N; };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / WN, wn = wv % WN;
  const int h = lane >> 4;
  const int groups = K / G;
  const int nsteps = (K + KS - 1) / KS;
  const int step0 = split * split_steps;                   // this workgroup's K steps:
  const int step1 = min(nsteps, step0 + split_steps);      // [step0, step1), never empty

  const rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const rsrc_t rq = make_rsrc(qw, qw_bytes);
  const rsrc_t rs = make_rsrc(scales, (uint32_t)groups * (uint32_t)N * 2u);
  const rsrc_t rz = make_rsrc(zeros, (uint32_t)groups * (uint32_t)(N / 8) * 4u);

  // Activation load j of this thread fills slab chunk p = (j*NW + wave)*64 + lane:
  // row p / CPR, stored column p % CPR, i.e. global chunk (p % CPR) ^ (row % CPR).
  // Consecutive loads are NW*64/CPR rows apart, a multiple of CPR, so the
  // chunk (and the column a_k it starts at) is the same for every j.
  static_assert((C::NW * 64 / C::CPR) % C::CPR == 0, "one swizzled chunk per thread");
  // Rows past M lie past the end of x (M*K*2 < 2^31 bytes, so no offset
  // wraps) and read zeros through the buffer's range check.
  constexpr int A_ROWS = C::NW * 64 / C::CPR;  // rows between consecutive loads
  uint32_t a_base, a_k;
  {
    const uint32_t p0 = (uint32_t)wv * 64u + (uint32_t)lane;
    a_k = 8u * ((p0 % C::CPR) ^ ((p0 / C::CPR) % C::CPR));
    a_base = ((uint32_t)(m0 + (int)(p0 / C::CPR)) * (uint32_t)K + a_k) * 2u;
  }
  const uint32_t a_step = (uint32_t)A_ROWS * (uint32_t)K * 2u;
  // Dword tid of the scale region: columns 2c, 2c+1 of group row gi; of the
  // zero region: packed word c of group row gi.
  const int sc_gi = tid / (C::BN / 2), sc_col = gcol(2 * (tid % (C::BN / 2)));
  const bool sc_ok = sc_gi < GS && gvalid(2 * (tid % (C::BN / 2)));
  const int zw_gi = tid / (C::BN / 8), zw_w = gcol(8 * (tid % (C::BN / 8))) / 8;
  const bool zw_ok = zw_gi < GS && gvalid(8 * (tid % (C::BN / 8)));
  // Logical column (within the workgroup tile) of the wave's column tile nt;
  // gated: tiles 0 .. NTW/2-1 are gate columns, the rest the up columns of
  // the same outputs.
  auto lcol = [&](int nt) {
    return EPI ? (nt < NTW / 2 ? 0 : C::BN / 2) + 16 * (NTW / 2) * wn + 16 * (nt % (NTW / 2)) : 16 * (NTW * wn + nt);
  };
  // This lane's slice of the wave's column tiles in band 0: the tiles of one
  // half (all NTW plain, NTW/2 gate or up) are consecutive, 1 KiB apart.
  // Tiles past the last column read whatever the buffer holds there (zero
  // past its end); their outputs are never stored.
  uint32_t b_off[EPI ? 2 : 1];
#pragma unroll
  for (int hh = 0; hh < (EPI ? 2 : 1); ++hh)
    b_off[hh] = (uint32_t)(gcol(lcol(hh * (NTW / 2))) / 16) * 1024u + (uint32_t)lane * 16u;
  f4 acc[MTW][NTW];
#pragma unroll
  for (int a = 0; a < MTW; ++a)
#pragma unroll
    for (int b = 0; b < NTW; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};

  constexpr int KB = C::KB;
  constexpr int NIT = KB * NTW;            // (substep, column tile) iterations per step
  constexpr int NLD = NTW + C::A_DMA + 2;  // next-stage loads, spread evenly over the iterations

  DecodeConsts kc;
  kc.m1 = 0x000F000Fu;
  kc.m2 = 0x00F000F0u;
  kc.o1 = 0x64006400u;
  kc.o2 = 0x54005400u;
  // masks in VGPRs, OR patterns in SGPRs: one v_and_or_b32 each
  asm volatile("" : "+v"(kc.m1), "+v"(kc.m2), "+s"(kc.o1), "+s"(kc.o2));

  const int arow0 = 16 * MTW * wm + (lane & 15);
  wvec cb[NTW], rb[NTW];
  h8 af[MTW];
  ZeroConst zc[NTW];
  h2 s2[NTW];
  // zero point and scale of column tile nt for group gi of a stage
  auto zs_of = [&](const char* st, int gi, int nt) {
    const uint16_t* sc_l = reinterpret_cast<const uint16_t*>(st + C::SC_OFF);
    const uint32_t* zw_l = reinterpret_cast<const uint32_t*>(st + C::ZW_OFF);
    const int c = lcol(nt) + (lane & 15);
    const uint32_t zw = zw_l[gi * (C::BN / 8) + c / 8];
    zc[nt] = zero_const((zw >> (4 * (c % 8))) & 0xFu);
    s2[nt] = splat_h2(sc_l[gi * C::BN + c]);
  };
  auto grp = [](int s) { return GS == 1 ? 0 : s / (KB / GS); };
  auto wband = [&](int step) {
    return KS == 128 ? (uint32_t)step * (uint32_t)NT * 1024u
                     : (uint32_t)(step >> 1) * (uint32_t)NT * 1024u + (uint32_t)(step & 1) * 8u;
  };
  auto woff = [&](int nt) {
    return EPI ? b_off[nt / (NTW / 2)] + (uint32_t)(nt % (NTW / 2)) * 1024u : b_off[0] + (uint32_t)nt * 1024u;
  };
  // Load item i of the next stage: weight tile i (into the copy), then
  // activation chunk j, then the scale and the zero-point dword. inv (bit
  // 31) puts a load out of range: it reads zeros (past the last step).
  auto issue_item = [&](int i, int step, int buf, uint32_t inv) {
    if (i < NTW) {
      rb[i] = WW::load(rq, (woff(i) + wband(step)) | inv);
      return;
    }
    char* stn = smem + buf * C::STAGE;
    const uint32_t k0 = (uint32_t)step * KS;
    if (i < NTW + C::A_DMA) {
      const int j = i - NTW;
      const uint32_t bad = ((uint32_t)!(k0 + a_k < (uint32_t)K) << 31) | inv;
      uint32_t a0 = a_base + k0 * 2u;
      asm volatile("" : "+v"(a0));  // keeps the per-load offsets out of the loop's invariants
      load_to_lds16(rx, stn + (j * C::NW + wv) * 1024, (a0 + (uint32_t)j * a_step) | bad);
      return;
    }
    const int g0 = GS > 1 ? step * GS : (step * KS) / G;  // first group of the step
    if (i == NTW + C::A_DMA) {
      const int sg = g0 + sc_gi;
      const uint32_t sbad = ((uint32_t)!(sc_ok && sg < groups) << 31) | inv;
      load_to_lds4(rs, stn + C::SC_OFF + wv * 256, ((uint32_t)sg * (uint32_t)N + (uint32_t)sc_col) * 2u | sbad);
    } else {
      const int zg = g0 + zw_gi;
      const uint32_t zbad = ((uint32_t)!(zw_ok && zg < groups) << 31) | inv;
      load_to_lds4(rz, stn + C::ZW_OFF + wv * 256, ((uint32_t)zg * (uint32_t)(N / 8) + (uint32_t)zw_w) * 4u | zbad);
    }
  };

  // Prologue: the first stage and its weights.
#pragma unroll
  for (int i = NTW; i < NLD; ++i) issue_item(i, step0, 0, 0u);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) cb[nt] = WW::load(rq, woff(nt) + wband(step0));

  for (int step = step0; step < step1; ++step) {
    // Wait for this wave's loads of the current stage, then for everyone's;
    // the barrier also frees the other buffer (read during the last step).
    // The wait is explicit: the compiler does not count loads that write LDS
    // directly when it lowers the barrier's fence (it waited for only part
    // of them), and an explicit s_waitcnt is never relaxed.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const uint32_t inv = (uint32_t)!(step + 1 < step1) << 31;
    const int nbuf = (step + 1 - step0) & 1;
    const char* st = smem + ((step - step0) & 1) * C::STAGE;
    auto frag = [&](int s, int mt) -> h8 {
      return *reinterpret_cast<const h8*>(st + swz<C::CPR>((uint32_t)(arow0 + 16 * mt), (uint32_t)(4 * s + h)));
    };
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) zs_of(st, 0, nt);
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) af[mt] = frag(0, mt);
    h8 bcur = decode_weight_vk(cb[0][0], zc[0], s2[0], kc), bnext;
    if (GS > 1 && KB > 1 && grp(1) != grp(0)) zs_of(st, grp(1), 0);
    // Iteration (s, nt): the MTW MFMAs of column tile nt in substep s, with
    // the next tile's decode and a share of the next stage's loads between
    // them. A scheduling fence ends each iteration: left free, the compiler
    // hoists loads and decodes across iterations and runs out of registers.
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int s = it / NTW, nt = it % NTW;
      // the next stage's loads, weights first; past the last step they read
      // zeros, so the step has no branch
#pragma unroll
      for (int i = (it * NLD + NIT - 1) / NIT; i < ((it + 1) * NLD + NIT - 1) / NIT; ++i)
        issue_item(i, step + 1, nbuf, inv);
      // decode the next column tile while this one's MFMAs run; at a group
      // boundary, that tile's zero point and scale for its next substep
      if (it + 1 < NIT) {
        const int s1 = (it + 1) / NTW, n1 = (it + 1) % NTW;
        bnext = decode_weight_vk(cb[n1][s1], zc[n1], s2[n1], kc);
        if (GS > 1 && s1 + 1 < KB && grp(s1 + 1) != grp(s1)) zs_of(st, grp(s1 + 1), n1);
      }
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt) {
        acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt], bcur, acc[mt][nt], 0, 0, 0);
        // the next substep's fragment right after this one's last use
        if (nt == NTW - 1 && s + 1 < KB) af[mt] = frag(s + 1, mt);
      }
      if (it + 1 < NIT) bcur = bnext;
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) cb[nt] = rb[nt];
  }

  // Lane l, register r of tile (mt, nt): row 4(l/16) + r, column l%16.
  if (EPI && !ws) {
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW / 2; ++nt) {
        const int c = lcol(nt) + (lane & 15);
        const int col = gcol(c);  // gate column = output column
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + 16 * (MTW * wm + mt) + 4 * h + r;
          const float g = acc[mt][nt][r], v = acc[mt][nt + NTW / 2][r];
          if (row < M && gvalid(c)) y[(int64_t)row * NO + col] = __builtin_bit_cast(uint16_t, (_Float16)(g / (1.f + expf(-g)) * v));
        }
      }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int c = lcol(nt) + (lane & 15);
      const int col = gcol(c);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 16 * (MTW * wm + mt) + 4 * h + r;
        const float v = acc[mt][nt][r];
        if (row < M && gvalid(c)) {
          if (ws)
            ws[((int64_t)split * M + row) * N + col] = v;
          else
            y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)v);
        }
      }
    }
}

// y = fp16(sum over s of ws[s]), s in increasing order; four elements per thread.
__global__ __launch_bounds__(256) void prefill_reduce_kernel(const float* __restrict__ ws, uint16_t* __restrict__ y,
                                                             int64_t mn, int splits) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= mn) return;
  f4 a = *reinterpret_cast<const f4*>(ws + i);
  for (int s = 1; s < splits; ++s) a += *reinterpret_cast<const f4*>(ws + (int64_t)s * mn + i);
  typedef uint16_t us4 __attribute__((ext_vector_type(4)));
  us4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = __builtin_bit_cast(uint16_t, (_Float16)a[e]);
  *reinterpret_cast<us4*>(y + i) = o;
}

// Gated epilogue: y[m, i] = fp16(silu(g) * u) with g = sum over s of
// ws[s][m][i] and u = sum over s of ws[s][m][N/2 + i] (increasing s); four
// outputs per thread. N/2 is a multiple of 4.
__global__ __launch_bounds__(256) void prefill_reduce_silu_mul_kernel(const float* __restrict__ ws,
                                                                      uint16_t* __restrict__ y, int M, int N,
                                                                      int splits) {
  const int NO = N / 2;
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (int64_t)M * NO) return;
  const int64_t m = i / NO, c = i % NO;
  const int64_t mn = (int64_t)M * N;
  const float* gp = ws + m * N + c;
  f4 g = *reinterpret_cast<const f4*>(gp);
  f4 u = *reinterpret_cast<const f4*>(gp + NO);
  for (int s = 1; s < splits; ++s) {
    g += *reinterpret_cast<const f4*>(gp + s * mn);
    u += *reinterpret_cast<const f4*>(gp + s * mn + NO);
  }
  typedef uint16_t us4 __attribute__((ext_vector_type(4)));
  us4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = __builtin_bit_cast(uint16_t, (_Float16)(g[e] / (1.f + expf(-g[e])) * u[e]));
  *reinterpret_cast<us4*>(y + i) = o;
}

namespace {

template <int WM, int WN, int MTW, int NTW, int KS, int GS, bool EPI>
hipError_t launch_prefill_e(const LinearArgs& a, int splits, float* ws, const Launch& L) {
  constexpr bool gated = EPI;
  using C = PrefillCfg<WM, WN, MTW, NTW, KS, GS>;
  const int NT = (a.N + 15) / 16;
  const int KT = (a.K + 127) / 128;
  const int n_mtiles = (a.M + C::BM - 1) / C::BM;
  const int n_ntiles = EPI ? (a.N / 2 + C::BN / 2 - 1) / (C::BN / 2) : (a.N + C::BN - 1) / C::BN;
  const int nsteps = (a.K + KS - 1) / KS;
  // Steps per split rounded so that every split is non-empty.
  const int split_steps = (nsteps + splits - 1) / splits;
  splits = (nsteps + split_steps - 1) / split_steps;
  auto k = prefill_kernel<WM, WN, MTW, NTW, KS, GS, EPI>;
  if (C::LDS_BYTES > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       C::LDS_BYTES);
    if (e != hipSuccess) return e;
  }
  const uint32_t qw_bytes = (uint32_t)((size_t)NT * KT * 1024);
  const int n_tiles = n_mtiles * n_ntiles;
  // fp32 partials go to the workspace when K is split (the gated epilogue is
  // then applied where they are added)
  float* part = splits > 1 ? ws : nullptr;
  const Launch first{L.stream, L.start, part ? nullptr : L.stop};
  hipError_t e = launch_kernel(k, dim3((unsigned)(n_tiles * splits)), dim3(C::NTH), C::LDS_BYTES, first, a.x, a.qw,
                               a.scales, a.zeros, a.y, part, a.M, a.K, a.N, a.G, NT, n_mtiles, n_tiles, split_steps,
                               qw_bytes);
  if (e != hipSuccess || !part) return e;
  const int64_t mn = (int64_t)a.M * a.N;
  const Launch second{L.stream, nullptr, L.stop};
  if (gated)
    return launch_kernel(prefill_reduce_silu_mul_kernel, dim3((unsigned)((mn / 2 / 4 + 255) / 256)), dim3(256), 0,
                         second, static_cast<const float*>(part), a.y, a.M, a.N, splits);
  return launch_kernel(prefill_reduce_kernel, dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0, second, part, a.y,
                       mn, splits);
}

template <int WM, int WN, int MTW, int NTW, int KS, int GS>
hipError_t launch_prefill_t(const LinearArgs& a, int splits, float* ws, bool gated, const Launch& L) {
  if (gated) return launch_prefill_e<WM, WN, MTW, NTW, KS, GS, true>(a, splits, ws, L);
  return launch_prefill_e<WM, WN, MTW, NTW, KS, GS, false>(a, splits, ws, L);
}

// Groups per step: KS / G for G < KS, else 1 (G is then a multiple of KS).
template <int WM, int WN, int MTW, int NTW, int KS>
hipError_t launch_prefill_k(const LinearArgs& a, int splits, float* ws, bool gated, const Launch& L) {
  if (a.G < KS) {
    if (KS / a.G == 2) return launch_prefill_t<WM, WN, MTW, NTW, KS, 2>(a, splits, ws, gated, L);
    if (KS == 128 && a.G == 32)
      return launch_prefill_t<WM, WN, MTW, NTW, KS, (KS == 128 ? 4 : 2)>(a, splits, ws, gated, L);
    return hipErrorInvalidValue;
  }
  return launch_prefill_t<WM, WN, MTW, NTW, KS, 1>(a, splits, ws, gated, L);
}

}  // namespace

hipError_t launch_prefill_reduce(float* ws, uint16_t* y, int M, int N, int splits, bool gated, const Launch& L) {
  const int64_t mn = (int64_t)M * N;
  if (gated)
    return launch_kernel(prefill_reduce_silu_mul_kernel, dim3((unsigned)((mn / 2 / 4 + 255) / 256)), dim3(256), 0, L,
                         static_cast<const float*>(ws), y, M, N, splits);
  return launch_kernel(prefill_reduce_kernel, dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0, L,
                       static_cast<const float*>(ws), y, mn, splits);
}

int prefill_steps(int K, int tile) { return (K + (tile == 1 ? 63 : 127)) / (tile == 1 ? 64 : 128); }

namespace {

// Estimated time of a prefill plan, from a model fitted to measurements on
// the LLaMA-shaped layers (MI355X): the workgroups run in rounds of
// `slots` (resident workgroups per chip), each round takes one workgroup's
// K range, and the split-K partials cost a write and a read of fp32 per
// output per split (the partial stores plus the reduction kernel). For the
// fp16 GEMM's 256 x 256 tile the time of one K step depends on how many
// workgroups run at once: with all 256 CUs busy the chip is held at its
// power limit and its clock drops (to about 2.0 GHz), so a round that
// leaves CUs idle runs each step faster (measured: about 2.5 us with 100 or
// fewer busy, 2.7-2.9 with 160, 3.45 with 256). The W4A8 GEMM's steps take
// about 0.7 of the flat fp16 figure and do not speed up on a partly idle
// chip (2.75 us per step at 160 busy, as at 256). Times in microseconds.
double prefill_cost(int M, int K, int N, int tile, int splits, PrefillKind kind) {
  const int bm = tile == 3 ? 256 : 128, bn = tile == 3 ? 256 : 128;
  const double tiles = (double)((M + bm - 1) / bm) * (double)((N + bn - 1) / bn);
  const int steps = prefill_steps(K, tile);
  const double wgs = tiles * splits;
  const double wg_steps = std::ceil((double)steps / splits);
  if (tile == 3 && kind == PrefillKind::kFp16) {
    auto t_step = [](double busy) { return busy <= 96 ? 2.5 : 2.5 + (std::min(busy, 256.0) - 96) * (0.95 / 160); };
    const double full = std::floor(wgs / 256), rest = wgs - full * 256;
    const double reduce = splits > 1 ? 1.1e-6 * splits * (double)M * (double)N : 0.0;
    return wg_steps * (full * t_step(256) + (rest > 0 ? t_step(rest) : 0.0)) + reduce;
  }
  double slots, t_step;  // t_step: one K step of one workgroup
  if (tile == 3) {
    slots = 256, t_step = 3.8;
  } else if (tile == 2) {
    slots = 512, t_step = wgs <= 256 ? 1.6 : 2.8;  // alone on its CU, or sharing it
  } else {
    slots = 768, t_step = 1.9;
  }
  if (kind == PrefillKind::kW4A8) t_step *= 0.7;
  const double reduce = splits > 1 ? 1.4e-6 * splits * (double)M * (double)N : 0.0;
  return std::ceil(wgs / slots) * wg_steps * t_step + reduce;
}

int best_split(int M, int K, int N, int tile, PrefillKind kind, double* cost) {
  const int steps = prefill_steps(K, tile);
  int best = 1;
  double bc = prefill_cost(M, K, N, tile, 1, kind);
  for (int s = 2; s <= 8 && s * 4 <= steps; ++s) {
    const double c = prefill_cost(M, K, N, tile, s, kind);
    if (c < bc) bc = c, best = s;
  }
  if (cost) *cost = bc;
  return best;
}

}  // namespace

void prefill_auto_plan(int M, int K, int N, int* tile, int* splits, PrefillKind kind) {
  // A fixed tile gets its best split; a fixed split its best tile; else both.
  if (*tile && !*splits) {
    *splits = best_split(M, K, N, *tile, kind, nullptr);
    return;
  }
  double bc = 0;
  int bt = 0, bs = 1;
  for (int t = 2; t <= 3; ++t) {
    double c;
    int s = *splits ? *splits : best_split(M, K, N, t, kind, &c);
    if (*splits) c = prefill_cost(M, K, N, t, s, kind);
    if (!bt || c < bc) bc = c, bt = t, bs = s;
  }
  if (!*tile) *tile = bt;
  if (!*splits) *splits = bs;
}

size_t prefill_workspace_bytes(int M, int N, int splits, bool gated) {
  (void)gated;  // the gated epilogue needs the workspace only when K is split
  return splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(float) : 0;
}

bool prefill_fits(int K, int N) { return (size_t)((N + 15) / 16) * ((K + 127) / 128) * 1024 < ((size_t)1 << 31); }

hipError_t noalloc_scratch(float** ptr) {
  // one address per device, looked up with that device current (the caller's)
  static std::atomic<float*> addr[kNoAllocMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
  float* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* v = nullptr;
    e = hipGetSymbolAddress(&v, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    p = static_cast<float*>(v);
    addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_prefill(const LinearArgs& a, int tile, int splits, float* ws, bool gated, const Launch& L) {
  if (!prefill_fits(a.K, a.N)) return hipErrorInvalidValue;
  if (splits > 1 && !ws) return hipErrorInvalidValue;
  if (gated && a.N % 32) return hipErrorInvalidValue;
  switch (tile) {
    case 1: return launch_prefill_k<2, 2, 4, 4, 64>(a, splits, ws, gated, L);   // 128 x 128, 4 waves of 64 x 64, 64-row steps
    case 2: return launch_prefill_k<2, 2, 4, 4, 128>(a, splits, ws, gated, L);  // 128 x 128, 4 waves of 64 x 64, 128-row steps
    case 3: return launch_prefill_k<1, 8, 16, 2, 128>(a, splits, ws, gated, L);  // 256 x 256, 8 waves of 256 x 32, 128-row steps
  }
  return hipErrorInvalidValue;
}

}  // namespace awq
