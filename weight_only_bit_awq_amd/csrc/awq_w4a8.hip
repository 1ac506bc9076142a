// W4A8-FP8 form of the group-quantised linear layer: activations quantised
// per token to FP8 (OCP E4M3), 4-bit weights decoded to exact FP8 (q - z),
// products on the gfx950 FP8 matrix cores, group scales and the token scale
// applied in fp32.
//
// The TensorRT-LLM news page (Falcon-180B with INT4 AWQ on one H200) has the
// AWQ kernels compute in FP8. On gfx950 the FP8 matrix cores run at twice the
// fp16 rate, so for prefill-sized M the layer can pass the fp16 MFMA bound.
//
// Arithmetic
//   * Activation row m: amax = max |x|, inv = fp32(448 / amax),
//     code = E4M3(fp32(x * inv)) (round to nearest even), sx = fp32(amax / 448);
//     a zero row gets codes 0 and sx = 0.
//   * (q - z) is an integer in [-15, 15], exact in E4M3; the MFMA sums
//     x8 * (q - z) over one 128-row group (exact products, fp32 sums), the
//     group's fp16 scale multiplies that sum into the fp32 accumulator, and
//     the token scale multiplies the result before the fp16 rounding.
//
// Layout of the quantised activations (internal): [M, K] bytes, and inside
// every 128-column block the 8-column chunk c = 4j + h (columns 8c .. 8c+7) is
// stored at chunk position 4h + j. A lane of MFMA row group h then finds the
// 32 bytes it multiplies with its weight words (rows 32j + 8h .. +7 of a
// 128-row band, j = 0..3, the device layout's row set of that lane) as one
// contiguous 32-byte run.
//
// GEMM: workgroup tiles of (16 MTW) x (16 NTW WN) outputs, each of the WN
// waves over all rows of its NTW column tiles (every weight decoded once per
// workgroup), one 128-row K step per group row; the activation slab copied
// global -> LDS by buffer loads with the LDS bit one step ahead
// (XOR-swizzled 16-byte chunks); each lane's weight words, zero word and
// scale loaded into registers two steps ahead and decoded to FP8 one step
// ahead, under the current step's MFMAs; split-K through an fp32 workspace
// summed in a fixed order by the prefill reduction kernel.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef short s2v __attribute__((ext_vector_type(2)));
typedef uint32_t u2w __attribute__((ext_vector_type(2)));

namespace {

// Two fp32 (or the fp16 pair) -> two E4M3 bytes in the low or high half of
// `old` (round to nearest even; unit scale).
template <bool HI>
__device__ __forceinline__ s2v fp8x2_f32(s2v old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, a, b, 1.0f, HI);
}
template <bool HI>
__device__ __forceinline__ s2v fp8x2_f16(s2v old, h2 v) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(old, v, 1.0f, HI);
}

// Eight rows (q - z) of one device word as E4M3 bytes in row order: the
// exact fp16 pairs of the code decode, converted (exactly) to FP8.
__device__ __forceinline__ u2w decode_fp8(uint32_t w, ZeroConst c, const DecodeConsts& k) {
  const uint32_t w8 = w >> 8;
  const h2 p0 = as_h2(and_or(w, k.m1, k.o1)) + as_h2(c.c1024);
  const h2 p1 = as_h2(and_or(w, k.m2, k.o2)) + as_h2(c.c64);
  const h2 p2 = as_h2(and_or(w8, k.m1, k.o1)) + as_h2(c.c1024);
  const h2 p3 = as_h2(and_or(w8, k.m2, k.o2)) + as_h2(c.c64);
  s2v lo = s2v{0, 0}, hi = s2v{0, 0};
  lo = fp8x2_f16<false>(lo, p0);
  lo = fp8x2_f16<true>(lo, p1);
  hi = fp8x2_f16<false>(hi, p2);
  hi = fp8x2_f16<true>(hi, p3);
  return u2w{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

}  // namespace

// One workgroup of 256 threads per activation row.
__global__ __launch_bounds__(256) void act_quant_fp8_kernel(const uint16_t* __restrict__ x, int K,
                                                            uint8_t* __restrict__ x8, float* __restrict__ sx) {
  const int m = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* xr = x + (int64_t)m * K;
  uint8_t* outr = x8 + (int64_t)m * K;
  const int nch = K / 8;
  float amax = 0.f;
  for (int c = tid; c < nch; c += 256) {
    const h8 v = *reinterpret_cast<const h8*>(xr + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[e]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  __shared__ float red[4];
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if (tid == 0) sx[m] = amax > 0.f ? amax / 448.0f : 0.f;
  const float inv = amax > 0.f ? 448.0f / amax : 0.f;
  for (int c = tid; c < nch; c += 256) {
    u2w out = u2w{0u, 0u};
    if (amax > 0.f) {
      const h8 v = *reinterpret_cast<const h8*>(xr + 8 * c);
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = (float)v[e] * inv;
      s2v lo = s2v{0, 0}, hi = s2v{0, 0};
      lo = fp8x2_f32<false>(lo, f[0], f[1]);
      lo = fp8x2_f32<true>(lo, f[2], f[3]);
      hi = fp8x2_f32<false>(hi, f[4], f[5]);
      hi = fp8x2_f32<true>(hi, f[6], f[7]);
      out = u2w{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    }
    const int ci = c & 15;  // chunk 4j + h of its 128-column block -> position 4h + j
    const int pos = (c & ~15) | ((ci & 3) << 2) | (ci >> 2);
    *reinterpret_cast<u2w*>(outr + 8 * pos) = out;
  }
}

template <int WN, int MTW, int NTW>
struct W8Cfg {
  static constexpr int NW = WN;                 // waves side by side along N, each over all BM rows
  static constexpr int NTH = 64 * NW;
  static constexpr int BM = 16 * MTW;
  static constexpr int BN = 16 * NTW * WN;
  static constexpr int KS = 128;                // one step = one 128-row band
  static constexpr int CPR = KS / 16;           // 16-byte chunks per slab row (fp8)
  static constexpr int A_BYTES = BM * KS;       // one activation slab
  static constexpr int A_DMA = BM * CPR / NTH;  // 16-byte loads per thread per step
  static constexpr int LDS_BYTES = 2 * A_BYTES;
  static_assert((BM * CPR) % NTH == 0, "activation slab must split evenly over the threads");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// Byte offset of 16-byte chunk `chunk` of slab row `row`: the chunk index is
// XORed with (row / 2) % 8, so the 16-byte reads of 16 consecutive rows at
// one chunk fall on 16 distinct bank groups (two 128-byte rows per 256-byte
// bank row).
__device__ __forceinline__ uint32_t swz8(uint32_t row, uint32_t chunk) {
  return row * 128u + ((chunk ^ ((row >> 1) & 7u)) << 4);
}

// What a lane needs of one step for its NTW column tiles: its 16-byte slice
// of each 128-row weight tile, the packed zero word and the fp16 scale of
// its column.
template <int NTW, int GPS>
struct StepWords {
  u4 w[NTW];
  uint32_t zw[NTW][GPS];
  uint32_t sc[NTW][GPS];
};

// Each wave owns NTW column tiles over all BM rows, so every weight word is
// decoded once per workgroup. A step's words, zero words and scales arrive
// in registers two steps ahead and are decoded to FP8 one step ahead, in the
// shadow of the current step's MFMAs (the loop body has no branches: loads
// past the last step read zero through out-of-range buffer offsets).
// GPS: groups per 128-row step (1 for G a multiple of 128; 2 for G = 64 and
// 4 for G = 32, where each 32-row block of a lane's words -- one word, eight
// FP8 bytes -- is the B operand of one v_mfma_f32_16x16x32_fp8_fp8 and the
// group's scale multiplies the sum of its blocks).
template <int WN, int MTW, int NTW, int GPS>
__global__ __launch_bounds__(64 * WN) void w4a8_gemm_kernel(const uint8_t* __restrict__ x8,
                                                          const float* __restrict__ sx,
                                                          const uint32_t* __restrict__ qw,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint32_t* __restrict__ zeros,
                                                          uint16_t* __restrict__ y, float* __restrict__ ws, int M,
                                                          int K, int N, int G, int NT, int n_mtiles, int n_tiles,
                                                          int split_steps, uint32_t qw_bytes) {
  using C = W8Cfg<WN, MTW, NTW>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int u = xcd_remap(blockIdx.x, gridDim.x);
  const int split = u / n_tiles;
  const int tile = u - split * n_tiles;
  const int n_ntiles = n_tiles / n_mtiles;
  const int mtile = tile / n_ntiles;
  const int ntile = tile % n_ntiles;
  const int m0 = mtile * C::BM;
  const int n0 = ntile * C::BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 4;
  const int groups = K / G;
  const int nsteps = K / C::KS;
  const int step0 = split * split_steps;
  const int step1 = min(nsteps, step0 + split_steps);

  const rsrc_t rx = make_rsrc(x8, (uint32_t)M * (uint32_t)K);
  const rsrc_t rq = make_rsrc(qw, qw_bytes);
  const rsrc_t rs = make_rsrc(scales, (uint32_t)groups * (uint32_t)N * 2u);
  const rsrc_t rz = make_rsrc(zeros, (uint32_t)groups * (uint32_t)(N / 8) * 4u);

  // Activation load j of this thread fills slab chunk p = (j*NW + wave)*64 + lane:
  // row p / CPR, stored position p % CPR, global chunk (p % CPR) ^ ((row/2) % 8).
  uint32_t a_goff[C::A_DMA];
#pragma unroll
  for (int j = 0; j < C::A_DMA; ++j) {
    const uint32_t p = (uint32_t)(j * C::NW + wn) * 64u + (uint32_t)lane;
    const uint32_t row = p / C::CPR;
    const uint32_t ch = (p % C::CPR) ^ ((row >> 1) & 7u);
    const int grow = m0 + (int)row;
    a_goff[j] = grow < M ? (uint32_t)grow * (uint32_t)K + 16u * ch : kOOB;
  }
  // This lane's column in each of its tiles.
  uint32_t b_off[NTW], z_off[NTW], s_off[NTW], zsh[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int c0 = n0 + 16 * (NTW * wn + nt);
    const int col = c0 + (lane & 15);
    b_off[nt] = c0 < N ? (uint32_t)(c0 / 16) * 1024u + (uint32_t)lane * 16u : kOOB;
    z_off[nt] = col < N ? (uint32_t)(col / 8) * 4u : kOOB;
    s_off[nt] = col < N ? (uint32_t)col * 2u : kOOB;
    zsh[nt] = 4u * (uint32_t)(col % 8);
  }

  auto issue_stage = [&](int step, int buf) {
    char* st = smem + buf * C::A_BYTES;
    const uint32_t bad = (uint32_t)!(step < step1) << 31;
    const uint32_t k0 = (uint32_t)step * C::KS;
#pragma unroll
    for (int j = 0; j < C::A_DMA; ++j) load_to_lds16(rx, st + (j * C::NW + wn) * 1024, (a_goff[j] + k0) | bad);
  };
  auto load_step = [&](int step, StepWords<NTW, GPS>& d) {
    const uint32_t bad = (uint32_t)!(step < step1) << 31;
    const uint32_t band = (uint32_t)step * (uint32_t)NT * 1024u;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      d.w[nt] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rq, (b_off[nt] + band) | bad, 0, 0));
#pragma unroll
      for (int gi = 0; gi < GPS; ++gi) {
        const uint32_t g = (uint32_t)((step * C::KS) / G + gi);
        d.zw[nt][gi] = __builtin_amdgcn_raw_buffer_load_b32(rz, (z_off[nt] + g * (uint32_t)(N / 8) * 4u) | bad, 0, 0);
        d.sc[nt][gi] = __builtin_amdgcn_raw_buffer_load_b16(rs, (s_off[nt] + g * (uint32_t)N * 2u) | bad, 0, 0);
      }
    }
  };
  const DecodeConsts kc = decode_consts();
  auto decode_step = [&](const StepWords<NTW, GPS>& d, v8i (&bf)[NTW], float (&sc)[NTW][GPS]) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
      for (int gi = 0; gi < GPS; ++gi) sc[nt][gi] = (float)__builtin_bit_cast(_Float16, (uint16_t)d.sc[nt][gi]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const ZeroConst zc = zero_const((d.zw[nt][j * GPS / 4] >> zsh[nt]) & 0xFu);
        const u2w dd = decode_fp8(d.w[nt][j], zc, kc);
        bf[nt][2 * j] = (int)dd[0];
        bf[nt][2 * j + 1] = (int)dd[1];
      }
    }
  };

  f4 acc[MTW][NTW];
#pragma unroll
  for (int a = 0; a < MTW; ++a)
#pragma unroll
    for (int b = 0; b < NTW; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};

  StepWords<NTW, GPS> dn;  // words of the next step
  v8i bf[NTW];             // current step, decoded
  float sc[NTW][GPS];
  issue_stage(step0, 0);
  {
    StepWords<NTW, GPS> d0;
    load_step(step0, d0);
    load_step(step0 + 1, dn);
    __builtin_amdgcn_s_waitcnt(0);
    decode_step(d0, bf, sc);
  }

  const int arow0 = lane & 15;
  for (int step = step0; step < step1; ++step) {
    // Explicit wait: the barrier's own fence does not count the loads that
    // write LDS directly.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    issue_stage(step + 1, (step + 1 - step0) & 1);
    StepWords<NTW, GPS> d2;
    load_step(step + 2, d2);
    // Next step's weights into a second set of registers (their loads were
    // waited for at the top), free to interleave with this step's MFMAs.
    v8i bfn[NTW];
    float scn[NTW][GPS];
    decode_step(dn, bfn, scn);
    const char* st = smem + ((step - step0) & 1) * C::A_BYTES;
    auto a_frag = [&](int mt) {
      const uint32_t row = (uint32_t)(arow0 + 16 * mt);  // the 32 bytes of row group h
      const u4 a0 = *reinterpret_cast<const u4*>(st + swz8(row, 2u * h));
      const u4 a1 = *reinterpret_cast<const u4*>(st + swz8(row, 2u * h + 1u));
      return v8i{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    };
    if constexpr (GPS == 1) {
      // Row tiles in a software pipeline: the MFMAs of row tile mt go to
      // their own temporaries before the group-scale multiply-adds of row
      // tile mt-1.
      f4 tp[2][NTW];
#pragma unroll
      for (int mt = 0; mt <= MTW; ++mt) {
        if (mt < MTW) {
          const v8i af = a_frag(mt);
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt)
            tp[mt & 1][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[nt], f4{0.f, 0.f, 0.f, 0.f}, 0,
                                                                               0, 0, 127, 0, 127);
        }
        if (mt > 0) {
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) acc[mt - 1][nt] += sc[nt][0] * tp[(mt - 1) & 1][nt];
        }
      }
    } else {
      // Each 32-row block j: the lane's bytes 8j .. 8j+7 of A and B; the
      // blocks of one group summed by the MFMA, then scaled.
      constexpr int BPG = 4 / GPS;  // 32-row blocks per group
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt) {
        const v8i af = a_frag(mt);
        f4 tg[NTW][GPS];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int gi = 0; gi < GPS; ++gi) {
            f4 tt = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jb = 0; jb < BPG; ++jb) {
              const int j = gi * BPG + jb;
              const long a8 = (long)(uint32_t)af[2 * j] | ((long)(uint32_t)af[2 * j + 1] << 32);
              const long b8 = (long)(uint32_t)bf[nt][2 * j] | ((long)(uint32_t)bf[nt][2 * j + 1] << 32);
              tt = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a8, b8, tt, 0, 0, 0);
            }
            tg[nt][gi] = tt;
          }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int gi = 0; gi < GPS; ++gi) acc[mt][nt] += sc[nt][gi] * tg[nt][gi];
      }
    }
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      bf[nt] = bfn[nt];
#pragma unroll
      for (int gi = 0; gi < GPS; ++gi) sc[nt][gi] = scn[nt][gi];
    }
    dn = d2;
  }

  // Lane l, register r of tile (mt, nt): row 4(l/16) + r, column l%16.
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + 16 * mt + 4 * h + r;
      if (row >= M) continue;
      const float s_row = sx[row];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int col = n0 + 16 * (NTW * wn + nt) + (lane & 15);
        if (col >= N) continue;
        const float v = acc[mt][nt][r] * s_row;
        if (ws)
          ws[((int64_t)split * M + row) * N + col] = v;
        else
          y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
}

hipError_t launch_act_quant_fp8(const uint16_t* x, int M, int K, uint8_t* x8, float* sx, const Launch& L) {
  if (M == 0 || K == 0) return hipSuccess;
  return launch_kernel(act_quant_fp8_kernel, dim3((unsigned)M), dim3(256), 0, L, x, K, x8, sx);
}

size_t w4a8_workspace_bytes(int M, int K, int N, int splits) {
  const size_t a = ((size_t)M * K + 255) / 256 * 256;
  const size_t s = ((size_t)M * 4 + 255) / 256 * 256;
  return a + s + (splits > 1 ? (size_t)splits * M * N * 4 : 0);
}

namespace {
template <int WN, int MTW, int NTW, int GPS>
hipError_t launch_w4a8_tile(const uint8_t* x8, const float* sx, const LinearArgs& a, int splits, float* ws,
                            const Launch& L) {
  using C = W8Cfg<WN, MTW, NTW>;
  const int n_mtiles = (a.M + C::BM - 1) / C::BM;
  const int n_ntiles = (a.N + C::BN - 1) / C::BN;
  const int n_tiles = n_mtiles * n_ntiles;
  const int nsteps = a.K / C::KS;
  const int split_steps = (nsteps + splits - 1) / splits;
  const int used = (nsteps + split_steps - 1) / split_steps;
  const int NT = (a.N + 15) / 16;
  const uint32_t qw_bytes = (uint32_t)((size_t)NT * ((a.K + 127) / 128) * 1024);
  auto k = w4a8_gemm_kernel<WN, MTW, NTW, GPS>;
  if (C::LDS_BYTES > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       C::LDS_BYTES);
    if (e != hipSuccess) return e;
  }
  const Launch first{L.stream, L.start, used > 1 ? nullptr : L.stop};
  hipError_t e = launch_kernel(k, dim3((unsigned)(n_tiles * used)), dim3(C::NTH), C::LDS_BYTES, first, x8, sx, a.qw,
                               a.scales, a.zeros, a.y, used > 1 ? ws : (float*)nullptr, a.M, a.K, a.N, a.G, NT,
                               n_mtiles, n_tiles, split_steps, qw_bytes);
  if (e != hipSuccess || used <= 1) return e;
  return launch_prefill_reduce(ws, a.y, a.M, a.N, used, false, Launch{L.stream, nullptr, L.stop});
}
}  // namespace

hipError_t launch_w4a8(const LinearArgs& a, int tile, int splits, void* ws, const Launch& L) {
  uint8_t* x8 = (uint8_t*)ws;
  const size_t a_bytes = ((size_t)a.M * a.K + 255) / 256 * 256;
  float* sx = (float*)((char*)ws + a_bytes);
  float* part = (float*)((char*)ws + a_bytes + ((size_t)a.M * 4 + 255) / 256 * 256);
  hipError_t e = launch_act_quant_fp8(a.x, a.M, a.K, x8, sx, L.start ? Launch{L.stream, L.start, nullptr} : L);
  if (e != hipSuccess) return e;
  const Launch L2{L.stream, nullptr, L.stop};
  // 256 x 256 (8 waves of 256 x 32) or 128 x 128 (4 waves of 128 x 32); groups per 128-row step
  if (a.G % 128 == 0)
    return tile == 3 ? launch_w4a8_tile<8, 16, 2, 1>(x8, sx, a, splits, part, L2)
                     : launch_w4a8_tile<4, 8, 2, 1>(x8, sx, a, splits, part, L2);
  if (a.G == 64)
    return tile == 3 ? launch_w4a8_tile<8, 16, 2, 2>(x8, sx, a, splits, part, L2)
                     : launch_w4a8_tile<4, 8, 2, 2>(x8, sx, a, splits, part, L2);
  if (a.G == 32)
    return tile == 3 ? launch_w4a8_tile<8, 16, 2, 4>(x8, sx, a, splits, part, L2)
                     : launch_w4a8_tile<4, 8, 2, 4>(x8, sx, a, splits, part, L2);
  return hipErrorInvalidValue;
}

}  // namespace awq
