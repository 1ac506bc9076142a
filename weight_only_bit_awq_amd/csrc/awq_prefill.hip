// Prefill path of the W4A16 linear layer (large M): a dequantise-then-MFMA
// fp16 GEMM with fp32 accumulation.
//
// At prefill sizes (hundreds to thousands of activation rows, as in the
// context stage of "TinyChat: Efficient and Lightweight Chatbot with AWQ",
// section "New Optimization of Context Stage") every weight is reused by many
// rows, so the layer is a dense contraction bound by the matrix cores. Each
// packed weight is decoded to its exact fp16 value (q - z) * s once per wave
// that uses it and fed to v_mfma_f32_16x16x32_f16.
//
// Structure (per workgroup: WM x WN waves, each wave MTW x NTW tiles of 16x16
// outputs; K advances 64 rows per step):
//   * Activations: a BM x 64 fp16 slab per step goes global -> registers ->
//     LDS, double-buffered, so the next slab's loads are in flight while the
//     current one is multiplied. 16-byte chunks of a row are XOR-swizzled by
//     the row index, so the 16-byte fragment reads of 16 consecutive rows hit
//     distinct banks without padding.
//   * Weights: each wave reads the packed words of its own columns straight
//     from global memory into registers one step ahead (8 bytes per lane per
//     16-column tile per step: half of the lane's 16-byte slice of a 128-row
//     tile), and decodes them right before their MFMA. Tiles of one 128-row
//     band are adjacent in the device layout, so these reads are contiguous.
//   * Scale and zero point of every column of the workgroup are staged per
//     step in LDS as one 32-bit word (scale bits | zero << 16).
//   * One barrier per step. Out-of-range rows, columns and K read zero through
//     raw buffer loads and are never stored.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

typedef uint32_t u2 __attribute__((ext_vector_type(2)));

template <int WM, int WN, int MTW, int NTW, int GPS>
struct PrefillCfg {
  static constexpr int NTH = 64 * WM * WN;
  static constexpr int BM = 16 * MTW * WM;
  static constexpr int BN = 16 * NTW * WN;
  static constexpr int KS = 64;                // rows of K per step
  static constexpr int A_BYTES = BM * KS * 2;  // one activation slab
  static constexpr int A_CHUNKS = BM * (KS / 8);
  static constexpr int A_PER_THREAD = A_CHUNKS / NTH;
  static constexpr int SZ_WORDS = GPS * BN;  // (scale, zero) words per step
  static constexpr int SZ_PER = SZ_WORDS >= NTH ? SZ_WORDS / NTH : 1;
  static constexpr int LDS_BYTES = 2 * A_BYTES + 2 * SZ_WORDS * 4;
  static_assert(A_CHUNKS % NTH == 0, "activation slab must split evenly over the threads");
  static_assert(SZ_WORDS % NTH == 0 || NTH % SZ_WORDS == 0, "scale staging split");
};

// Byte offset of 16-byte chunk `chunk` (0..7) of slab row `row` (128-byte rows).
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) {
  return row * 128u + ((chunk ^ (row & 7u)) << 4);
}

template <int WM, int WN, int MTW, int NTW, int GPS>
__global__ __launch_bounds__(64 * WM * WN) void prefill_kernel(const uint16_t* __restrict__ x,
                                                               const uint32_t* __restrict__ qw,
                                                               const uint16_t* __restrict__ scales,
                                                               const uint32_t* __restrict__ zeros,
                                                               uint16_t* __restrict__ y, int M, int K, int N, int G,
                                                               int NT, int n_mtiles, uint32_t qw_bytes) {
  using C = PrefillCfg<WM, WN, MTW, NTW, GPS>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* a_lds = smem;                                                      // 2 x A_BYTES
  uint32_t* sz_lds = reinterpret_cast<uint32_t*>(smem + 2 * C::A_BYTES);  // 2 x SZ_WORDS

  const int u = xcd_remap(blockIdx.x, gridDim.x);
  const int mtile = u % n_mtiles;
  const int ntile = u / n_mtiles;
  const int m0 = mtile * C::BM;
  const int n0 = ntile * C::BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv / WN, wn = wv % WN;
  const int h = lane >> 4;
  const int groups = K / G;
  const int nsteps = (K + C::KS - 1) / C::KS;

  const rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const rsrc_t rq = make_rsrc(qw, qw_bytes);
  const rsrc_t rs = make_rsrc(scales, (uint32_t)groups * (uint32_t)N * 2u);
  const rsrc_t rz = make_rsrc(zeros, (uint32_t)groups * (uint32_t)(N / 8) * 4u);

  // Activation chunk c = tid + i*NTH of a slab: row c / 8, 16-byte chunk c % 8.
  uint32_t a_goff[C::A_PER_THREAD], a_loff[C::A_PER_THREAD];
#pragma unroll
  for (int i = 0; i < C::A_PER_THREAD; ++i) {
    const uint32_t c = tid + i * C::NTH;
    const uint32_t row = c >> 3, ch = c & 7u;
    const int grow = m0 + (int)row;
    a_goff[i] = grow < M ? ((uint32_t)grow * K + ch * 8u) * 2u : kOOB;
    a_loff[i] = swz(row, ch);
  }
  // This lane's slice of each of the wave's NTW column tiles in band 0.
  uint32_t b_off[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int ct = n0 / 16 + NTW * wn + nt;
    b_off[nt] = ct < NT ? (uint32_t)ct * 1024u + (uint32_t)lane * 16u : kOOB;
  }

  auto load_a = [&](int step, u4(&ra)[C::A_PER_THREAD]) {
    const uint32_t kb = (uint32_t)step * C::KS * 2u;
#pragma unroll
    for (int i = 0; i < C::A_PER_THREAD; ++i) {
      // chunks past K (a ragged last step) would read the next row: mask them
      const uint32_t ch = (tid + i * C::NTH) & 7u;
      const uint32_t bad = (uint32_t)!(step * C::KS + (int)ch * 8 < K) << 31;
      ra[i] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rx, (a_goff[i] + kb) | bad, 0, 0));
    }
  };
  auto load_b = [&](int step, u2(&rb)[NTW]) {
    const uint32_t band = (uint32_t)(step >> 1) * (uint32_t)NT * 1024u + (uint32_t)(step & 1) * 8u;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
      rb[nt] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(rq, b_off[nt] + band, 0, 0));
  };
  auto load_sz = [&](int step, uint32_t(&rs_)[C::SZ_PER], uint32_t(&rz_)[C::SZ_PER]) {
#pragma unroll
    for (int i = 0; i < C::SZ_PER; ++i) {
      const int e = tid + i * C::NTH;
      const int gi = e / C::BN, cc = e % C::BN;
      const int col = n0 + cc;
      const int g = (step * C::KS + gi * 32) / G;
      const uint32_t bad = (uint32_t)!(e < C::SZ_WORDS && col < N && g < groups) << 31;
      rs_[i] = __builtin_amdgcn_raw_buffer_load_b16(rs, ((uint32_t)(g * N + col) * 2u) | bad, 0, 0);
      const uint32_t zw =
          __builtin_amdgcn_raw_buffer_load_b32(rz, ((uint32_t)(g * (N / 8) + (col >> 3)) * 4u) | bad, 0, 0);
      rz_[i] = (zw >> (4 * (col & 7))) & 0xFu;
    }
  };
  auto store_stage = [&](int buf, const u4(&ra)[C::A_PER_THREAD], const uint32_t(&rs_)[C::SZ_PER],
                         const uint32_t(&rz_)[C::SZ_PER]) {
    char* ab = a_lds + buf * C::A_BYTES;
#pragma unroll
    for (int i = 0; i < C::A_PER_THREAD; ++i) *reinterpret_cast<u4*>(ab + a_loff[i]) = ra[i];
    uint32_t* sb = sz_lds + buf * C::SZ_WORDS;
#pragma unroll
    for (int i = 0; i < C::SZ_PER; ++i) {
      const int e = tid + i * C::NTH;
      if (e < C::SZ_WORDS) sb[e] = rs_[i] | (rz_[i] << 16);
    }
  };

  f4 acc[MTW][NTW];
#pragma unroll
  for (int a = 0; a < MTW; ++a)
#pragma unroll
    for (int b = 0; b < NTW; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};

  u4 ra[C::A_PER_THREAD];
  u2 rb[NTW], cb[NTW];
  uint32_t rsv[C::SZ_PER], rzv[C::SZ_PER];
  load_a(0, ra);
  load_b(0, cb);
  load_sz(0, rsv, rzv);
  store_stage(0, ra, rsv, rzv);
  __syncthreads();

  const DecodeConsts kc = decode_consts();
  const int arow0 = 16 * MTW * wm + (lane & 15);
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) {
      load_a(step + 1, ra);
      load_b(step + 1, rb);
      load_sz(step + 1, rsv, rzv);
    }
    const char* ab = a_lds + buf * C::A_BYTES;
    const uint32_t* sb = sz_lds + buf * C::SZ_WORDS;
#pragma unroll
    for (int s = 0; s < 2; ++s) {  // two 32-row MFMA steps per 64-row step
      h8 af[MTW];
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
        af[mt] = *reinterpret_cast<const h8*>(ab + swz((uint32_t)(arow0 + 16 * mt), (uint32_t)(4 * s + h)));
      const int gi = GPS == 2 ? s : 0;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const uint32_t mw = sb[gi * C::BN + 16 * (NTW * wn + nt) + (lane & 15)];
        const h8 bw = decode_weight_vk(cb[nt][s], zero_const(mw >> 16), splat_h2((uint16_t)(mw & 0xFFFFu)), kc);
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt], bw, acc[mt][nt], 0, 0, 0);
      }
    }
    if (more) {
      store_stage(buf ^ 1, ra, rsv, rzv);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) cb[nt] = rb[nt];
    }
    __syncthreads();
  }

  // Lane l, register r of tile (mt, nt): row 4(l/16) + r, column l%16.
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int col = n0 + 16 * (NTW * wn + nt) + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 16 * (MTW * wm + mt) + 4 * h + r;
        const float v = acc[mt][nt][r];
        if (row < M && col < N) y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
}

namespace {

template <int WM, int WN, int MTW, int NTW, int GPS>
hipError_t launch_prefill_t(const LinearArgs& a, const Launch& L) {
  using C = PrefillCfg<WM, WN, MTW, NTW, GPS>;
  const int NT = (a.N + 15) / 16;
  const int KT = (a.K + 127) / 128;
  const int n_mtiles = (a.M + C::BM - 1) / C::BM;
  const int n_ntiles = (a.N + C::BN - 1) / C::BN;
  auto k = prefill_kernel<WM, WN, MTW, NTW, GPS>;
  if (C::LDS_BYTES > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       C::LDS_BYTES);
    if (e != hipSuccess) return e;
  }
  const uint32_t qw_bytes = (uint32_t)((size_t)NT * KT * 1024);
  return launch_kernel(k, dim3((unsigned)(n_mtiles * n_ntiles)), dim3(C::NTH), C::LDS_BYTES, L, a.x, a.qw,
                       a.scales, a.zeros, a.y, a.M, a.K, a.N, a.G, NT, n_mtiles, qw_bytes);
}

template <int GPS>
hipError_t launch_prefill_g(const LinearArgs& a, int tile, const Launch& L) {
  switch (tile) {
    case 1: return launch_prefill_t<2, 2, 4, 4, GPS>(a, L);  // 128 x 128, 4 waves of 64 x 64
    case 2: return launch_prefill_t<2, 4, 4, 4, GPS>(a, L);  // 128 x 256, 8 waves of 64 x 64
    case 3: return launch_prefill_t<2, 4, 8, 4, GPS>(a, L);  // 256 x 256, 8 waves of 128 x 64
  }
  return hipErrorInvalidValue;
}

}  // namespace

int prefill_auto_tile(int M, int N) {
  // The 256 x 256 tile halves the activation and weight re-reads of the
  // 128 x 128 one and does half the redundant decoding per MFMA, but holds a
  // CU with one workgroup: it wins once there are enough of them to cover
  // most of the 256 CUs (measured: 216 tiles already beat 864 small ones).
  const long t3 = (long)((M + 255) / 256) * ((N + 255) / 256);
  return t3 >= 200 ? 3 : 1;
}

bool prefill_fits(int K, int N) { return (size_t)((N + 15) / 16) * ((K + 127) / 128) * 1024 < ((size_t)1 << 31); }

hipError_t launch_prefill(const LinearArgs& a, int tile, const Launch& L) {
  if (!prefill_fits(a.K, a.N)) return hipErrorInvalidValue;
  if (a.G == 32) return launch_prefill_g<2>(a, tile, L);
  return launch_prefill_g<1>(a, tile, L);
}

}  // namespace awq
