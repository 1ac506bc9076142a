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
//     from global memory into registers one step ahead (KS/128 of the lane's
//     16-byte slice of a 128-row tile per column tile) and decodes them right
//     before their MFMA. Tiles of one 128-row band are adjacent in the device
//     layout, so these reads are contiguous.
//   * One barrier per step; out-of-range rows, columns and K read zero (the
//     loads' out-of-range lanes write zeros to LDS) and are never stored.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

typedef uint32_t u2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr;

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

// Copy 16 (or 4) bytes per lane from the buffer at byte offset `off` into
// LDS at lds + 16 * lane (lds + 4 * lane). The size must be a literal here:
// inside a template the host pass of the compiler rejects it.
__device__ __forceinline__ void load_to_lds16(rsrc_t r, char* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void load_to_lds4(rsrc_t r, char* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)lds, 4, off, 0, 0, 0);
}

// Byte offset of 16-byte chunk `chunk` of slab row `row` (rows of CPR chunks).
template <int CPR>
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk) {
  return row * (16u * CPR) + ((chunk ^ (row % CPR)) << 4);
}

template <int WM, int WN, int MTW, int NTW, int KS, int GS>
__global__ __launch_bounds__(64 * WM * WN) void prefill_kernel(const uint16_t* __restrict__ x,
                                                               const uint32_t* __restrict__ qw,
                                                               const uint16_t* __restrict__ scales,
                                                               const uint32_t* __restrict__ zeros,
                                                               uint16_t* __restrict__ y, int M, int K, int N, int G,
                                                               int NT, int n_mtiles, uint32_t qw_bytes) {
  using C = PrefillCfg<WM, WN, MTW, NTW, KS, GS>;
  using WW = WeightWords<C::KB>;
  typedef typename WW::T wvec;
  extern __shared__ __attribute__((aligned(16))) char smem[];

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
  const int nsteps = (K + KS - 1) / KS;

  const rsrc_t rx = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const rsrc_t rq = make_rsrc(qw, qw_bytes);
  const rsrc_t rs = make_rsrc(scales, (uint32_t)groups * (uint32_t)N * 2u);
  const rsrc_t rz = make_rsrc(zeros, (uint32_t)groups * (uint32_t)(N / 8) * 4u);

  // Activation load j of this thread fills slab chunk p = (j*NW + wave)*64 + lane:
  // row p / CPR, stored column p % CPR, i.e. global chunk (p % CPR) ^ (row % CPR).
  uint32_t a_goff[C::A_DMA], a_k[C::A_DMA];
#pragma unroll
  for (int j = 0; j < C::A_DMA; ++j) {
    const uint32_t p = (uint32_t)(j * C::NW + wv) * 64u + (uint32_t)lane;
    const uint32_t row = p / C::CPR;
    const uint32_t ch = (p % C::CPR) ^ (row % C::CPR);
    const int grow = m0 + (int)row;
    a_goff[j] = grow < M ? ((uint32_t)grow * (uint32_t)K + 8u * ch) * 2u : kOOB;
    a_k[j] = 8u * ch;
  }
  // Dword tid of the scale region: columns 2c, 2c+1 of group row gi; of the
  // zero region: packed word c of group row gi.
  const int sc_gi = tid / (C::BN / 2), sc_col = n0 + 2 * (tid % (C::BN / 2));
  const bool sc_ok = sc_gi < GS && sc_col < N;
  const int zw_gi = tid / (C::BN / 8), zw_w = n0 / 8 + tid % (C::BN / 8);
  const bool zw_ok = zw_gi < GS && zw_w < N / 8;
  // This lane's slice of each of the wave's NTW column tiles in band 0.
  uint32_t b_off[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int ct = n0 / 16 + NTW * wn + nt;
    b_off[nt] = ct < NT ? (uint32_t)ct * 1024u + (uint32_t)lane * 16u : kOOB;
  }

  auto issue_stage = [&](int step, int buf) {
    char* st = smem + buf * C::STAGE;
    const uint32_t k0 = (uint32_t)step * KS;
#pragma unroll
    for (int j = 0; j < C::A_DMA; ++j) {
      const uint32_t bad = (uint32_t)!(k0 + a_k[j] < (uint32_t)K) << 31;
      load_to_lds16(rx, st + (j * C::NW + wv) * 1024, (a_goff[j] + k0 * 2u) | bad);
    }
    const int g0 = GS > 1 ? step * GS : (step * KS) / G;  // first group of the step
    const int sg = g0 + sc_gi, zg = g0 + zw_gi;
    const uint32_t sbad = (uint32_t)!(sc_ok && sg < groups) << 31;
    const uint32_t zbad = (uint32_t)!(zw_ok && zg < groups) << 31;
    load_to_lds4(rs, st + C::SC_OFF + wv * 256, ((uint32_t)sg * (uint32_t)N + (uint32_t)sc_col) * 2u | sbad);
    load_to_lds4(rz, st + C::ZW_OFF + wv * 256, ((uint32_t)zg * (uint32_t)(N / 8) + (uint32_t)zw_w) * 4u | zbad);
  };
  auto load_b = [&](int step, wvec(&rb)[NTW]) {
    const uint32_t band = KS == 128 ? (uint32_t)step * (uint32_t)NT * 1024u
                                    : (uint32_t)(step >> 1) * (uint32_t)NT * 1024u + (uint32_t)(step & 1) * 8u;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) rb[nt] = WW::load(rq, b_off[nt] + band);
  };

  f4 acc[MTW][NTW];
#pragma unroll
  for (int a = 0; a < MTW; ++a)
#pragma unroll
    for (int b = 0; b < NTW; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};

  wvec cb[NTW], rb[NTW];
  issue_stage(0, 0);
  load_b(0, cb);

  const DecodeConsts kc = decode_consts();
  const int arow0 = 16 * MTW * wm + (lane & 15);
  const int ccol0 = 16 * NTW * wn + (lane & 15);  // column within the workgroup tile, nt = 0
  for (int step = 0; step < nsteps; ++step) {
    // Wait for this wave's loads of the current stage, then for everyone's;
    // the barrier also frees the other buffer (read during the last step).
    // The wait is explicit: the compiler does not count loads that write LDS
    // directly when it lowers the barrier's fence (it waited for only part
    // of them), and an explicit s_waitcnt is never relaxed.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const bool more = step + 1 < nsteps;
    if (more) {
      load_b(step + 1, rb);
      issue_stage(step + 1, (step + 1) & 1);
    }
    const char* st = smem + (step & 1) * C::STAGE;
    const uint16_t* sc_l = reinterpret_cast<const uint16_t*>(st + C::SC_OFF);
    const uint32_t* zw_l = reinterpret_cast<const uint32_t*>(st + C::ZW_OFF);
    ZeroConst zc[NTW];
    h2 s2[NTW];
#pragma unroll
    for (int s = 0; s < C::KB; ++s) {
      const int gi = GS == 1 ? 0 : s / (C::KB / GS);
      if (s == 0 || (GS > 1 && s % (C::KB / GS) == 0)) {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const int c = ccol0 + 16 * nt;
          const uint32_t zw = zw_l[gi * (C::BN / 8) + c / 8];
          zc[nt] = zero_const((zw >> (4 * (c % 8))) & 0xFu);
          s2[nt] = splat_h2(sc_l[gi * C::BN + c]);
        }
      }
      h8 af[MTW];
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt)
        af[mt] = *reinterpret_cast<const h8*>(st + swz<C::CPR>((uint32_t)(arow0 + 16 * mt), (uint32_t)(4 * s + h)));
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const h8 bw = decode_weight_vk(cb[nt][s], zc[nt], s2[nt], kc);
#pragma unroll
        for (int mt = 0; mt < MTW; ++mt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt], bw, acc[mt][nt], 0, 0, 0);
      }
    }
    if (more) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) cb[nt] = rb[nt];
    }
  }

  // Lane l, register r of tile (mt, nt): row 4(l/16) + r, column l%16.
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int col = n0 + ccol0 + 16 * nt;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 16 * (MTW * wm + mt) + 4 * h + r;
        const float v = acc[mt][nt][r];
        if (row < M && col < N) y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)v);
      }
    }
}

namespace {

template <int WM, int WN, int MTW, int NTW, int KS, int GS>
hipError_t launch_prefill_t(const LinearArgs& a, const Launch& L) {
  using C = PrefillCfg<WM, WN, MTW, NTW, KS, GS>;
  const int NT = (a.N + 15) / 16;
  const int KT = (a.K + 127) / 128;
  const int n_mtiles = (a.M + C::BM - 1) / C::BM;
  const int n_ntiles = (a.N + C::BN - 1) / C::BN;
  auto k = prefill_kernel<WM, WN, MTW, NTW, KS, GS>;
  if (C::LDS_BYTES > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                                       C::LDS_BYTES);
    if (e != hipSuccess) return e;
  }
  const uint32_t qw_bytes = (uint32_t)((size_t)NT * KT * 1024);
  return launch_kernel(k, dim3((unsigned)(n_mtiles * n_ntiles)), dim3(C::NTH), C::LDS_BYTES, L, a.x, a.qw,
                       a.scales, a.zeros, a.y, a.M, a.K, a.N, a.G, NT, n_mtiles, qw_bytes);
}

// Groups per step: KS / G for G < KS, else 1 (G is then a multiple of KS).
template <int WM, int WN, int MTW, int NTW, int KS>
hipError_t launch_prefill_k(const LinearArgs& a, const Launch& L) {
  if (a.G < KS) {
    if (KS / a.G == 2) return launch_prefill_t<WM, WN, MTW, NTW, KS, 2>(a, L);
    if (KS == 128 && a.G == 32) return launch_prefill_t<WM, WN, MTW, NTW, KS, (KS == 128 ? 4 : 2)>(a, L);
    return hipErrorInvalidValue;
  }
  return launch_prefill_t<WM, WN, MTW, NTW, KS, 1>(a, L);
}

}  // namespace

int prefill_auto_tile(int M, int N) {
  // The 256 x 256 tile halves the activation and weight re-reads of the
  // 128 x 128 ones and does half the redundant decoding per MFMA, but holds a
  // CU with one workgroup: measured on the LLaMA-shaped layers it wins from
  // about 150 tiles up (160 tiles on 256 CUs already beat 640 small ones);
  // below that the 128 x 128 tile with 128-row steps is best.
  const long t3 = (long)((M + 255) / 256) * ((N + 255) / 256);
  return t3 >= 150 ? 3 : 2;
}

bool prefill_fits(int K, int N) { return (size_t)((N + 15) / 16) * ((K + 127) / 128) * 1024 < ((size_t)1 << 31); }

hipError_t launch_prefill(const LinearArgs& a, int tile, const Launch& L) {
  if (!prefill_fits(a.K, a.N)) return hipErrorInvalidValue;
  switch (tile) {
    case 1: return launch_prefill_k<2, 2, 4, 4, 64>(a, L);   // 128 x 128, 4 waves of 64 x 64, 64-row steps
    case 2: return launch_prefill_k<2, 2, 4, 4, 128>(a, L);  // 128 x 128, 4 waves of 64 x 64, 128-row steps
    case 3: return launch_prefill_k<2, 4, 8, 4, 128>(a, L);  // 256 x 256, 8 waves of 128 x 64
  }
  return hipErrorInvalidValue;
}

}  // namespace awq
