// Prefill path of the W4A16 linear layer (large M): an LDS-tiled
// dequantise-then-MFMA fp16 GEMM with fp32 accumulation.
//
// At prefill sizes (hundreds to thousands of activation rows, as in the
// context stage of "TinyChat: Efficient and Lightweight Chatbot with AWQ",
// section "New Optimization of Context Stage") every weight is reused by many
// rows, so the layer is a dense contraction bound by the matrix cores. Each
// packed weight is decoded to its exact fp16 value (q - z) * s once per
// workgroup tile and fed to v_mfma_f32_16x16x32_f16.
//
// Workgroup tile 128 x 128 outputs, four waves of 64 x 64; K advances one
// 128-row tile of the device layout at a time. The activation tile is staged
// in LDS (rows padded by 16 bytes so the 16-byte fragment reads of 16
// consecutive rows fall on distinct banks); each wave streams the packed
// weight tiles of its 64 columns straight into registers -- one 16-byte load
// per lane per 16-column tile is already the MFMA B-operand layout -- and
// decodes them there.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

namespace prefill {
constexpr int BM = 128;
constexpr int BN = 128;
constexpr int LDA = 128 + 8;  // halfs per LDS row (16 bytes of padding)
}  // namespace prefill

template <int GPT>
__global__ __launch_bounds__(256) void prefill_kernel(const uint16_t* __restrict__ x, const u4* __restrict__ qw,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint32_t* __restrict__ zeros,
                                                      uint16_t* __restrict__ y, int M, int K, int N, int G, int KT,
                                                      int NT, int n_mtiles) {
  using namespace prefill;
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA];

  const int u = xcd_remap(blockIdx.x, gridDim.x);
  // Work ids run along M first so that consecutive workgroups (same XCD)
  // share the same weight columns.
  const int mtile = u % n_mtiles;
  const int ntile = u / n_mtiles;
  const int m0 = mtile * BM;
  const int n0 = ntile * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int h = lane >> 4;
  const int groups = K / G;
  constexpr int JPG = 4 / GPT;

  f4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f4{0.f, 0.f, 0.f, 0.f};

  for (int kt = 0; kt < KT; ++kt) {
    __syncthreads();
    // Stage x[m0 .. m0+127][128kt .. +127] into LDS: 16 lanes per row.
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = p * 16 + (tid >> 4);
      const int seg = tid & 15;
      const int row = m0 + r;
      const int k = 128 * kt + 8 * seg;
      u4 v = {0u, 0u, 0u, 0u};
      if (row < M && k < K) v = *reinterpret_cast<const u4*>(x + (int64_t)row * K + k);
      *reinterpret_cast<u4*>(&As[r * LDA + 8 * seg]) = v;
    }
    // Packed weights, scales and zero points of this wave's four column tiles.
    u4 wq[4];
    uint32_t sb[4][GPT], zb[4][GPT];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int t = n0 / 16 + 4 * wn + nt;
      const int col = 16 * t + (lane & 15);
      u4 v = {0u, 0u, 0u, 0u};
      if (t < NT) v = qw[((int64_t)kt * NT + t) * 64 + lane];
      wq[nt] = v;
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        const int g = (GPT == 1) ? (128 * kt) / G : kt * GPT + gi;
        const bool ok = col < N && (GPT == 1 || g < groups);
        sb[nt][gi] = ok ? (uint32_t)scales[(int64_t)g * N + col] : 0u;
        zb[nt][gi] = ok ? zeros[(int64_t)g * (N / 8) + (col >> 3)] : 0u;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h8 af[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int r = 64 * wm + 16 * mt + (lane & 15);
        af[mt] = *reinterpret_cast<const h8*>(&As[r * LDA + 32 * j + 8 * h]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int gi = j / JPG;
        const int col = n0 + 64 * wn + 16 * nt + (lane & 15);
        const ZeroConst zc = zero_const(zero_nibble(zb[nt][gi], col));
        const h8 bw = decode_weight(wq[nt][j], zc, splat_h2((uint16_t)sb[nt][gi]));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[mt], bw, acc[mt][nt], 0, 0, 0);
      }
    }
  }

  // Lane l, register r of tile (mt, nt): row 4(l/16) + r, column l%16.
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + 64 * wm + 16 * mt + 4 * h + r;
        const int col = n0 + 64 * wn + 16 * nt + (lane & 15);
        if (row < M && col < N) y[(int64_t)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)acc[mt][nt][r]);
      }
}

hipError_t launch_prefill(const LinearArgs& a, const Launch& L) {
  using namespace prefill;
  const int KT = (a.K + 127) / 128;
  const int NT = (a.N + 15) / 16;
  const int n_mtiles = (a.M + BM - 1) / BM;
  const int n_ntiles = (a.N + BN - 1) / BN;
  const dim3 grid((unsigned)(n_mtiles * n_ntiles));
  const u4* qw = reinterpret_cast<const u4*>(a.qw);
  if (a.G == 32)
    return launch_kernel(prefill_kernel<4>, grid, dim3(256), 0, L, a.x, qw, a.scales, a.zeros, a.y, a.M, a.K, a.N, a.G,
                         KT, NT, n_mtiles);
  if (a.G == 64)
    return launch_kernel(prefill_kernel<2>, grid, dim3(256), 0, L, a.x, qw, a.scales, a.zeros, a.y, a.M, a.K, a.N, a.G,
                         KT, NT, n_mtiles);
  return launch_kernel(prefill_kernel<1>, grid, dim3(256), 0, L, a.x, qw, a.scales, a.zeros, a.y, a.M, a.K, a.N, a.G, KT,
                       NT, n_mtiles);
}

}  // namespace awq
