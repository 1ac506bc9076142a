// Packing, unpacking and dequantisation kernels (gfx950).
//
// The 4-bit weights, their per-group fp16 scales and 4-bit zero points follow
// "TinyChat: Efficient and Lightweight Chatbot with AWQ", section "Usage",
// step 3 (--w_bit 4 --q_group_size 128, --q_backend real). The device tile
// layout is this library's own (see include/awq.h).
//
// Thread mapping for the tile layout: thread -> (n, h, j, kt) with the column
// n fastest, so the 64 lanes of a wave read or write 64 consecutive bytes of
// one row of the [K, N] code matrix; h = (lane group within the tile) and
// j = (word slot) select the 8-row block k0 = 128kt + 32j + 8h.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

__device__ __forceinline__ int nibble_pos(int e) { return 4 * (e & 1) + (e >> 1); }

struct TileCoord {
  int64_t word;  // index of the device word
  int n;         // column
  int k0;        // first of the 8 rows
};

__device__ __forceinline__ TileCoord tile_coord(int64_t tid, int Npad, int KT) {
  TileCoord c;
  const int n = (int)(tid % Npad);
  int64_t r = tid / Npad;
  const int h = (int)(r % 4);
  r /= 4;
  const int j = (int)(r % 4);
  const int kt = (int)(r / 4);
  c.n = n;
  c.k0 = 128 * kt + 32 * j + 8 * h;
  c.word = ((int64_t)kt * (Npad / 16) + n / 16) * 256 + 4 * (16 * h + (n % 16)) + j;
  return c;
}

__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ q, uint32_t* __restrict__ out,
                                                   int K, int N, int Npad, int KT, int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const TileCoord c = tile_coord(tid, Npad, KT);
  uint32_t word = 0;
  if (c.n < N) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int k = c.k0 + e;
      if (k < K) word |= (uint32_t)(q[(int64_t)k * N + c.n] & 0xF) << (4 * nibble_pos(e));
    }
  }
  out[c.word] = word;
}

__global__ __launch_bounds__(256) void unpack_kernel(const uint32_t* __restrict__ in, uint8_t* __restrict__ q,
                                                     int K, int N, int Npad, int KT, int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const TileCoord c = tile_coord(tid, Npad, KT);
  if (c.n >= N) return;
  const uint32_t word = in[c.word];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = c.k0 + e;
    if (k < K) q[(int64_t)k * N + c.n] = (uint8_t)((word >> (4 * nibble_pos(e))) & 0xF);
  }
}

__global__ __launch_bounds__(256) void pack_zeros_kernel(const uint8_t* __restrict__ z, uint32_t* __restrict__ out,
                                                         int N, int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const int N8 = N / 8;
  const int64_t g = tid / N8;
  const int c = (int)(tid % N8);
  const uint8_t* src = z + g * N + 8 * c;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= (uint32_t)(src[i] & 0xF) << (4 * i);
  out[tid] = word;
}

__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ qw,
                                                      const uint16_t* __restrict__ scales,
                                                      const uint32_t* __restrict__ zeros,
                                                      uint16_t* __restrict__ w, int K, int N, int Npad,
                                                      int KT, int G, int64_t total) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= total) return;
  const TileCoord c = tile_coord(tid, Npad, KT);
  if (c.n >= N || c.k0 >= K) return;
  const int g = c.k0 / G;
  const uint16_t sbits = scales[(int64_t)g * N + c.n];
  const uint32_t z = zero_nibble(zeros[(int64_t)g * (N / 8) + c.n / 8], c.n);
  // Rows (k0+2i, k0+2i+1) are the low and high halves of word i of the
  // result. (Vector elements are read through a whole-vector bit cast: a bit
  // cast of a single element of an fp16 vector is not reliable here.)
  const u4 v = __builtin_bit_cast(u4, decode_weight(qw[c.word], zero_const(z), splat_h2(sbits)));
  // K % 32 == 0 and k0 % 8 == 0, so rows k0 .. k0+7 are all < K here.
  uint16_t* dst = w + (int64_t)c.k0 * N + c.n;
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[(int64_t)e * N] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint16_t* __restrict__ y, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) y[i] = 0;
}

static inline unsigned grid_for(int64_t total) { return (unsigned)((total + 255) / 256); }

hipError_t launch_pack(const uint8_t* q, int K, int N, uint32_t* out, hipStream_t st) {
  const int KT = (K + 127) / 128, Npad = (N + 15) / 16 * 16;
  const int64_t total = (int64_t)Npad * KT * 16;
  hipLaunchKernelGGL(pack_kernel, dim3(grid_for(total)), dim3(256), 0, st, q, out, K, N, Npad, KT, total);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* in, int K, int N, uint8_t* q, hipStream_t st) {
  const int KT = (K + 127) / 128, Npad = (N + 15) / 16 * 16;
  const int64_t total = (int64_t)Npad * KT * 16;
  hipLaunchKernelGGL(unpack_kernel, dim3(grid_for(total)), dim3(256), 0, st, in, q, K, N, Npad, KT, total);
  return hipGetLastError();
}

hipError_t launch_pack_zeros(const uint8_t* z, int groups, int N, uint32_t* out, hipStream_t st) {
  const int64_t total = (int64_t)groups * (N / 8);
  hipLaunchKernelGGL(pack_zeros_kernel, dim3(grid_for(total)), dim3(256), 0, st, z, out, N, total);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint32_t* qw, const uint16_t* scales, const uint32_t* zeros, int K, int N,
                          int G, uint16_t* w, hipStream_t st) {
  const int KT = (K + 127) / 128, Npad = (N + 15) / 16 * 16;
  const int64_t total = (int64_t)Npad * KT * 16;
  hipLaunchKernelGGL(dequant_kernel, dim3(grid_for(total)), dim3(256), 0, st, qw, scales, zeros, w, K, N, Npad,
                     KT, G, total);
  return hipGetLastError();
}

hipError_t launch_fill_zero(uint16_t* y, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n)), dim3(256), 0, st, y, n);
  return hipGetLastError();
}

}  // namespace awq
