// Round-to-nearest group quantiser (gfx950): fp16 W [K, N] -> the device
// qweight layout, fp16 scales [K/G, N] and packed zero points [K/G, N/8].
//
// The step that produces the "real" INT4 weights the W4A16 layer consumes
// ("TinyChat: Efficient and Lightweight Chatbot with AWQ", section "Usage",
// step 3: --w_bit 4 --q_group_size 128, --q_backend real); the Sagemaker
// page names the plain variant, round-to-nearest, in its section on GGUF.
// Per group of G input channels and output column (asymmetric min-max):
//     lo, hi = min, max of the group;  s = fp16((hi - lo) / 15), 1 if that is 0
//     z = clamp(rne(-lo / s), 0, 15);  q = clamp(rne(w / s) + z, 0, 15)
// with every step one IEEE float32 operation (rne: round half to even).
//
// Groups of 32, 64 or 128 rows (band kernel): one workgroup per 128-row band
// and 128 columns (eight device tiles). Each lane loads an 8 x 8 block (8 rows
// of 8 columns, one 16-byte load per row) and keeps it in registers; the
// block's per-column min and max are combined through LDS per group, each
// (group, column) gets its scale and zero point, and every lane turns its
// block into eight device words, which go through LDS so that the tiles are
// written with whole 16-byte stores (padding rows and columns included).
// Larger groups (multiples of 128 rows; generic kernel): one workgroup per
// (group, 64 columns), min and max reduced over the whole group, then the
// block is read again (from L2) and written word by word.
//
// The quotient w / s is formed as w * (1/s) and rounded; only when that
// product lies within 2^-16 of a half-integer (where the two could round
// differently) is the exact quotient needed. The test is made once per device
// word (eight rows of one column): if any of its eight products is that
// close, the whole word is recomputed from exact quotients, so the codes
// equal those of the plain division for every input and the common path has
// no branch per weight.
#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

constexpr int kQuantCols = 64;

// The device word of eight consecutive rows of one column: codes
// clamp(rne(w / s) + z, 0, 15), row e in nibble 4(e % 2) + e / 2. The
// quotients come from w * (1/s), which differs from w / s by a few units in
// the last place, so the two can round differently only when the product
// lies next to a half-integer; if any of the eight does, all eight are taken
// from the exact quotient (one branch per word, rarely taken).
__device__ __forceinline__ uint32_t rtn_word(const float (&f)[8], float s, float inv, float zf) {
  float r[8], d = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float t = f[e] * inv;
    r[e] = rintf(t);
    d = fmaxf(d, fabsf(t - r[e]));
  }
  if (d > 0.5f - 1.52587890625e-05f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = rintf(f[e] / s);
  }
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float q = fminf(fmaxf(r[e] + zf, 0.f), 15.f);
    word |= (uint32_t)q << (4 * (4 * (e & 1) + (e >> 1)));
  }
  return word;
}

// Scale (as float), its reciprocal and the zero point of one (group, column)
// from the group's min and max; `bits` receives the fp16 scale.
__device__ __forceinline__ void rtn_params(float lo, float hi, float& sf, float& inv, float& zf, uint16_t& bits) {
  _Float16 s16 = (_Float16)((hi - lo) / 15.0f);
  if (s16 == (_Float16)0.0f) s16 = (_Float16)1.0f;
  sf = (float)s16;
  inv = 1.0f / sf;
  zf = fminf(fmaxf(rintf(-lo / sf), 0.f), 15.f);
  bits = __builtin_bit_cast(uint16_t, s16);
}

__device__ __forceinline__ float half_at(const u4& v, int i) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v[i >> 1] >> (16 * (i & 1))));
}

// Band kernel (G = 32, 64 or 128): workgroup = 128-row band kt x 128 columns;
// lane (co, ro) = (tid % 16, tid / 16) holds rows 8ro .. 8ro+7 and columns
// 8co .. 8co+7 of that block.
template <int G>
__global__ __launch_bounds__(256) void quantize_band_kernel(const uint16_t* __restrict__ w, int K, int N, int NT,
                                                            int col_blocks, uint32_t* __restrict__ qw,
                                                            uint16_t* __restrict__ scales,
                                                            uint32_t* __restrict__ zeros) {
  constexpr int GB = 128 / G;  // groups per band
  constexpr int OPG = G / 8;   // row octets per group
  __shared__ float red_lo[16][128];
  __shared__ float red_hi[16][128];
  __shared__ float p_s[GB][128], p_inv[GB][128], p_z[GB][128];
  __shared__ uint32_t tiles[8][256];
  const int kt = blockIdx.x / col_blocks;
  const int bx = blockIdx.x % col_blocks;
  const int c0 = bx * 128;
  const int tid = threadIdx.x;
  const int co = tid & 15, ro = tid >> 4;
  const int k0 = kt * 128 + 8 * ro;
  const int n0 = c0 + 8 * co;
  const bool ok = k0 < K && n0 < N;

  u4 v[8];
  float lo[8], hi[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) lo[i] = INFINITY, hi[i] = -INFINITY;
  if (ok) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = *reinterpret_cast<const u4*>(w + (int64_t)(k0 + e) * N + n0);
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float f = half_at(v[e], i);
        lo[i] = fminf(lo[i], f);
        hi[i] = fmaxf(hi[i], f);
      }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red_lo[ro][8 * co + i] = lo[i], red_hi[ro][8 * co + i] = hi[i];
  __syncthreads();

  // one (group, column) pair per thread and turn
  for (int pidx = tid; pidx < GB * 128; pidx += 256) {
    const int gi = pidx / 128, c = pidx % 128;
    float l = INFINITY, h = -INFINITY;
#pragma unroll
    for (int o = 0; o < OPG; ++o) l = fminf(l, red_lo[gi * OPG + o][c]), h = fmaxf(h, red_hi[gi * OPG + o][c]);
    float sf, inv, zf;
    uint16_t bits;
    rtn_params(l, h, sf, inv, zf, bits);
    p_s[gi][c] = sf, p_inv[gi][c] = inv, p_z[gi][c] = zf;
    const int g = (kt * 128) / G + gi;
    const int n = c0 + c;
    if (g * G < K && n < N) scales[(int64_t)g * N + n] = bits;
  }
  __syncthreads();
  if (tid < GB * 16) {
    const int gi = tid / 16, oc = tid % 16;
    const int g = (kt * 128) / G + gi;
    const int n = c0 + 8 * oc;
    if (g * G < K && n < N) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= (uint32_t)p_z[gi][8 * oc + i] << (4 * i);
      zeros[(int64_t)g * (N / 8) + n / 8] = word;
    }
  }

  // codes: lane's rows 8ro.. of column 8co+i form device word (lane 16h + cc, slot j)
  {
    const int gi = (8 * ro) / G;
    const int tt = co >> 1, j = ro >> 2, h = ro & 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = 8 * co + i;
      uint32_t word = 0;
      if (ok) {
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = half_at(v[e], i);
        word = rtn_word(f, p_s[gi][c], p_inv[gi][c], p_z[gi][c]);
      }
      const int cc = 8 * (co & 1) + i;
      tiles[tt][4 * (16 * h + cc) + j] = word;
    }
  }
  __syncthreads();
  // whole tiles out: 8 x 1 KiB, 16 bytes per lane and turn
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int u = tid + 256 * r;
    const int tt = u >> 6, lane = u & 63;
    const int t = bx * 8 + tt;
    if (t < NT) {
      const u4 val = *reinterpret_cast<const u4*>(&tiles[tt][4 * lane]);
      *reinterpret_cast<u4*>(qw + ((int64_t)kt * NT + t) * 256 + 4 * lane) = val;
    }
  }
}

// Generic kernel (G a multiple of 128).
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ w, int K, int N, int G, int NT,
                                                       int col_blocks, uint32_t* __restrict__ qw,
                                                       uint16_t* __restrict__ scales, uint32_t* __restrict__ zeros) {
  __shared__ float red_lo[32][kQuantCols + 1];
  __shared__ float red_hi[32][kQuantCols + 1];
  __shared__ float col_s[kQuantCols], col_inv[kQuantCols], col_z[kQuantCols];
  const int g = blockIdx.x / col_blocks;
  const int n0 = (blockIdx.x % col_blocks) * kQuantCols;
  const int tid = threadIdx.x;

  // Pass 1: per-column min and max over the group's G rows.
  {
    const int co = tid & 7;  // 8-column octet
    const int r0 = tid >> 3;  // 0..31
    const int n = n0 + 8 * co;
    float lo[8], hi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) lo[i] = INFINITY, hi[i] = -INFINITY;
    if (n < N) {
      for (int r = r0; r < G; r += 32) {
        const u4 v = *reinterpret_cast<const u4*>(w + ((int64_t)g * G + r) * N + n);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float f = half_at(v, i);
          lo[i] = fminf(lo[i], f);
          hi[i] = fmaxf(hi[i], f);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      red_lo[r0][8 * co + i] = lo[i];
      red_hi[r0][8 * co + i] = hi[i];
    }
  }
  __syncthreads();

  // Pass 2: scale and zero point per column.
  if (tid < kQuantCols) {
    float lo = red_lo[0][tid], hi = red_hi[0][tid];
    for (int r = 1; r < 32; ++r) {
      lo = fminf(lo, red_lo[r][tid]);
      hi = fmaxf(hi, red_hi[r][tid]);
    }
    const int n = n0 + tid;
    float sf, inv, zf;
    uint16_t bits;
    rtn_params(lo, hi, sf, inv, zf, bits);
    col_s[tid] = sf;
    col_inv[tid] = inv;
    col_z[tid] = zf;
    if (n < N) scales[(int64_t)g * N + n] = bits;
  }
  __syncthreads();
  if (tid < kQuantCols / 8) {
    const int n = n0 + 8 * tid;
    if (n < N) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) word |= (uint32_t)col_z[8 * tid + i] << (4 * i);
      zeros[(int64_t)g * (N / 8) + n / 8] = word;
    }
  }

  // Pass 3: codes, one device word (8 rows of one column) per thread and turn.
  const int words = (G / 8) * kQuantCols;
  for (int u = tid; u < words; u += 256) {
    const int c = u % kQuantCols;
    const int n = n0 + c;
    if (n >= N) continue;
    const int k0 = g * G + 8 * (u / kQuantCols);
    const uint16_t* src = w + (int64_t)k0 * N + n;
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (float)__builtin_bit_cast(_Float16, src[(int64_t)e * N]);
    const uint32_t word = rtn_word(f, col_s[c], col_inv[c], col_z[c]);
    const int kt = k0 / 128, j = (k0 % 128) / 32, h = (k0 % 32) / 8;
    qw[((int64_t)kt * NT + n / 16) * 256 + 4 * (16 * h + (n % 16)) + j] = word;
  }
}

hipError_t launch_quantize(const uint16_t* w, int K, int N, int G, uint32_t* qw, uint16_t* scales, uint32_t* zeros,
                           hipStream_t st) {
  const int NT = (N + 15) / 16, KT = (K + 127) / 128;
  if (G <= 128) {
    const int cb = (N + 127) / 128;
    const dim3 grid((unsigned)((int64_t)cb * KT));
    if (G == 32)
      hipLaunchKernelGGL(quantize_band_kernel<32>, grid, dim3(256), 0, st, w, K, N, NT, cb, qw, scales, zeros);
    else if (G == 64)
      hipLaunchKernelGGL(quantize_band_kernel<64>, grid, dim3(256), 0, st, w, K, N, NT, cb, qw, scales, zeros);
    else if (G == 128)
      hipLaunchKernelGGL(quantize_band_kernel<128>, grid, dim3(256), 0, st, w, K, N, NT, cb, qw, scales, zeros);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  // padding rows and columns of the device layout hold code 0
  if (K % 128 || N % 16) {
    hipError_t e = launch_fill_zero(reinterpret_cast<uint16_t*>(qw), (int64_t)NT * KT * 256 * 2, st);
    if (e != hipSuccess) return e;
  }
  const int col_blocks = (N + kQuantCols - 1) / kQuantCols;
  const int64_t grid = (int64_t)col_blocks * (K / G);
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)grid), dim3(256), 0, st, w, K, N, G, NT, col_blocks, qw,
                     scales, zeros);
  return hipGetLastError();
}

}  // namespace awq
