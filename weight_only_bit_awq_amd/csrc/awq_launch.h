// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

hipError_t launch_pack(const uint8_t* q, int K, int N, uint32_t* out, hipStream_t st);
hipError_t launch_unpack(const uint32_t* in, int K, int N, uint8_t* q, hipStream_t st);
hipError_t launch_pack_zeros(const uint8_t* z, int groups, int N, uint32_t* out, hipStream_t st);
hipError_t launch_dequant(const uint32_t* qw, const uint16_t* scales, const uint32_t* zeros, int K, int N,
                          int G, uint16_t* w, hipStream_t st);

hipError_t launch_fill_zero(uint16_t* y, int64_t n, hipStream_t st);

// Round-to-nearest group quantiser: fp16 w [K, N] -> device qweight, fp16
// scales [K/G, N], packed zeros [K/G, N/8].
hipError_t launch_quantize(const uint16_t* w, int K, int N, int G, uint32_t* qw, uint16_t* scales, uint32_t* zeros,
                           hipStream_t st);

struct LinearArgs {
  const uint16_t* x;
  const uint32_t* qw;
  const uint16_t* scales;
  const uint32_t* zeros;
  uint16_t* y;
  int M, K, N, G;
};

// Where and how a kernel is launched. With timing events set, the kernel is
// launched through hipExtLaunchKernelGGL, which records `start` and `stop` at
// the kernel's own start and end on `stream`.
struct Launch {
  hipStream_t stream;
  hipEvent_t start;
  hipEvent_t stop;
};

template <typename F, typename... Args>
hipError_t launch_kernel(F kernel, dim3 grid, dim3 block, size_t lds, const Launch& L, Args... args) {
  if (L.start || L.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, L.stream, L.start, L.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, L.stream, args...);
  return hipGetLastError();
}

// Decode path. Staged: activations and per-(group, column) scale/zero words
// are copied to LDS once per workgroup (M <= 16, fits kDecodeLdsBytes), each
// workgroup owns `tpw` 16-column tiles. Streamed: they are read per tile.
// Either way `waves` waves split the K range and are summed through LDS.
constexpr int64_t kDecodeLdsBytes = 160 * 1024;
struct DecodeConfig {
  int waves;
  int tpw;
  bool staged;
  bool gated;  // y[M, N/2] = silu(x W[:, :N/2]) * (x W[:, N/2:]); N % 32 == 0
  int splits;  // streamed: K split over workgroups (fp32 partials in ws, then the fixed-order reduction)
  float* ws;
  bool slab;   // not staged: activations staged per two-band slab in LDS, shared by four waves that
               // each own `tpw` column tiles (M <= 32, G a multiple of 128, waves = 4, tpw 2 or 4)
};
bool decode_staged_fits(int M, int K, int G, int waves, int tpw);
// Splits a streamed decode plan actually runs with (whole bands per split,
// every split non-empty).
int decode_splits(int K, int splits);
hipError_t launch_decode(const LinearArgs& a, const DecodeConfig& cfg, const Launch& L);

// Prefill path: dequantise-then-MFMA GEMM; `tile` selects the workgroup tile
// (1 = 128x128 with 64-row K steps, 2 = 128x128 with 128-row steps,
// 3 = 256x256 with 128-row steps). With splits > 1 the K steps are divided
// into that many contiguous ranges whose fp32 partials go to `ws`
// (prefill_workspace_bytes) and are summed by a second kernel.
int prefill_steps(int K, int tile);
// Fills *tile and/or *splits where they are 0, from a cost model of the
// fp16 GEMM (kFp16) or of the W4A8 GEMM (kW4A8), whose K steps are shorter
// and, unlike the fp16 GEMM's, no faster when part of the chip is idle.
enum class PrefillKind { kFp16, kW4A8 };
void prefill_auto_plan(int M, int K, int N, int* tile, int* splits, PrefillKind kind = PrefillKind::kFp16);
// Gated (y[M, N/2] = silu(gate) * up): the partials always go through the
// workspace and the reduction applies the epilogue.
size_t prefill_workspace_bytes(int M, int N, int splits, bool gated);
bool prefill_fits(int K, int N);

// Library-owned device memory for the split-K partials of callers that
// cannot allocate: kNoAllocScratchBytes per device, shared by every such call
// on that device. noalloc_scratch gives its address on the current device
// (looked up once per device; allocates nothing).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
constexpr int kNoAllocMaxDevices = 64;
hipError_t noalloc_scratch(float** ptr);
hipError_t launch_prefill(const LinearArgs& a, int tile, int splits, float* ws, bool gated, const Launch& L);

// Sum of `splits` fp32 partials ws[s][M][N] in increasing s, rounded to
// fp16 into y [M, N]; gated: y [M, N/2] = silu(sum of the gate half) * (sum
// of the up half).
hipError_t launch_prefill_reduce(float* ws, uint16_t* y, int M, int N, int splits, bool gated, const Launch& L);

// W4A8-FP8: per-token FP8 (E4M3) activation quantiser, and the layer on the
// FP8 matrix cores (G a multiple of 128). The workspace holds the FP8
// activations [M, K] (128-column blocks with permuted 8-column chunks), the
// token scales and, with splits > 1, the fp32 partials.
hipError_t launch_act_quant_fp8(const uint16_t* x, int M, int K, uint8_t* x8, float* sx, const Launch& L);
size_t w4a8_workspace_bytes(int M, int K, int N, int splits);
hipError_t launch_w4a8(const LinearArgs& a, int tile, int splits, void* ws, const Launch& L);

// Fused decode-step attention (rotary embedding, MHA/GQA/MQA, key-value
// cache append). Caches: keys [B, Hkv, S, D], values [B, Hkv, S/32, D, 32]
// (tiles of 32 positions, d-major inside a tile).
struct AttnParams {
  const uint16_t* qkv;
  int64_t qkv_stride;
  uint16_t* kc;
  uint16_t* vc;
  const int32_t* lengths;
  uint16_t* out;
  float* part;         // partial softmax states (workspace)
  uint32_t* counters;  // one per unit, zero between calls (workspace)
  int64_t units;       // B * Hkv * T
  int Hq, Hkv, S, max_cached, g, T, C, steps, style;
  float scale_log2;    // softmax scale * log2(e)
  double log2_theta;
};
// Work split: g query heads per kv head, T tiles of 16 of them, C workgroups
// per unit, `steps` 32-position blocks per wave (0: chosen here); workspace
// sizes.
struct AttnPlan {
  int g, T, C, steps;
  int64_t units;
  size_t counter_bytes, ws_bytes;
};
AttnPlan attention_plan(int B, int Hq, int Hkv, int D, int max_cached, int steps);
hipError_t launch_attention(const AttnParams& p, int D, const Launch& L);

// Plain streaming read of `bytes` (a multiple of 16) at `buf`; the 16 bytes at
// `sink` may receive a value derived from the data.
hipError_t launch_stream_read(const void* buf, uint64_t bytes, void* sink, const Launch& L);

}  // namespace awq
