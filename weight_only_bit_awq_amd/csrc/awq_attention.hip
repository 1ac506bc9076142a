// Fused decode-step attention: rotary position embedding, MHA / GQA / MQA
// scaled dot-product attention over a pre-allocated fp16 key-value cache, and
// the append of the new token's key and value, in one kernel launch.
//
// "TinyChat: Efficient and Lightweight Chatbot with AWQ", section "Speed
// Benchmarks": in the generation stage all operations of MHA/GQA/MQA run in
// a single kernel with the positional embedding fused into it, and the
// key-value caches are allocated up front. Per generated token the step reads
// every cached key and value once, so it is bound by HBM bandwidth.
//
// Design
//   * Work unit = (sequence b, key/value head, tile of 16 query heads of that
//     head's group). A workgroup of four waves takes one contiguous range of
//     cached positions of one unit; each wave streams `steps` blocks of 32
//     positions of its own sub-range with online softmax; the waves' states
//     (running max, sum, unnormalised output) are merged through LDS and the
//     workgroup's state goes to the workspace.
//   * Scores on the matrix cores: v_mfma_f32_16x16x32_f16 with the keys as the
//     A operand (lane l loads 16 bytes of key row k(l%16) at d = 8(l/16) of
//     each 32-wide d block) and the rotated queries as B. The key rows of a
//     32-position block are ordered so that the score tile a lane receives
//     (head l%16, four positions) is exactly the B operand of
//     v_mfma_f32_16x16x32_f16 for the value product once the two blocks of a
//     32-position step are side by side, and the values it needs (eight
//     consecutive positions of one d row) are one 16-byte load from the value
//     cache, kept in tiles of 32 positions (d-major inside a tile) so that
//     each load instruction reads one contiguous KiB. No cross-lane moves
//     besides two max reductions per step.
//   * The rotation angles are computed once per workgroup in fp64 (rate
//     theta^(-2i/D) times the position), kept as fp32 cos/sin in LDS.
//   * The last workgroup of a unit to finish (an agent-scope counter in the
//     workspace) merges the states in a fixed order, all its threads loading
//     several states at once (one round trip to memory for up to
//     8 x 16 / heads-per-tile workgroups), adds the new token (its rotated
//     key rounded to fp16, as it is stored, and its value), writes the fp16
//     output and, for the unit's first tile, appends the key and value to
//     the caches. It then
//     returns the counter and the states it read to zero, so that the
//     workspace is all zero between calls whatever their shapes.
//   * Positions at or beyond a sequence's length are masked: their scores are
//     replaced by -inf and their values by zero before the value product, so
//     stale cache contents (even NaN patterns) never reach the output.
#include <math.h>

#include <algorithm>

#include "awq_device.h"
#include "awq_launch.h"

namespace awq {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kAttnWaves = 4;
constexpr int kAttnBlock = 32;    // positions per wave step
constexpr float kNoMax = -3.0e38f;  // running max before any position

// Workgroup states travel between XCDs, whose L2 caches are not coherent
// with each other. They are written and read with agent-scope relaxed atomic
// accesses, which the hardware performs coherently without flushing or
// invalidating the L2 (a fence at agent scope would do both, for the whole
// cache, in every workgroup). Ordering: every wave waits until its state
// stores are acknowledged (s_waitcnt on all counters), then the workgroup
// barrier, then thread 0 increments the unit's counter; the last workgroup
// reads the states only after its own increment has returned.
__device__ __forceinline__ void coherent_store2(float* p, float a, float b) {
  const uint64_t v = (uint64_t)__builtin_bit_cast(uint32_t, a) | ((uint64_t)__builtin_bit_cast(uint32_t, b) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_load2(const float* p, float& a, float& b) {
  const uint64_t v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  a = __builtin_bit_cast(float, (uint32_t)v);
  b = __builtin_bit_cast(float, (uint32_t)(v >> 32));
}

__device__ __forceinline__ float xor_max(float v, int m) { return fmaxf(v, __shfl_xor(v, m)); }
__device__ __forceinline__ float xor_sum(float v, int m) { return v + __shfl_xor(v, m); }

template <int N>
using hvec_t = _Float16 __attribute__((ext_vector_type(N)));

// The inputs of a rotation of elements d0 .. d0+DP-1 of one head vector (fp16
// bits, D elements): the elements and their partners d0 +- D/2 (the pairs of
// style 1; styles 2 and 0 use `a` only). Loaded ahead of the angle table so
// that the load latency overlaps other work. DP divides D/2, d0 % DP == 0.
template <int DP>
struct RopeSrc {
  hvec_t<DP> a, b;
};

template <int D, int DP>
__device__ __forceinline__ RopeSrc<DP> rope_load(const uint16_t* v, int d0) {
  RopeSrc<DP> s;
  s.a = *reinterpret_cast<const hvec_t<DP>*>(v + d0);
  s.b = *reinterpret_cast<const hvec_t<DP>*>(v + (d0 < D / 2 ? d0 + D / 2 : d0 - D / 2));
  return s;
}

// Rotated values y[0..DP). Pairs: (i, i + D/2) for style 1, (2i, 2i+1) for
// style 2; style 0 copies.
template <int D, int DP>
__device__ __forceinline__ void rope_apply(const RopeSrc<DP>& s, int d0, int style, const float (*cs)[2], float* y) {
  if (style == 1) {
    const bool lo = d0 < D / 2;
    const int i0 = lo ? d0 : d0 - D / 2;
#pragma unroll
    for (int i = 0; i < DP; ++i) {
      const float a = (float)s.a[i], b = (float)s.b[i];
      const float c = cs[i0 + i][0], sn = cs[i0 + i][1];
      y[i] = lo ? a * c - b * sn : b * sn + a * c;
    }
  } else if (style == 2) {
#pragma unroll
    for (int i = 0; i < DP; i += 2) {
      const int pi = (d0 + i) >> 1;
      const float c = cs[pi][0], sn = cs[pi][1];
      const float a = (float)s.a[i], b = (float)s.a[i + 1];
      y[i] = a * c - b * sn;
      y[i + 1] = a * sn + b * c;
    }
  } else {
#pragma unroll
    for (int i = 0; i < DP; ++i) y[i] = (float)s.a[i];
  }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kAttnWaves * 64) void attn_decode_kernel(AttnParams p) {
  constexpr int NC = D / 32;  // 32-wide d blocks of the score product
  constexpr int NE = D / 16;  // 16-row d tiles of the value product
  constexpr int DP = D / 16;  // d values per thread when states are merged
  constexpr int HS = D + 4;   // floats per head of a state: o[D], max, sum, pad
  __shared__ float cs[D / 2][2];
  __shared__ float red[kAttnWaves][16][HS];  // the waves' states, then the merge groups'
  __shared__ int s_last;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r16 = l & 15, g4 = l >> 4;
  const int unit = blockIdx.x / p.C, chunk = blockIdx.x % p.C;
  const int tile = unit % p.T, bk = unit / p.T;  // bk = b * Hkv + kv head
  const int b = bk / p.Hkv, kvh = bk % p.Hkv;
  const int L = p.lengths[b];
  const bool valid = L >= 0 && L < p.S && L <= p.max_cached;
  const int span = p.steps * kAttnBlock;
  const int first = (chunk * kAttnWaves + w) * span;
  const int kend = valid ? min(L, first + span) : 0;  // this wave's cached positions: [first, kend)
  const bool wg_keys = valid && chunk * kAttnWaves * span < L;
  const int hv = min(16, p.g - 16 * tile);  // real query heads in this tile

  // Keys [S, D] per (b, kv head); values in tiles of 32 positions, d-major
  // inside a tile: element (d, j) at ((j / 32) * D + d) * 32 + j % 32.
  const uint16_t* kbase = p.kc + (int64_t)bk * p.S * D;
  const uint16_t* vbase = p.vc + (int64_t)bk * p.S * D;
  // A-row r of key block blk (of a 32-position step at k0) is position
  // k0 + 8(r/4) + 4blk + r%4; lane l's values are d row 16e + l%16,
  // positions k0 + 8(l/16) .. +7 (one contiguous 1 KiB per load instruction).
  h8 kx[2][NC];
  h8 vx[NE];
  auto load_block = [&](int k0) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int pos = k0 + 8 * (r16 >> 2) + 4 * blk + (r16 & 3);
      const uint16_t* kr = kbase + (int64_t)pos * D + 8 * g4;
#pragma unroll
      for (int c = 0; c < NC; ++c) kx[blk][c] = *reinterpret_cast<const h8*>(kr + 32 * c);
    }
    const uint16_t* vt = vbase + (int64_t)(k0 / kAttnBlock) * D * kAttnBlock + 8 * g4;
#pragma unroll
    for (int e = 0; e < NE; ++e) vx[e] = *reinterpret_cast<const h8*>(vt + (16 * e + r16) * kAttnBlock);
  };
  // The first block and the raw queries are requested before the sequence
  // length arrives (any wave starting at or below max_cached may hold keys,
  // and its first block then lies inside the cache); unused if it holds none.
  const bool may_hold = first <= p.max_cached;
  if (may_hold) load_block(first);
  const uint16_t* row = p.qkv + (int64_t)b * p.qkv_stride;
  const int hl = 16 * tile + r16;
  RopeSrc<8> qsrc[NC];
  if (may_hold && hl < p.g) {
    const uint16_t* qh = row + (int64_t)(kvh * p.g + hl) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) qsrc[c] = rope_load<D, 8>(qh, 32 * c + 8 * g4);
  }

  if (tid < D / 2) {
    float c = 1.f, s = 0.f;
    if (p.style != 0 && valid) {
      const double ang = (double)L * exp2(-(2.0 * tid / D) * p.log2_theta);
      double sd, cd;
      sincos(ang, &sd, &cd);
      c = (float)cd;
      s = (float)sd;
    }
    cs[tid][0] = c;
    cs[tid][1] = s;
  }
  __syncthreads();

  f4 acc[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) acc[e] = f4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNoMax, l_run = 0.f;
  if (first < kend) {
    // Rotated queries of the tile as the B operand: lane l holds head l%16,
    // d = 32c + 8(l/16) .. +7 of each block c.
    h8 bq[NC];
    {
      float y[NC][8];
      if (hl < p.g) {
#pragma unroll
        for (int c = 0; c < NC; ++c) rope_apply<D, 8>(qsrc[c], 32 * c + 8 * g4, p.style, cs, y[c]);
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) y[c][e] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) bq[c][e] = (_Float16)y[c][e];
    }

    for (int k0 = first; k0 < kend; k0 += kAttnBlock) {
      // Scores: lane l gets head l%16, positions kb + 4blk + t (t = 0..3).
      const int kb = k0 + 8 * g4;
      float s[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        f4 sa = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) sa = __builtin_amdgcn_mfma_f32_16x16x32_f16(kx[blk][c], bq[c], sa, 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          s[blk][t] = (kb + 4 * blk + t < L) ? sa[t] * p.scale_log2 : -INFINITY;
          mx = fmaxf(mx, s[blk][t]);
        }
      }
      mx = xor_max(mx, 16);
      mx = xor_max(mx, 32);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      m_run = m_new;
      // Probabilities of positions kb .. kb+7: the B operand of the value
      // product (head l%16, eight consecutive positions per lane).
      float psum = 0.f;
      h8 pb;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float pv = exp2f(s[blk][t] - m_new);
          psum += pv;
          pb[4 * blk + t] = (_Float16)pv;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] *= alpha;
      if (k0 + kAttnBlock > L) {
#pragma unroll
        for (int e = 0; e < NE; ++e)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (kb + j >= L) vx[e][j] = (_Float16)0.f;
      }
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vx[e], pb, acc[e], 0, 0, 0);
      if (k0 + kAttnBlock < kend) load_block(k0 + kAttnBlock);
    }
    l_run = xor_sum(l_run, 16);
    l_run = xor_sum(l_run, 32);
  }

  // The four waves' states (head l%16; d = 16e + 4(l/16) .. +3) merged in
  // LDS into the workgroup's, which goes to its slot of the workspace.
  if (wg_keys) {
#pragma unroll
    for (int e = 0; e < NE; ++e) *reinterpret_cast<f4*>(&red[w][r16][16 * e + 4 * g4]) = acc[e];
    if (g4 == 0) {
      red[w][r16][D] = m_run;
      red[w][r16][D + 1] = l_run;
    }
  }
  __syncthreads();
  const int j = tid >> 4, d0 = (tid & 15) * DP;  // head j, d range [d0, d0 + DP)
  if (wg_keys && j < hv) {
    float M = kNoMax;
#pragma unroll
    for (int ww = 0; ww < kAttnWaves; ++ww) M = fmaxf(M, red[ww][j][D]);
    float lsum = 0.f, o[DP];
#pragma unroll
    for (int i = 0; i < DP; ++i) o[i] = 0.f;
#pragma unroll
    for (int ww = 0; ww < kAttnWaves; ++ww) {
      const float c = exp2f(red[ww][j][D] - M);
      lsum += red[ww][j][D + 1] * c;
#pragma unroll
      for (int i = 0; i < DP; ++i) o[i] += red[ww][j][d0 + i] * c;
    }
    float* ph = p.part + ((int64_t)unit * p.C + chunk) * 16 * HS + j * HS;
#pragma unroll
    for (int i = 0; i < DP; i += 2) coherent_store2(ph + d0 + i, o[i], o[i + 1]);
    if ((tid & 15) == 0) coherent_store2(ph + D, M, lsum);
  }

  // The new token's inputs for the merge (needed by the last workgroup only;
  // requested here so that their latency overlaps the counter step).
  const uint16_t* kh = row + (int64_t)(p.Hq + kvh) * D;
  const uint16_t* vh = row + (int64_t)(p.Hq + p.Hkv + kvh) * D;
  const bool head_ok = j < hv;
  const RopeSrc<DP> ksrc = rope_load<D, DP>(kh, d0);
  RopeSrc<DP> qnew;
  if (head_ok) qnew = rope_load<D, DP>(row + (int64_t)(kvh * p.g + 16 * tile + j) * D, d0);
  const hvec_t<DP> vnew = *reinterpret_cast<const hvec_t<DP>*>(vh + d0);

  // Count this workgroup once its state is stored (every wave waits for its
  // stores to be acknowledged, then the barrier); the last one merges.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(p.counters + unit, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (unsigned)(p.C - 1);
  __syncthreads();
  if (!s_last) return;

  // Merge: the workgroups' states of this unit are spread over SG groups of
  // threads (thread = group sg, head jj, d range), each group folds its slots
  // with independent loads, the groups' results meet in LDS.
  const int hvp = hv <= 1 ? 1 : hv <= 2 ? 2 : hv <= 4 ? 4 : hv <= 8 ? 8 : 16;
  const int jj = (tid >> 4) % hvp, sg = (tid >> 4) / hvp;
  const int nsl = valid ? min(p.C, (L + kAttnWaves * span - 1) / (kAttnWaves * span)) : 0;
  // Groups in use: about four slots each (a slot folded inside a thread is a
  // few arithmetic steps; a group folded at the end adds an LDS round trip
  // to the chain), at most 16 / hvp.
  const int SG = max(1, min(16 / hvp, (nsl + 3) / 4));
  {
    float M = kNoMax, lsum = 0.f, o[DP];
#pragma unroll
    for (int i = 0; i < DP; ++i) o[i] = 0.f;
    if (jj < hv && sg < SG) {
      const float* pu = p.part + (int64_t)unit * p.C * 16 * HS + jj * HS;
      for (int base = sg; base < nsl; base += 8 * SG) {
        float ms[8], ls[8], os[8][DP];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int sl = base + u * SG;
          if (sl < nsl) {
            const float* ph = pu + (int64_t)sl * 16 * HS;
            coherent_load2(ph + D, ms[u], ls[u]);
#pragma unroll
            for (int i = 0; i < DP; i += 2) coherent_load2(ph + d0 + i, os[u][i], os[u][i + 1]);
          } else {
            ms[u] = kNoMax;
            ls[u] = 0.f;
#pragma unroll
            for (int i = 0; i < DP; ++i) os[u][i] = 0.f;
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float m2 = fmaxf(M, ms[u]);
          const float a = exp2f(M - m2), c = exp2f(ms[u] - m2);
          lsum = lsum * a + ls[u] * c;
#pragma unroll
          for (int i = 0; i < DP; ++i) o[i] = o[i] * a + os[u][i] * c;
          M = m2;
        }
      }
    }
    __syncthreads();  // the workgroup's own state in `red` has been written out
    float* g = &red[0][0][0] + (sg * hvp + jj) * 16 * (DP + 2) + (tid & 15) * (DP + 2);
#pragma unroll
    for (int i = 0; i < DP; ++i) g[i] = o[i];
    g[DP] = M;
    g[DP + 1] = lsum;
  }
  __syncthreads();

  uint16_t* out = p.out + ((int64_t)b * p.Hq + kvh * p.g + 16 * tile + j) * D + d0;
  if (!valid) {
    if (j < hv)
#pragma unroll
      for (int i = 0; i < DP; ++i) out[i] = 0x7E00;  // fp16 quiet NaN
  } else {
    // New token: rotated q (fp32) and key (rounded to fp16, as stored).
    float kr[DP], qr[DP], o[DP];
    _Float16 k16[DP];
    rope_apply<D, DP>(ksrc, d0, p.style, cs, kr);
    if (head_ok) rope_apply<D, DP>(qnew, d0, p.style, cs, qr);
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < DP; ++i) {
      k16[i] = (_Float16)kr[i];
      dot += head_ok ? qr[i] * (float)k16[i] : 0.f;
      o[i] = (float)vnew[i];
    }
    dot = xor_sum(dot, 1);
    dot = xor_sum(dot, 2);
    dot = xor_sum(dot, 4);
    dot = xor_sum(dot, 8);
    if (head_ok) {
      float M = dot * p.scale_log2, lsum = 1.f;
      const int hvp_j = j % hvp;
      // group gi holds slots gi, gi + SG, ...: only the first nsl groups hold any
      const int SGu = min(SG, nsl);
      for (int gi = 0; gi < SGu; ++gi) {
        const float* g = &red[0][0][0] + (gi * hvp + hvp_j) * 16 * (DP + 2) + (tid & 15) * (DP + 2);
        const float mg = g[DP];
        const float m2 = fmaxf(M, mg);
        const float a = exp2f(M - m2), c = exp2f(mg - m2);
        lsum = lsum * a + g[DP + 1] * c;
#pragma unroll
        for (int i = 0; i < DP; ++i) o[i] = o[i] * a + g[i] * c;
        M = m2;
      }
      const float inv = 1.f / lsum;
#pragma unroll
      for (int i = 0; i < DP; ++i) out[i] = __builtin_bit_cast(uint16_t, (_Float16)(o[i] * inv));
    }
    if (tile == 0 && j == 0) {
      uint16_t* kdst = p.kc + ((int64_t)bk * p.S + L) * D + d0;
      uint16_t* vdst = p.vc + (int64_t)bk * p.S * D + ((int64_t)(L / kAttnBlock) * D + d0) * kAttnBlock + L % kAttnBlock;
#pragma unroll
      for (int i = 0; i < DP; ++i) {
        // element copied to a scalar first: a bit cast applied to a vector
        // element expression reads element 0
        const _Float16 ki = k16[i], vi = vnew[i];
        kdst[i] = __builtin_bit_cast(uint16_t, ki);
        vdst[i * kAttnBlock] = __builtin_bit_cast(uint16_t, vi);
      }
    }
  }
  // Leave the unit's part of the workspace as it was found, all zero: the
  // counter, and the nsl states this call wrote (their hv head rows), which
  // were all read above and consumed before the last barrier. A later call
  // with another shape may place its counters where these states lie.
  {
    float* pu = p.part + (int64_t)unit * p.C * 16 * HS;
    const int per_slot = hv * HS / 2;  // 8-byte stores per state
    for (int e = tid; e < nsl * per_slot; e += kAttnWaves * 64) {
      const int sl = e / per_slot, r = e - sl * per_slot;
      coherent_store2(pu + (int64_t)sl * 16 * HS + 2 * r, 0.f, 0.f);
    }
  }
  if (tid == 0) __hip_atomic_store(p.counters + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

AttnPlan attention_plan(int B, int Hq, int Hkv, int D, int max_cached, int steps) {
  AttnPlan pl;
  pl.g = Hq / Hkv;
  pl.T = (pl.g + 15) / 16;
  const int64_t units = (int64_t)B * Hkv * pl.T;
  const int64_t spu = max_cached > 0 ? (max_cached + kAttnBlock - 1) / kAttnBlock : 1;
  // About eight waves per CU over 256 CUs, each wave at least one 32-position step.
  const int64_t target = 2048;
  auto wgs = [&](int s) { return (int)((spu + (int64_t)kAttnWaves * s - 1) / ((int64_t)kAttnWaves * s)); };
  pl.steps = steps > 0 ? steps : (int)std::max<int64_t>(1, (units * spu + target - 1) / target);
  // Units of several query heads carry that many heads per merged state:
  // more than 8 states to merge then cost more than the longer per-wave
  // range of twice the steps (measured at B = 1: LLaMA-3-8B GQA, 4096
  // cached, 14.5 -> 12.8 us; Falcon-7B MQA, 2048 cached, 9.6 -> 8.8 us).
  if (steps <= 0 && pl.g > 1 && wgs(pl.steps) > 8) pl.steps *= 2;
  pl.C = wgs(pl.steps);
  pl.units = units;
  pl.counter_bytes = (size_t)((units * 4 + 255) / 256 * 256);
  pl.ws_bytes = pl.counter_bytes + (size_t)units * pl.C * 16 * (D + 4) * sizeof(float);
  return pl;
}

hipError_t launch_attention(const AttnParams& p, int D, const Launch& L) {
  const dim3 grid((unsigned)(p.C * (int64_t)(p.units)));
  const dim3 block(kAttnWaves * 64);
  if (D == 64) return launch_kernel(attn_decode_kernel<64>, grid, block, 0, L, p);
  return launch_kernel(attn_decode_kernel<128>, grid, block, 0, L, p);
}

}  // namespace awq
