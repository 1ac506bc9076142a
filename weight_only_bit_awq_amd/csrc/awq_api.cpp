// C ABI of the W4A16 group-quantised linear layer: argument validation,
// execution planning and dispatch to the gfx950 kernels. Declared in
// include/awq.h; every entry point validates before it enqueues anything and
// reports failures as negative status codes, never by throwing or aborting.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <algorithm>
#include <stdlib.h>

#include "../../include/awq.h"
#include "../../include/awq_probe.h"
#include "awq_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = (int64_t)1 << 30;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return AWQ_OK;
  g_last_hip_error = (int)e;
  return AWQ_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool group_ok(int G) { return G == 32 || G == 64 || (G > 0 && G % 128 == 0); }

int check_dims(int64_t M, int64_t K, int64_t N) {
  if (M < 0 || K < 0 || N < 0) return AWQ_ERR_SHAPE;
  if (M > kMaxDim || K > kMaxDim || N > kMaxDim) return AWQ_ERR_SHAPE;
  if (K * N > ((int64_t)1 << 40)) return AWQ_ERR_SHAPE;
  return AWQ_OK;
}

int check_layer(int64_t K, int64_t N, int G) {
  if (!group_ok(G)) return AWQ_ERR_GROUP;
  if (K % G != 0 || N % 8 != 0) return AWQ_ERR_SHAPE;
  return AWQ_OK;
}

struct Resolved {
  int path, split, waves, tpw, x_stage, tile;
  size_t ws_bytes;
  size_t counter_bytes;
};

constexpr int kDecodeMaxM = 64;

// Gated (silu(gate) * up) plans: on the decode path only the LDS-staged
// variant with the gate and up tiles paired in one workgroup exists (half of
// its waves on each tile), so the automatic choice takes the prefill path
// whenever that does not fit.
// Returns the number of waves the fused kernel uses (0 if it cannot run).
int gated_decode_waves(int64_t M, int64_t K, int G, const awq_plan& p) {
  if (M < 1 || M > 16 || p.tpw > 1 || p.x_stage == 2 || p.waves == 1 || p.waves == 2) return 0;
  for (int w : {8, 4, 16})
    if ((!p.waves || p.waves == w) && awq::decode_staged_fits((int)M, (int)K, G, w, 1)) return w;
  return 0;
}
// The streamed variant with the gate and up tiles sharing each band's
// activation loads (M <= 32, four or eight waves).
bool gated_stream_ok(int64_t M, const awq_plan& p) {
  return M >= 1 && M <= 32 && (!p.waves || p.waves == 4 || p.waves == 8) && p.x_stage != 1 &&
         (!p.tpw || p.tpw == 2 || p.tpw == 4);
}
bool gated_decode_fits(int64_t M, int64_t K, int G, const awq_plan& p) {
  return gated_decode_waves(M, K, G, p) > 0 || gated_stream_ok(M, p);
}

// An automatic K split shrinks until its fp32 partials (split * M * N * 4
// bytes, on either path) fit a workspace bound.
void cap_split(Resolved* out, int64_t M, int64_t N, size_t ws_cap, bool automatic) {
  while (automatic && out->split > 1 && out->ws_bytes > ws_cap) {
    --out->split;
    out->ws_bytes = out->split > 1 ? (size_t)out->split * (size_t)M * (size_t)N * 4 : 0;
  }
}

// ws_cap: a bound on the workspace (the library's own scratch for callers
// that cannot allocate).
int resolve_plan(int64_t M, int64_t K, int64_t N, int G, const awq_plan* in, Resolved* out, bool gated = false,
                 size_t ws_cap = SIZE_MAX) {
  awq_plan p = {};
  if (in) p = *in;
  if (p.path < 0 || p.path > 2 || p.split_k < 0 || p.waves < 0 || p.tpw < 0 || p.x_stage < 0 || p.x_stage > 3 ||
      p.tile < 0 || p.tile > 3)
    return AWQ_ERR_PLAN;
  if (gated && N % 32) return AWQ_ERR_SHAPE;
  // Automatic path: decode up to M = 64, except wide layers above M = 32,
  // where the prefill GEMM streams the weights faster than a decode kernel
  // that re-reads the activations per band and tile.
  if (p.path == 0)
    p.path = gated ? (gated_decode_fits(M, K, G, p) ? 1 : 2)
                   : (M <= kDecodeMaxM && !(M > 32 && (N + 15) / 16 > 1024)) ? 1 : 2;
  if (p.path == 1 && M > kDecodeMaxM) return AWQ_ERR_PLAN;
  if (p.path == 1 && gated && !gated_decode_fits(M, K, G, p)) return AWQ_ERR_PLAN;
  const int64_t KT = (K + 127) / 128;
  const int64_t NT = (N + 15) / 16;
  out->path = p.path;
  out->split = 1;
  out->waves = 0;
  out->tpw = 0;
  out->x_stage = 0;
  out->tile = 0;
  out->ws_bytes = 0;
  out->counter_bytes = 0;
  if (p.path == 1) {
    // The K range of a column tile is split over the waves of its workgroup
    // and summed through LDS in a fixed order. The streamed variant can also
    // split K over workgroups (split_k > 1): fp32 partials in the workspace,
    // added in a fixed order by a second kernel.
    if (p.split_k > 16) return AWQ_ERR_PLAN;
    if (p.split_k > 1 && p.x_stage == 1) return AWQ_ERR_PLAN;
    if (p.split_k > 1 && !p.x_stage) p.x_stage = 2;
    if (p.waves && p.waves != 1 && p.waves != 2 && p.waves != 4 && p.waves != 8 && p.waves != 16)
      return AWQ_ERR_PLAN;
    if (p.tpw > 4 || p.tpw == 3) return AWQ_ERR_PLAN;
    // Automatic choice (measured on the LLaMA-shaped decode layers, M = 1):
    // one 16-column tile per workgroup and eight waves splitting K, unless
    // the layer has fewer than 8 full 128-row bands or is so wide that the
    // workgroups need more than one round of the chip's wave slots: four
    // waves above 8192 waves at G = 128 (the kernel is held to 64 VGPRs,
    // 32 waves per CU; LLaMA-2-7B gate+up, 1376 tiles: 10.6-10.7 against
    // 11.2 us), above about 12k at other group sizes (Falcon-7B up at
    // G = 64, 1136 tiles: eight waves 13.3 against 13.6 us).
    if (gated) {
      // Fused gate+up: the staged kernel (halves of its waves on the gate
      // and the up tile) for one or two rows, else the streamed one with the
      // two tiles sharing each band's activation loads.
      if (p.tile) return AWQ_ERR_PLAN;
      // the slab variant with each wave on tpw/2 gate tiles and the matching
      // up tiles, automatic where the plain layer takes it (measured on the
      // LLaMA-3-8B gate+up, 4096 x 28672: 29.6 -> 24.7 us at M = 32, 24.9 ->
      // 22.9 at M = 24, level at M = 16; a 14848 x 59392 layer at M = 16:
      // 112.7 -> 86.4 us)
      const bool gslab_auto = !p.x_stage && !p.tpw && !p.waves && !p.split_k && M >= 16 && M <= 32 &&
                              G % 128 == 0 && (NT * KT >= 200000 || (M > 16 && NT >= 1024));
      if (p.x_stage == 3 || gslab_auto) {
        if (M < 1 || M > 32 || G % 128 || (p.waves && p.waves != 8) || (p.tpw && p.tpw != 2 && p.tpw != 4))
          return AWQ_ERR_PLAN;
        out->waves = 8;
        out->tpw = p.tpw ? p.tpw : 2;
        out->x_stage = 3;
        const int64_t groups = (NT / 2 + 4 * out->tpw - 1) / (4 * out->tpw);
        const int64_t slots = out->tpw == 2 ? 512 : 256;
        const int64_t auto_split =
            std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(slots / groups, KT / 16), 16));
        out->split = awq::decode_splits((int)K, p.split_k ? p.split_k : (int)auto_split);
        out->ws_bytes = out->split > 1 ? (size_t)out->split * (size_t)M * (size_t)N * 4 : 0;
        cap_split(out, M, N, ws_cap, p.split_k == 0);
        return AWQ_OK;
      }
      const int sw = gated_decode_waves(M, K, G, p);
      const bool st = gated_stream_ok(M, p);
      if (sw && (p.x_stage == 1 || M <= 2 || !st)) {
        out->waves = sw, out->tpw = 1, out->x_stage = 1;
      } else if (st) {
        // tpw = tiles per workgroup, half gate and half up: four (two
        // pairs) on wide layers, as for the plain layer
        const int64_t NH = NT / 2;
        int tw = p.tpw ? p.tpw : (NH >= 448 && NH % 2 == 0 && (M <= 16 || G >= 64)) ? 4 : 2;
        if (tw == 4 && NH % 2) return AWQ_ERR_PLAN;
        out->waves = p.waves ? p.waves : 4, out->tpw = tw, out->x_stage = 2;
        out->split = awq::decode_splits((int)K, p.split_k ? p.split_k : 1);
      } else {
        return AWQ_ERR_PLAN;
      }
      if (out->split > 1 && out->x_stage != 2) return AWQ_ERR_PLAN;
      out->ws_bytes = out->split > 1 ? (size_t)out->split * (size_t)M * (size_t)N * 4 : 0;
      cap_split(out, M, N, ws_cap, p.split_k == 0);
      return AWQ_OK;
    }
    // Slab variant: eight waves on the same bands, each with its own tpw
    // column tiles, the activations of two bands at a time staged in LDS
    // once per workgroup (one activation load per 8 * tpw tiles). Automatic
    // for 16-32 rows on the largest layers and, above 16 rows, on wide ones
    // (measured at M = 16: Falcon-180B-shaped up 14848 x 59392 108 -> 83 us,
    // down 59392 x 14848 103 -> 84 us; its QKV and O within 3% either way,
    // so left streamed; LLaMA-3-8B gate+up 4096 x 28672 at M = 32: 27.0 ->
    // 23.6 us, at M = 16 slower, 18.6 -> 19.8). Its workgroups run best as
    // one round: K is split until about that many workgroups, keeping at
    // least 16 bands per split.
    const bool slab_auto = !p.x_stage && !p.tpw && !p.waves && !p.split_k && M >= 16 && M <= 32 && G % 128 == 0 &&
                           (NT * KT >= 200000 || (M > 16 && NT >= 1024));
    if (p.x_stage == 3 || slab_auto) {
      if (p.tile || M < 1 || M > 32 || G % 128 || (p.waves && p.waves != 8) || p.tpw == 3)
        return AWQ_ERR_PLAN;
      out->waves = 8;
      // above 16 rows one tile per wave, one workgroup per CU (LLaMA-3-8B
      // gate+up at M = 32: 23.1-23.3 us against 24.8-24.9 with two tiles and
      // a K split, on three boxes)
      out->tpw = p.tpw ? p.tpw : (M > 16 ? 1 : 2);
      out->x_stage = 3;
      const int64_t groups = (NT + 8 * out->tpw - 1) / (8 * out->tpw);
      // workgroups per round: two per CU with one or two tiles per wave (at
      // most 121 VGPRs), one with four; above 16 rows the automatic plan
      // keeps one per CU
      const int64_t slots = (out->tpw == 4 || (M > 16 && !p.tpw)) ? 256 : 512;
      const int64_t auto_split = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(slots / groups, KT / 16), 16));
      out->split = awq::decode_splits((int)K, p.split_k ? p.split_k : (int)auto_split);
      out->ws_bytes = out->split > 1 ? (size_t)out->split * (size_t)M * (size_t)N * 4 : 0;
      cap_split(out, M, N, ws_cap, p.split_k == 0);
      return AWQ_OK;
    }
    int waves = p.waves;
    if (!waves) waves = (NT * 8 > (G == 128 ? 8192 : 12288) || KT < 8) ? 4 : 8;
    int tpw = p.tpw;
    if (!tpw) tpw = 1;
    int x_stage = p.x_stage;
    int auto_split = 1;
    if (!p.x_stage && !p.tpw && !p.waves && !p.split_k && M >= 16 && M <= 32 && NT <= 512 && KT >= 64) {
      // Many rows on a narrow layer with a long K (e.g. the LLaMA-3-8B down
      // projection, 14336 x 4096, at M = 16 .. 32): four K ranges over
      // workgroups of eight waves and four tiles, partials added by the
      // reduction kernel (measured 29.7 -> 19.6 us at M = 32, 16.8 -> 15.4
      // at M = 16; at M <= 8 or on shorter K the second launch costs more
      // than it saves).
      x_stage = 2, waves = 8, auto_split = 4;
    } else if (!p.x_stage && M >= 4 && M <= 32 && (NT >= 384 || M >= 8)) {
      // Batched rows on layers of 384 or more tiles, and from 8 rows on
      // narrower ones: the streamed variant, with adjacent tiles sharing
      // each band's activation loads, beats staging the activations per
      // workgroup (measured on the LLaMA-3-8B layers, M = 4 .. 32: e.g. QKV
      // at M = 8, 5.9 against 11.6 us; O at M = 8, 5.6 against 6.5 with 16
      // staging waves; O at M = 4 stays staged, 4.6 against 5.2).
      x_stage = 2;
      if (!p.waves) waves = 4;
    } else if (!p.waves && !p.x_stage && M >= 1 && !awq::decode_staged_fits((int)M, (int)K, G, waves, tpw)) {
      // Activations too large to stage with these waves: sixteen waves
      // stage twice as much per pass, but a 1024-thread workgroup with that
      // much LDS holds a whole CU, so only where there are few workgroups;
      // otherwise the streamed variant, with eight waves for one or two rows
      // (the Falcon-180B-shaped down projection, 59392 x 14848 at M = 1:
      // 84.9 us streamed with eight waves and four tiles per workgroup,
      // against 92.8 staged with sixteen waves and 106.8 streamed with four)
      // and four for more.
      if (NT <= 256 && awq::decode_staged_fits((int)M, (int)K, G, 16, tpw))
        waves = 16;
      else
        waves = M <= 2 ? 8 : 4;
    }
    const bool fits = M >= 1 && p.tpw <= 2 && awq::decode_staged_fits((int)M, (int)K, G, waves, tpw);
    if (x_stage == 0) x_stage = fits ? 1 : 2;
    if (x_stage == 1 && !fits) return AWQ_ERR_PLAN;
    if (x_stage == 2) {
      // Streamed: up to four adjacent tiles per workgroup share each band's
      // activation loads (M <= 32, four or eight waves); automatic: four
      // from 896 tiles (e.g. the Falcon-180B layers at M = 16: QKV 38.8 ->
      // 29.6 us, down 140 -> 107 us), two from 384.
      const bool multi = M <= 32 && (waves == 4 || waves == 8);
      if (p.tpw > 1 && !multi) return AWQ_ERR_PLAN;
      // (four tiles of 32 rows with four groups per band hold too many
      // registers: two there)
      tpw = p.tpw ? p.tpw
                  : !multi                                      ? 1
                  : auto_split > 1                              ? 4
                  : (NT >= 896 && (M <= 16 || G >= 64))         ? 4
                  : NT >= 384                                   ? 2
                                                                : 1;
      // two tiles per workgroup at up to 8 rows: eight waves (LLaMA-3-8B
      // QKV, 384 tiles: 5.7 against 6.3 us at M = 4, 6.0 against 6.3 at
      // M = 8; four waves from 16 rows, and with four tiles)
      if (!p.waves && auto_split == 1 && tpw == 2 && M <= 8) waves = 8;
    }
    if (p.tile) return AWQ_ERR_PLAN;
    out->waves = waves;
    out->tpw = tpw;
    out->x_stage = x_stage;
    if (p.split_k > 1 && x_stage != 2) return AWQ_ERR_PLAN;
    out->split = x_stage == 2 ? awq::decode_splits((int)K, p.split_k ? p.split_k : auto_split) : 1;
    out->ws_bytes = out->split > 1 ? (size_t)out->split * (size_t)M * (size_t)N * 4 : 0;
  } else {
    if (p.waves || p.tpw || p.x_stage) return AWQ_ERR_PLAN;
    if (!awq::prefill_fits((int)K, (int)N)) return AWQ_ERR_SHAPE;
    // K split over workgroups: at most one split per K step, at most 16.
    if (p.split_k > 16) return AWQ_ERR_PLAN;
    int tile = p.tile, split = p.split_k;
    awq::prefill_auto_plan((int)M, (int)K, (int)N, &tile, &split);
    out->tile = tile;
    const int steps = awq::prefill_steps((int)K, out->tile);
    if (split > steps) split = steps > 0 ? steps : 1;
    out->split = split;
    out->ws_bytes = awq::prefill_workspace_bytes((int)M, (int)N, split, gated);
  }
  cap_split(out, M, N, ws_cap, p.split_k == 0);
  return AWQ_OK;
}

}  // namespace

namespace {

// noalloc: the split-K partials go to the library's static scratch (the
// caller passes no workspace); nothing is allocated.
int run_linear(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros, int64_t M,
               int64_t K, int64_t N, int group, uint16_t* y, void* workspace, size_t workspace_bytes,
               const awq_plan* plan, void* stream, void* start_event, void* stop_event, bool gated,
               bool noalloc = false) {
  int st = check_dims(M, K, N);
  if (st) return st;
  if ((st = check_layer(K, N, group))) return st;
  Resolved r;
  if ((st = resolve_plan(M, K, N, group, plan, &r, gated, noalloc ? awq::kNoAllocScratchBytes : SIZE_MAX)))
    return st;
  if (M == 0 || N == 0) return AWQ_OK;
  if (!y) return AWQ_ERR_NULL;
  const int64_t n_out = gated ? N / 2 : N;
  if (K == 0) {
    // Empty contraction: y = 0 (silu(0) * 0 = 0 for the gated form).
    if (!aligned(y, 2)) return AWQ_ERR_ALIGN;
    return hip_status(awq::launch_fill_zero(y, M * n_out, (hipStream_t)stream));
  }
  if (!x || !qweight || !scales || !zeros) return AWQ_ERR_NULL;
  // y: 8-byte aligned wherever four outputs are stored at once (the gated
  // prefill epilogue, and the reduction of split-K partials)
  const bool y_by_four = (r.path == 2 && gated) || r.split > 1;
  if (!aligned(x, 16) || !aligned(qweight, 16) || !aligned(scales, 2) || !aligned(zeros, 4) ||
      !aligned(y, y_by_four ? 8 : 2))
    return AWQ_ERR_ALIGN;
  if (r.ws_bytes && noalloc) {
    if (r.ws_bytes > awq::kNoAllocScratchBytes) return AWQ_ERR_WORKSPACE;
    float* p = nullptr;
    if ((st = hip_status(awq::noalloc_scratch(&p)))) return st;
    workspace = p;
    workspace_bytes = awq::kNoAllocScratchBytes;
  }
  if (r.ws_bytes) {
    if (!workspace || workspace_bytes < r.ws_bytes) return AWQ_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return AWQ_ERR_ALIGN;
  }
  if (M * K * 2 >= ((int64_t)1 << 31) || (K / group) * N * 2 >= ((int64_t)1 << 31))
    return AWQ_ERR_SHAPE;  // the kernels address x and scales with 32-bit buffer offsets
  awq::LinearArgs a{x, qweight, scales, zeros, y, (int)M, (int)K, (int)N, group};
  const awq::Launch L{(hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event};
  if (r.path == 1) {
    const awq::DecodeConfig cfg{r.waves, r.tpw, r.x_stage == 1, gated, r.split, static_cast<float*>(workspace),
                                r.x_stage == 3};
    return hip_status(awq::launch_decode(a, cfg, L));
  }
  return hip_status(awq::launch_prefill(a, r.tile, r.split, static_cast<float*>(workspace), gated, L));
}

int plan_out(int64_t M, int64_t K, int64_t N, int group, awq_plan* plan, bool gated) {
  int st = check_dims(M, K, N);
  if (st) return st;
  if ((st = check_layer(K, N, group))) return st;
  if (!plan) return AWQ_ERR_NULL;
  Resolved r;
  if ((st = resolve_plan(M, K, N, group, plan, &r, gated))) return st;
  plan->path = r.path;
  plan->split_k = r.split;
  plan->waves = r.waves;
  plan->tpw = r.tpw;
  plan->x_stage = r.x_stage;
  plan->tile = r.tile;
  return AWQ_OK;
}

int workspace_out(int64_t M, int64_t K, int64_t N, int group, const awq_plan* plan, size_t* bytes, bool gated) {
  int st = check_dims(M, K, N);
  if (st) return st;
  if ((st = check_layer(K, N, group))) return st;
  if (!bytes) return AWQ_ERR_NULL;
  Resolved r;
  if ((st = resolve_plan(M, K, N, group, plan, &r, gated))) return st;
  *bytes = (M == 0 || K == 0 || N == 0) ? 0 : r.ws_bytes;
  return AWQ_OK;
}

}  // namespace

namespace {

// W4A8-FP8: shapes the FP8 path supports (groups of whole 128-row bands).
int w4a8_check(int64_t M, int64_t K, int64_t N, int G) {
  int st = check_dims(M, K, N);
  if (st) return st;
  if (!(G == 32 || G == 64 || (G > 0 && G % 128 == 0))) return AWQ_ERR_GROUP;
  if (K % G || K % 128 || N % 8) return AWQ_ERR_SHAPE;
  if (M * K >= ((int64_t)1 << 31) || !awq::prefill_fits((int)K, (int)N)) return AWQ_ERR_SHAPE;
  return AWQ_OK;
}

// Tile 2 (128 x 128) or 3 (256 x 256) and the K split; explicit plan fields
// (tile, split_k) are honoured, the rest chosen by the prefill cost model.
int w4a8_plan(int64_t M, int64_t K, int64_t N, const awq_plan* plan, int* tile, int* splits) {
  *tile = plan ? plan->tile : 0;
  *splits = plan ? plan->split_k : 0;
  if (plan && (plan->path || plan->waves || plan->tpw || plan->x_stage)) return AWQ_ERR_PLAN;
  if (*tile == 1 || *tile < 0 || *tile > 3 || *splits < 0 || *splits > 16) return AWQ_ERR_PLAN;
  if (*splits > (int)(K / 128)) return AWQ_ERR_PLAN;
  // the W4A8 form of the model picks the measured best plan on every
  // LLaMA-2-13B shape at M = 512 and 2048
  awq::prefill_auto_plan((int)M, (int)K, (int)N, tile, splits, awq::PrefillKind::kW4A8);
  return AWQ_OK;
}

int w4a8_run(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros, int64_t M,
             int64_t K, int64_t N, int group, uint16_t* y, void* workspace, size_t workspace_bytes,
             const awq_plan* plan, const awq::Launch& L) {
  int st = w4a8_check(M, K, N, group);
  if (st) return st;
  if (M == 0 || N == 0) return AWQ_OK;
  if (!y) return AWQ_ERR_NULL;
  if (!aligned(y, 16)) return AWQ_ERR_ALIGN;
  // empty contraction: y = 0, nothing else is read
  if (K == 0) return hip_status(awq::launch_fill_zero(y, M * N, L.stream));
  if (!x || !qweight || !scales || !zeros) return AWQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(qweight, 16) || !aligned(y, 16) || !aligned(scales, 4) || !aligned(zeros, 4))
    return AWQ_ERR_ALIGN;
  int tile, splits;
  if ((st = w4a8_plan(M, K, N, plan, &tile, &splits))) return st;
  const size_t need = awq::w4a8_workspace_bytes((int)M, (int)K, (int)N, splits);
  if (!workspace || workspace_bytes < need) return AWQ_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return AWQ_ERR_ALIGN;
  const awq::LinearArgs a{x, qweight, scales, zeros, y, (int)M, (int)K, (int)N, group};
  return hip_status(awq::launch_w4a8(a, tile, splits, workspace, L));
}

// Attention: validation of the descriptor and the work split it implies.
int attention_check(const awq_attn_desc* d, awq::AttnPlan* pl) {
  if (!d) return AWQ_ERR_NULL;
  if (d->batch < 0 || d->batch > (1 << 24) || d->q_heads < 1 || d->kv_heads < 1 || d->q_heads > 65536 ||
      d->q_heads % d->kv_heads)
    return AWQ_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return AWQ_ERR_SHAPE;
  if (d->capacity < 32 || d->capacity % 32 || d->capacity > (1 << 24)) return AWQ_ERR_SHAPE;
  if (d->max_cached < 0 || d->max_cached >= d->capacity) return AWQ_ERR_SHAPE;
  if (d->qkv_stride < (d->q_heads + 2 * d->kv_heads) * d->head_dim || d->qkv_stride % 8) return AWQ_ERR_SHAPE;
  if (d->rope_style < AWQ_ROPE_NONE || d->rope_style > AWQ_ROPE_INTERLEAVED) return AWQ_ERR_ARG;
  if (d->rope_style != AWQ_ROPE_NONE && !(d->rope_theta > 0.f && d->rope_theta < INFINITY)) return AWQ_ERR_ARG;
  if (!(d->softmax_scale >= 0.f && d->softmax_scale < INFINITY)) return AWQ_ERR_ARG;
  if (d->steps < 0 || d->steps > 4096) return AWQ_ERR_PLAN;
  *pl = awq::attention_plan((int)d->batch, (int)d->q_heads, (int)d->kv_heads, (int)d->head_dim,
                            (int)d->max_cached, d->steps);
  if ((int64_t)pl->C * pl->units > 0x7FFFFFFF) return AWQ_ERR_SHAPE;
  return AWQ_OK;
}

int attention_run(const awq_attn_desc* d, const uint16_t* qkv, uint16_t* kc, uint16_t* vc, const int32_t* lengths,
                  uint16_t* out, void* ws, size_t ws_bytes, const awq::Launch& L) {
  awq::AttnPlan pl;
  int st = attention_check(d, &pl);
  if (st != AWQ_OK) return st;
  if (d->batch == 0) return AWQ_OK;
  if (!qkv || !kc || !vc || !lengths || !out) return AWQ_ERR_NULL;
  if (!aligned(qkv, 16) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(out, 16) || !aligned(lengths, 4))
    return AWQ_ERR_ALIGN;
  if (!ws || ws_bytes < pl.ws_bytes) return AWQ_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return AWQ_ERR_ALIGN;
  awq::AttnParams p;
  p.qkv = qkv;
  p.qkv_stride = d->qkv_stride;
  p.kc = kc;
  p.vc = vc;
  p.lengths = lengths;
  p.out = out;
  p.counters = (uint32_t*)ws;
  p.part = (float*)((char*)ws + pl.counter_bytes);
  p.units = pl.units;
  p.Hq = (int)d->q_heads;
  p.Hkv = (int)d->kv_heads;
  p.S = (int)d->capacity;
  p.max_cached = (int)d->max_cached;
  p.g = pl.g;
  p.T = pl.T;
  p.C = pl.C;
  p.steps = pl.steps;
  p.style = d->rope_style;
  const double scale = d->softmax_scale > 0.f ? (double)d->softmax_scale : 1.0 / sqrt((double)d->head_dim);
  p.scale_log2 = (float)(scale * 1.4426950408889634);
  p.log2_theta = d->rope_style != AWQ_ROPE_NONE ? log2((double)d->rope_theta) : 0.0;
  return hip_status(awq::launch_attention(p, (int)d->head_dim, L));
}

}  // namespace

extern "C" {

const char* awq_status_string(int status) {
  switch (status) {
    case AWQ_OK: return "AWQ_OK";
    case AWQ_ERR_NULL: return "AWQ_ERR_NULL: a required pointer is NULL";
    case AWQ_ERR_SHAPE: return "AWQ_ERR_SHAPE: invalid sizes (negative, N % 8, K % group, ...)";
    case AWQ_ERR_GROUP: return "AWQ_ERR_GROUP: group must be 32, 64 or a positive multiple of 128";
    case AWQ_ERR_ALIGN: return "AWQ_ERR_ALIGN: a pointer is not suitably aligned";
    case AWQ_ERR_WORKSPACE: return "AWQ_ERR_WORKSPACE: workspace missing or too small";
    case AWQ_ERR_HIP: return "AWQ_ERR_HIP: the HIP runtime reported an error";
    case AWQ_ERR_PLAN: return "AWQ_ERR_PLAN: an explicit plan field is out of range";
    case AWQ_ERR_ARG: return "AWQ_ERR_ARG: a scalar argument is out of range";
  }
  return "AWQ: unknown status";
}

int awq_last_hip_error(void) { return g_last_hip_error; }

int awq_abi_version(void) { return 1; }

size_t awq_qweight_words(int64_t K, int64_t N) {
  if (K <= 0 || N <= 0) return 0;
  return (size_t)((K + 127) / 128) * (size_t)((N + 15) / 16) * 256;
}

int awq_pack(const uint8_t* q, int64_t K, int64_t N, uint32_t* qweight, void* stream) {
  int st = check_dims(0, K, N);
  if (st) return st;
  if (K % 8 || N % 8) return AWQ_ERR_SHAPE;
  if (K == 0 || N == 0) return AWQ_OK;
  if (!q || !qweight) return AWQ_ERR_NULL;
  if (!aligned(qweight, 16)) return AWQ_ERR_ALIGN;
  return hip_status(awq::launch_pack(q, (int)K, (int)N, qweight, (hipStream_t)stream));
}

int awq_unpack(const uint32_t* qweight, int64_t K, int64_t N, uint8_t* q, void* stream) {
  int st = check_dims(0, K, N);
  if (st) return st;
  if (K % 8 || N % 8) return AWQ_ERR_SHAPE;
  if (K == 0 || N == 0) return AWQ_OK;
  if (!q || !qweight) return AWQ_ERR_NULL;
  if (!aligned(qweight, 16)) return AWQ_ERR_ALIGN;
  return hip_status(awq::launch_unpack(qweight, (int)K, (int)N, q, (hipStream_t)stream));
}

int awq_pack_zeros(const uint8_t* z, int64_t groups, int64_t N, uint32_t* zeros, void* stream) {
  int st = check_dims(0, groups, N);
  if (st) return st;
  if (N % 8) return AWQ_ERR_SHAPE;
  if (groups == 0 || N == 0) return AWQ_OK;
  if (!z || !zeros) return AWQ_ERR_NULL;
  if (!aligned(zeros, 4)) return AWQ_ERR_ALIGN;
  return hip_status(awq::launch_pack_zeros(z, (int)groups, (int)N, zeros, (hipStream_t)stream));
}

int awq_dequant(const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros, int64_t K, int64_t N,
                int group, uint16_t* w, void* stream) {
  int st = check_dims(0, K, N);
  if (st) return st;
  if ((st = check_layer(K, N, group))) return st;
  if (K == 0 || N == 0) return AWQ_OK;
  if (!qweight || !scales || !zeros || !w) return AWQ_ERR_NULL;
  if (!aligned(qweight, 16) || !aligned(scales, 2) || !aligned(zeros, 4) || !aligned(w, 2)) return AWQ_ERR_ALIGN;
  return hip_status(awq::launch_dequant(qweight, scales, zeros, (int)K, (int)N, group, w, (hipStream_t)stream));
}

int awq_quantize(const uint16_t* w, int64_t K, int64_t N, int group, uint32_t* qweight, uint16_t* scales,
                 uint32_t* zeros, void* stream) {
  int st = check_dims(0, K, N);
  if (st) return st;
  if ((st = check_layer(K, N, group))) return st;
  if (K == 0 || N == 0) return AWQ_OK;
  if (!w || !qweight || !scales || !zeros) return AWQ_ERR_NULL;
  if (!aligned(w, 16) || !aligned(qweight, 16) || !aligned(scales, 2) || !aligned(zeros, 4)) return AWQ_ERR_ALIGN;
  return hip_status(awq::launch_quantize(w, (int)K, (int)N, group, qweight, scales, zeros, (hipStream_t)stream));
}

int awq_linear_plan(int64_t M, int64_t K, int64_t N, int group, awq_plan* plan) {
  return plan_out(M, K, N, group, plan, false);
}

int awq_linear_workspace_bytes_ex(int64_t M, int64_t K, int64_t N, int group, const awq_plan* plan,
                                  size_t* bytes) {
  return workspace_out(M, K, N, group, plan, bytes, false);
}

int awq_linear_workspace_bytes(int64_t M, int64_t K, int64_t N, int group, size_t* bytes) {
  return awq_linear_workspace_bytes_ex(M, K, N, group, nullptr, bytes);
}

size_t awq_linear_workspace_size(int64_t M, int64_t K, int64_t N, int group) {
  size_t bytes = 0;
  return awq_linear_workspace_bytes(M, K, N, group, &bytes) == AWQ_OK ? bytes : SIZE_MAX;
}

int awq_linear_timed(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                     int64_t M, int64_t K, int64_t N, int group, uint16_t* y, void* workspace, size_t workspace_bytes,
                     const awq_plan* plan, void* stream, void* start_event, void* stop_event) {
  return run_linear(x, qweight, scales, zeros, M, K, N, group, y, workspace, workspace_bytes, plan, stream,
                    start_event, stop_event, false);
}

int awq_linear_silu_mul_ex(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                           const uint32_t* zeros, int64_t M, int64_t K, int64_t N, int group, uint16_t* y,
                           void* workspace, size_t workspace_bytes, const awq_plan* plan, void* stream,
                           void* start_event, void* stop_event) {
  return run_linear(x, qweight, scales, zeros, M, K, N, group, y, workspace, workspace_bytes, plan, stream,
                    start_event, stop_event, true);
}

int awq_linear_silu_mul(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                        int64_t M, int64_t K, int64_t N, int group, uint16_t* y, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return run_linear(x, qweight, scales, zeros, M, K, N, group, y, workspace, workspace_bytes, nullptr, stream,
                    nullptr, nullptr, true);
}

int awq_linear_silu_mul_plan(int64_t M, int64_t K, int64_t N, int group, awq_plan* plan) {
  return plan_out(M, K, N, group, plan, true);
}

int awq_linear_silu_mul_workspace_bytes(int64_t M, int64_t K, int64_t N, int group, const awq_plan* plan,
                                        size_t* bytes) {
  return workspace_out(M, K, N, group, plan, bytes, true);
}

int awq_linear_ex(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                  int64_t M, int64_t K, int64_t N, int group, uint16_t* y, void* workspace, size_t workspace_bytes,
                  const awq_plan* plan, void* stream) {
  return awq_linear_timed(x, qweight, scales, zeros, M, K, N, group, y, workspace, workspace_bytes, plan, stream,
                          nullptr, nullptr);
}

int awq_stream_read(const void* buf, size_t bytes, void* sink, void* stream, void* start_event, void* stop_event) {
  if (bytes == 0) return AWQ_OK;
  if (!buf || !sink) return AWQ_ERR_NULL;
  if (bytes % 16) return AWQ_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 16)) return AWQ_ERR_ALIGN;
  const awq::Launch L{(hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event};
  return hip_status(awq::launch_stream_read(buf, (uint64_t)bytes, sink, L));
}

int awq_linear(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros, int64_t M,
               int64_t K, int64_t N, int group, uint16_t* y, void* workspace, size_t workspace_bytes, void* stream) {
  return awq_linear_ex(x, qweight, scales, zeros, M, K, N, group, y, workspace, workspace_bytes, nullptr, stream);
}

int awq_linear_noalloc(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                       int64_t M, int64_t K, int64_t N, int group, uint16_t* y, const awq_plan* plan, void* stream) {
  return run_linear(x, qweight, scales, zeros, M, K, N, group, y, nullptr, 0, plan, stream, nullptr, nullptr, false,
                    true);
}

int awq_quantize_act_fp8(const uint16_t* x, int64_t M, int64_t K, uint8_t* x8, float* sx, void* stream) {
  if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim || K % 128) return AWQ_ERR_SHAPE;
  if (M == 0 || K == 0) return AWQ_OK;
  if (!x || !x8 || !sx) return AWQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(sx, 4)) return AWQ_ERR_ALIGN;
  const awq::Launch L{(hipStream_t)stream, nullptr, nullptr};
  return hip_status(awq::launch_act_quant_fp8(x, (int)M, (int)K, x8, sx, L));
}

int awq_linear_w4a8_workspace_bytes(int64_t M, int64_t K, int64_t N, int group, const awq_plan* plan,
                                    size_t* bytes) {
  if (!bytes) return AWQ_ERR_NULL;
  int st = w4a8_check(M, K, N, group);
  if (st) return st;
  if (M == 0 || K == 0 || N == 0) {
    *bytes = 0;
    return AWQ_OK;
  }
  int tile, splits;
  if ((st = w4a8_plan(M, K, N, plan, &tile, &splits))) return st;
  *bytes = awq::w4a8_workspace_bytes((int)M, (int)K, (int)N, splits);
  return AWQ_OK;
}

int awq_linear_w4a8_plan(int64_t M, int64_t K, int64_t N, int group, awq_plan* plan) {
  if (!plan) return AWQ_ERR_NULL;
  int st = w4a8_check(M, K, N, group);
  if (st) return st;
  int tile, splits;
  if ((st = w4a8_plan(M, K, N, plan, &tile, &splits))) return st;
  *plan = awq_plan{};
  plan->path = 2;
  plan->tile = tile;
  plan->split_k = splits;
  return AWQ_OK;
}

int awq_linear_w4a8(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                    int64_t M, int64_t K, int64_t N, int group, uint16_t* y, void* workspace,
                    size_t workspace_bytes, void* stream) {
  const awq::Launch L{(hipStream_t)stream, nullptr, nullptr};
  return w4a8_run(x, qweight, scales, zeros, M, K, N, group, y, workspace, workspace_bytes, nullptr, L);
}

int awq_linear_w4a8_ex(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                       int64_t M, int64_t K, int64_t N, int group, uint16_t* y, void* workspace,
                       size_t workspace_bytes, const awq_plan* plan, void* stream, void* start_event,
                       void* stop_event) {
  const awq::Launch L{(hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event};
  return w4a8_run(x, qweight, scales, zeros, M, K, N, group, y, workspace, workspace_bytes, plan, L);
}

int awq_attention_workspace_bytes(const awq_attn_desc* desc, size_t* bytes) {
  if (!bytes) return AWQ_ERR_NULL;
  awq::AttnPlan pl;
  const int st = attention_check(desc, &pl);
  if (st != AWQ_OK) return st;
  *bytes = desc->batch ? pl.ws_bytes : 0;
  return AWQ_OK;
}

int awq_attention_plan(const awq_attn_desc* desc, int32_t* workgroups_per_unit, int32_t* steps) {
  awq::AttnPlan pl;
  const int st = attention_check(desc, &pl);
  if (st != AWQ_OK) return st;
  if (workgroups_per_unit) *workgroups_per_unit = pl.C;
  if (steps) *steps = pl.steps;
  return AWQ_OK;
}

int awq_attention_decode(const awq_attn_desc* desc, const uint16_t* qkv, uint16_t* k_cache, uint16_t* v_cache,
                         const int32_t* lengths, uint16_t* out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  const awq::Launch L{(hipStream_t)stream, nullptr, nullptr};
  return attention_run(desc, qkv, k_cache, v_cache, lengths, out, workspace, workspace_bytes, L);
}

int awq_attention_decode_timed(const awq_attn_desc* desc, const uint16_t* qkv, uint16_t* k_cache,
                               uint16_t* v_cache, const int32_t* lengths, uint16_t* out, void* workspace,
                               size_t workspace_bytes, void* stream, void* start_event, void* stop_event) {
  const awq::Launch L{(hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event};
  return attention_run(desc, qkv, k_cache, v_cache, lengths, out, workspace, workspace_bytes, L);
}

}  // extern "C"
