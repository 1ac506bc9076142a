/*
 * awq.h -- C ABI of the MI355X (gfx950) W4A16 group-quantised linear layer.
 *
 * The operation: y[M,N] = x[M,K] . W[K,N] with
 *     W[k,n] = (q[k,n] - z[k/G, n]) * s[k/G, n],
 * q and z unsigned 4-bit codes, s fp16 scales, x and y fp16, fp32 accumulation.
 * "TinyChat: Efficient and Lightweight Chatbot with AWQ", section "Usage",
 * steps 3-4: weights quantised to 4 bits in groups of 128 input channels
 * (64 for Falcon-7B) and run as W4A16 (4-bit weights, 16-bit activations);
 * section "Speed Benchmarks": the W4A16 GPU kernel serves the generation
 * stage. The pages print neither the dequantisation rule nor a packing
 * order; the asymmetric affine rule above and the layouts below are the
 * readings this library adopts.
 *
 * Conventions for every entry point
 *   - All array pointers are DEVICE pointers (hipMalloc / torch CUDA tensors),
 *     row-major and contiguous, 16-byte aligned. The caller owns every buffer;
 *     the library allocates no device memory and keeps no per-call state.
 *   - fp16 values are passed as their uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *     enqueues work on `stream` and returns without synchronising; inputs
 *     must stay unchanged until the stream has reached the call.
 *   - Return value: AWQ_OK (0) or a negative AWQ_ERR_* code. Arguments are
 *     validated before anything is enqueued; on error nothing is launched.
 *     M, K or N equal to 0 is a valid empty call that launches nothing.
 *   - Shapes: K % group == 0; group is 32, 64 or a multiple of 128; N % 8 == 0.
 *
 * Layouts
 *   q (unpacked codes)   uint8 [K, N]; only the low 4 bits of each byte are used.
 *   scales               fp16  [K/G, N].
 *   zeros (packed)       uint32 [K/G, N/8]; bits 4i..4i+3 of word (g, c) hold
 *                        z[g, 8c+i] (least-significant nibble first).
 *   qweight (device)     awq_qweight_words(K, N) uint32 words in tiles of
 *                        16 columns x 128 rows: KT = ceil(K/128), NT = ceil(N/16),
 *                        tile (t, kt) starts at word (kt*NT + t)*256 (the tiles
 *                        of one 128-row band are adjacent). Word w of
 *                        a tile, lane l = w/4, slot j = w%4, holds column
 *                        n = 16t + l%16 and rows k0..k0+7, k0 = 128kt + 32j + 8(l/16);
 *                        row k0+e sits in nibble position 4(e%2) + e/2.
 *                        Padding rows (k >= K) and columns (n >= N) hold 0.
 *                        One 64-lane 16-byte load reads one whole tile, and each
 *                        word unpacks into two-row fp16 pairs (k0, k0+1), ...
 *                        with a mask-and-or per pair. The choice follows the
 *                        idea of interleaved weight repacking for wide loads
 *                        ("PowerInfer_SmallThinker-4BA0.6B-Instruct-GGUF" page,
 *                        section "ARM/AVX information").
 */
#ifndef AWQ_MI355X_AWQ_H
#define AWQ_MI355X_AWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum awq_status {
  AWQ_OK = 0,
  AWQ_ERR_NULL = -1,      /* a required pointer is NULL                        */
  AWQ_ERR_SHAPE = -2,     /* negative size, N % 8 != 0, K % group != 0, ...   */
  AWQ_ERR_GROUP = -3,     /* group not 32, 64 or a positive multiple of 128   */
  AWQ_ERR_ALIGN = -4,     /* a pointer is not aligned as its entry requires    */
  AWQ_ERR_WORKSPACE = -5, /* workspace NULL or smaller than required          */
  AWQ_ERR_HIP = -6,       /* the HIP runtime reported an error (see below)    */
  AWQ_ERR_PLAN = -7,      /* an explicit plan field is out of range           */
  AWQ_ERR_ARG = -8        /* a scalar argument is out of range                */
};

/* Human-readable name of a status code (static string, never NULL). Error
 * reporting of this library; the pages define no API. */
const char* awq_status_string(int status);

/* hipError_t of the most recent AWQ_ERR_HIP on the calling thread (0 if none). */
int awq_last_hip_error(void);

/* ABI version: bumped when a signature or a layout changes. */
int awq_abi_version(void);

/* Number of uint32 words of the device qweight layout for a [K, N] matrix
 * (the "real" INT4 weights of TinyChat README "Usage" step 3, in the layout
 * above); 0 if K or N is not positive. */
size_t awq_qweight_words(int64_t K, int64_t N);

/*
 * awq_pack: codes q uint8 [K, N] -> device-layout qweight (awq_qweight_words
 * words, written entirely, padding included). K % 8 == 0, N % 8 == 0.
 * The "real" INT4 weights of TinyChat README "Usage" step 3 (--q_backend real),
 * arranged for 16-byte gfx950 vector loads.
 */
int awq_pack(const uint8_t* q, int64_t K, int64_t N, uint32_t* qweight, void* stream);

/*
 * awq_unpack: inverse of awq_pack (TinyChat README "Usage" step 3, the "real"
 * INT4 weights read back): qweight in the device layout -> q uint8 [K, N]
 * with values 0..15, written entirely. K % 8 == 0, N % 8 == 0; qweight
 * 16-byte aligned. A test and interchange aid, not on the layer's path.
 */
int awq_unpack(const uint32_t* qweight, int64_t K, int64_t N, uint8_t* q, void* stream);

/*
 * awq_pack_zeros: the 4-bit zero points of the group-wise weights (TinyChat
 * README "Usage" step 3: one per group of --q_group_size input channels and
 * output column), z uint8 [groups, N] (low nibble used) -> packed uint32
 * [groups, N/8], least-significant nibble first along N. N % 8 == 0; zeros
 * 4-byte aligned.
 */
int awq_pack_zeros(const uint8_t* z, int64_t groups, int64_t N, uint32_t* zeros, void* stream);

/*
 * awq_dequant: device qweight + scales + packed zeros -> W fp16 [K, N], with
 * W[k,n] = round_to_nearest_even_fp16((q[k,n] - z[k/G,n]) * s[k/G,n])
 * (the exact product rounded once; IEEE special values, subnormals kept).
 * The 16-bit weights a W4A16 layer multiplies (TinyChat README "Usage" step
 * 4, --precision W4A16), materialised: a reference and test aid, the layer
 * itself never writes them. qweight 16-byte, scales and w 2-byte, zeros
 * 4-byte aligned.
 */
int awq_dequant(const uint32_t* qweight, const uint16_t* scales, const uint32_t* zeros,
                int64_t K, int64_t N, int group, uint16_t* w, void* stream);

/*
 * awq_quantize: fp16 weights w [K, N] (16-byte aligned) -> device-layout
 * qweight (awq_qweight_words words, padding included), fp16 scales
 * [K/G, N] and packed zero points [K/G, N/8]: the round-to-nearest group
 * quantiser that makes the "real" INT4 weights (TinyChat README "Usage"
 * step 3; the plain round-to-nearest variant is named on the Sagemaker
 * page, section "GGUF"). Per group of G input channels and output column:
 *     s = fp16((max - min) / 15), or 1 if that rounds to 0,
 *     z = clamp(rne(-min / s), 0, 15),  q = clamp(rne(w / s) + z, 0, 15),
 * every step one IEEE float32 operation, rne = round half to even. Weights
 * must be finite. A group whose range does not contain 0 has its zero point
 * clamped and loses the far end of its range.
 */
int awq_quantize(const uint16_t* w, int64_t K, int64_t N, int group, uint32_t* qweight,
                 uint16_t* scales, uint32_t* zeros, void* stream);

/*
 * Execution plan of awq_linear. Zero fields mean "choose automatically".
 *   path:    1 = decode path (dequantise in registers, MFMA 16x16x32, M <= 64),
 *            2 = prefill path (LDS-tiled dequant-then-MFMA GEMM, any M).
 *   split_k: number of contiguous K ranges (1..16, whole 128-row bands on
 *            the decode path) computed by separate workgroups; their fp32
 *            partial sums go to the workspace and a second kernel adds them
 *            in a fixed order and rounds once to fp16 (results do not depend
 *            on scheduling). Prefill path: chosen automatically from a
 *            measured cost model when the output has fewer tiles than the
 *            chip has workgroup slots and the split saves more than its
 *            partials cost (e.g. 512 x 5120 outputs). Decode path: streamed
 *            and slab variants only (x_stage 2, 3); chosen automatically for
 *            16..32 rows on narrow layers with a long K and with the slab
 *            variant, elsewhere the second launch costs more than the extra
 *            parallelism gains.
 *   waves:   decode path: waves per workgroup (1, 2, 4, 8 or 16); with
 *            x_stage 1 or 2 they split the K range of the workgroup's columns
 *            and their partial sums are added through LDS in a fixed order;
 *            the slab variant runs 8 waves, each on its own columns.
 *   tpw:     decode path: 16-column tiles per workgroup: 1 or 2 with staged
 *            activations; 1, 2 or 4 with streamed activations (M <= 32, 4 or
 *            8 waves), where each wave's activation loads serve all of them;
 *            slab variant: tiles per wave, 1, 2 or 4 (automatic: 2 up to 16
 *            rows, 1 above; gated: 2 or 4, half gate and half up).
 *   x_stage: decode path: 1 = activations and the (scale, zero point) words
 *            of the workgroup's columns staged in LDS once per workgroup
 *            (needs M <= 16 and the data to fit in 160 KiB), 2 = activations,
 *            scales and zero points read per tile, 3 = slab: the workgroup's
 *            eight waves walk the same 128-row bands, the activations of two
 *            bands at a time staged in LDS once for all of them (M <= 32, G a
 *            multiple of 128; chosen automatically for 16..32 rows on the
 *            largest layers and, above 16 rows, on wide ones).
 *   tile:    prefill path: workgroup tile 1 = 128x128 outputs (4 waves,
 *            64-row K steps, smallest LDS), 2 = 128x128 (4 waves, 128-row
 *            steps), 3 = 256x256 (8 waves, 128-row steps).
 */
typedef struct awq_plan {
  int32_t path;
  int32_t split_k;
  int32_t waves;
  int32_t tpw;
  int32_t x_stage;
  int32_t tile;
  int32_t reserved[2];
} awq_plan;

/* Resolves the automatic fields of *plan for this shape (plan may be all-zero). */
int awq_linear_plan(int64_t M, int64_t K, int64_t N, int group, awq_plan* plan);

/*
 * Workspace bytes awq_linear needs for this shape and plan: 0, or
 * split_k * M * N * 4 bytes of fp32 partial sums for a plan with
 * split_k > 1 (the split-K of the layer, reduced in a fixed order; TinyChat
 * README "Usage" step 4, the W4A16 layer). The workspace needs no
 * initialisation (every byte used is written before it is read); it must be
 * 16-byte aligned, and calls that overlap in time must not share it.
 * The _bytes forms return a status and write *bytes; awq_linear_workspace_size
 * returns the size for the automatic plan directly, or SIZE_MAX when the
 * arguments are invalid (awq_linear rejects them too).
 */
int awq_linear_workspace_bytes(int64_t M, int64_t K, int64_t N, int group, size_t* bytes);
int awq_linear_workspace_bytes_ex(int64_t M, int64_t K, int64_t N, int group,
                                  const awq_plan* plan, size_t* bytes);
size_t awq_linear_workspace_size(int64_t M, int64_t K, int64_t N, int group);

/*
 * awq_linear: y[M,N] (fp16) = x[M,K] (fp16) . W[K,N], W dequantised from
 * qweight/scales/zeros as in awq_dequant, accumulated in fp32, rounded once
 * to fp16 (round to nearest even). Result within 2e-3 of the exact value
 * relative to sum_k |x[m,k] * W[k,n]|; the summation order is not specified.
 * The W4A16 layer of TinyChat README "Usage" step 4 (--precision W4A16), the
 * generation-stage kernel of its "Speed Benchmarks". x and qweight 16-byte,
 * zeros 4-byte, scales 2-byte aligned; y 2-byte aligned, or 8-byte aligned
 * when the plan has split_k > 1 (its reduction stores four outputs at a
 * time). The workspace as awq_linear_workspace_bytes gives it.
 */
int awq_linear(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
               const uint32_t* zeros, int64_t M, int64_t K, int64_t N, int group,
               uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);

/* awq_linear with an explicit plan (for tuning and for testing both paths);
 * same operation, citation and rules as awq_linear. */
int awq_linear_ex(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                  const uint32_t* zeros, int64_t M, int64_t K, int64_t N, int group,
                  uint16_t* y, void* workspace, size_t workspace_bytes,
                  const awq_plan* plan, void* stream);

/*
 * awq_linear_noalloc: awq_linear_ex for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). It takes no workspace and allocates nothing: the fp32
 * partial sums of a plan that splits K go to a 64 MiB (67108864-byte)
 * array the library holds on every GPU it is loaded on until the process
 * ends. With plan NULL or split_k 0 the plan is awq_linear's automatic one
 * with the K split lowered until split_k * M * N * 4 bytes fit in 64 MiB
 * (down to no split, which needs none); an explicit split_k whose partials
 * exceed 64 MiB returns AWQ_ERR_WORKSPACE before anything is enqueued. All
 * calls on one GPU share the array and calls that overlap in time on one GPU
 * (other streams, other threads) race on it; the array needs no clearing
 * (every partial is written before it is read). Other arguments, alignment
 * and errors as for awq_linear_ex.
 */
int awq_linear_noalloc(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                       const uint32_t* zeros, int64_t M, int64_t K, int64_t N, int group,
                       uint16_t* y, const awq_plan* plan, void* stream);

/*
 * awq_linear_timed: awq_linear_ex that also records two hipEvent_t handles
 * (passed as void*, either may be NULL): `start_event` at the start of the
 * call's first kernel and `stop_event` at the end of its last kernel
 * (hipExtLaunchKernelGGL), so that hipEventElapsedTime gives the call's own
 * kernel time. A call is one kernel, or two for a plan with split_k > 1
 * (the GEMM or decode kernel, then the fixed-order reduction of its
 * partials).
 * For measurement only: not for use under stream capture.
 */
int awq_linear_timed(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                     const uint32_t* zeros, int64_t M, int64_t K, int64_t N, int group,
                     uint16_t* y, void* workspace, size_t workspace_bytes,
                     const awq_plan* plan, void* stream, void* start_event, void* stop_event);

/*
 * Gated MLP projection: the fused gate+up layer of a LLaMA-style MLP with its
 * activation applied on the fp32 sums. W [K, N] holds the gate projection in
 * columns 0 .. N/2-1 and the up projection in columns N/2 .. N-1 (the column
 * order of a fused gate+up weight is not printed on the pages; this is the
 * reading taken), and
 *     y[m, i] = fp16( silu(g) * u ),  g = (x . W)[m, i],  u = (x . W)[m, N/2 + i],
 *     silu(g) = g / (1 + exp(-g)),
 * y is [M, N/2], 8-byte aligned. N % 32 == 0. TinyChat ("Speed Benchmarks",
 * LLaMA-family models) fuses the small operators around its W4A16 kernels;
 * here the activation runs in the decode kernel's epilogue (one launch, no
 * [M, N] intermediate), or, with a K split, where the fp32 partial sums are
 * added (the gate and up sums at their own columns of the split_k * M * N
 * workspace). Plans, workspace and errors as for awq_linear; on the decode
 * path (M <= 32) the staged variant pairs the gate and up tiles in one
 * workgroup (M <= 16), the streamed and slab variants in one wave (tpw 2 or
 * 4: half gate, half up tiles).
 */
int awq_linear_silu_mul(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                        const uint32_t* zeros, int64_t M, int64_t K, int64_t N, int group,
                        uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);
int awq_linear_silu_mul_ex(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                           const uint32_t* zeros, int64_t M, int64_t K, int64_t N, int group,
                           uint16_t* y, void* workspace, size_t workspace_bytes,
                           const awq_plan* plan, void* stream, void* start_event, void* stop_event);
/* Plan and workspace of awq_linear_silu_mul (as awq_linear_plan and
 * awq_linear_workspace_bytes_ex). */
int awq_linear_silu_mul_plan(int64_t M, int64_t K, int64_t N, int group, awq_plan* plan);
int awq_linear_silu_mul_workspace_bytes(int64_t M, int64_t K, int64_t N, int group,
                                        const awq_plan* plan, size_t* bytes);

/*
 * W4A8-FP8 form of the layer. The TensorRT-LLM news page (Falcon-180B with
 * INT4 AWQ on one H200) has the AWQ kernels compute in FP8; the readings
 * taken (the page prints no arithmetic):
 *   - FP8 is OCP E4M3 (bias 7, largest finite 448, no infinities), rounding
 *     to nearest even;
 *   - activations are quantised per row (per token) at run time, each step
 *     one IEEE float32 operation: amax = max_k |x[m,k]|, inv = 448 / amax,
 *     code = E4M3(x * inv), sx[m] = amax / 448 (a zero row: codes 0, sx 0);
 *   - y[m,n] = fp16( sx[m] * sum_g s[g,n] * sum_{k in g} x8[m,k] * (q[k,n] - z[g,n]) ),
 *     the inner sums over one group on the FP8 matrix cores in fp32 (the
 *     products are exact), the rest in fp32.
 * The weights (qweight, scales, zeros) are those of awq_linear. group is
 * 32, 64 or a positive multiple of 128 (groups below 128 rows use one
 * 16x16x32 FP8 MFMA per 32-row block); K % group == 0, K % 128 == 0;
 * N % 8 == 0; M * K < 2^31.
 *
 * awq_quantize_act_fp8: x fp16 [M, K] (K % 128 == 0) -> x8 [M, K] E4M3 codes
 *   in the kernel's layout: within each 128-column block, the 8-column chunk
 *   c = 4j + h (columns 8c .. 8c+7, j, h = 0..3) is stored at chunk position
 *   4h + j; sx float32 [M]. x and x8 16-byte aligned.
 * awq_linear_w4a8: y fp16 [M, N] from fp16 x [M, K]: the activations are
 *   quantised into the workspace (awq_linear_w4a8_workspace_bytes bytes for
 *   the same plan, 256-byte aligned; it also holds split-K partials), then
 *   multiplied on workgroup tiles of 128 x 128 (plan tile 2) or 256 x 256
 *   (tile 3) with an optional K split (split_k, at most K/128 and 16); other
 *   plan fields must be 0; NULL or zero fields are chosen automatically.
 *   awq_linear_w4a8_ex records events at the start of its first kernel and
 *   the end of its last (either may be NULL); awq_linear_w4a8_plan fills in
 *   the plan a call would use.
 */
/* The activation quantiser of the W4A8-FP8 form (TensorRT-LLM news page: AWQ
 * kernels computing in FP8), as described above. */
int awq_quantize_act_fp8(const uint16_t* x, int64_t M, int64_t K, uint8_t* x8, float* sx, void* stream);
int awq_linear_w4a8_workspace_bytes(int64_t M, int64_t K, int64_t N, int group, const awq_plan* plan,
                                    size_t* bytes);
int awq_linear_w4a8_plan(int64_t M, int64_t K, int64_t N, int group, awq_plan* plan);
int awq_linear_w4a8(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                    const uint32_t* zeros, int64_t M, int64_t K, int64_t N, int group,
                    uint16_t* y, void* workspace, size_t workspace_bytes, void* stream);
int awq_linear_w4a8_ex(const uint16_t* x, const uint32_t* qweight, const uint16_t* scales,
                       const uint32_t* zeros, int64_t M, int64_t K, int64_t N, int group,
                       uint16_t* y, void* workspace, size_t workspace_bytes, const awq_plan* plan,
                       void* stream, void* start_event, void* stop_event);

/*
 * Fused decode-step attention. "TinyChat: Efficient and Lightweight Chatbot
 * with AWQ", section "Speed Benchmarks": in the generation stage every
 * operation of multi-head, grouped-query and multi-query attention (MHA / GQA
 * / MQA) runs in a single kernel, the positional embedding is fused into it,
 * and the key-value caches are allocated up front. The pages define neither
 * the attention nor the embedding; the readings taken are the textbook ones
 * of the LLaMA and Falcon models in that section:
 *
 *   For each sequence b, with L = lengths[b] tokens already cached, the new
 *   token's q, k, v are read from the QKV projection's output row qkv[b],
 *   laid out as [Hq query heads | Hkv key heads | Hkv value heads] with D
 *   values per head. q and k are rotated by the rotary embedding at position
 *   L: pair i (i < D/2) turns counter-clockwise by L * theta^(-2i/D), the
 *   pairs being (i, i + D/2) for AWQ_ROPE_HALF (LLaMA, Falcon) or (2i, 2i+1)
 *   for AWQ_ROPE_INTERLEAVED; AWQ_ROPE_NONE leaves them as they are. Query
 *   head h attends over the L cached keys of kv head h / (Hq / Hkv) and the
 *   new key with softmax(scale * q . k), scale = softmax_scale (0: 1/sqrt(D)),
 *   and out[b, h*D + d] = fp16(sum_j p_j v_j[d]). The rotated key, rounded
 *   to fp16, and the value are written to slot L of the caches (the new token
 *   attends to its key as stored).
 *
 * Arithmetic: rotation angles in fp64, rotations in fp32; products of fp16
 * operands (q rounded to fp16, probabilities rounded to fp16 before the value
 * product) summed in fp32; softmax in fp32 with the running maximum.
 *
 * Layouts (fp16 as uint16_t bits; device pointers, 16-byte aligned):
 *   qkv      B rows of qkv_stride elements (>= (Hq + 2 Hkv) D, multiple of 8)
 *   k_cache  [B, Hkv, capacity, D]: key element d of position j of (b, kv
 *            head h) at ((b*Hkv + h)*capacity + j)*D + d
 *   v_cache  [B, Hkv, capacity/32, D, 32]: tiles of 32 positions, d-major
 *            inside a tile; value element d of position j of (b, kv head h)
 *            at (((b*Hkv + h)*(capacity/32) + j/32)*D + d)*32 + j%32, so that
 *            the value product reads each 32-position block as one
 *            contiguous run of D*64 bytes
 *   lengths  int32 [B]
 *   out      [B, Hq*D]
 * Sizes: D = 64 or 128; Hq a multiple of Hkv; capacity a multiple of 32 (at
 * most 2^24); 0 <= max_cached < capacity. max_cached is a host-side bound on
 * lengths[b]: the launch covers that many cached positions. A sequence whose
 * lengths[b] is negative, above max_cached or not below capacity is skipped
 * on the device: its output row is set to NaN and the caches keep their
 * contents (the call still returns AWQ_OK).
 * Workspace: awq_attention_workspace_bytes() bytes, 256-byte aligned. The
 * caller zero-fills it once when it is allocated; every call leaves every
 * byte it used zero again (it holds per-unit completion counters, which
 * return to zero, and partial softmax states, which the merging workgroup
 * clears after reading them), so a buffer filled once serves later calls of
 * any shape that fits in it. Calls that share a workspace must not overlap
 * (one stream).
 * steps: 32-position blocks per wave (0: automatic); it sets how the cached
 * positions are split over workgroups and changes only the summation order.
 * B = 0 is a valid empty call.
 */
enum awq_rope_style { AWQ_ROPE_NONE = 0, AWQ_ROPE_HALF = 1, AWQ_ROPE_INTERLEAVED = 2 };

typedef struct awq_attn_desc {
  int64_t batch;         /* B                                                   */
  int64_t q_heads;       /* Hq                                                  */
  int64_t kv_heads;      /* Hkv (Hq % Hkv == 0; Hq == Hkv is MHA, Hkv == 1 MQA) */
  int64_t head_dim;      /* D: 64 or 128                                        */
  int64_t capacity;      /* cache slots per (sequence, kv head)                 */
  int64_t max_cached;    /* host bound on lengths[b]                            */
  int64_t qkv_stride;    /* elements between rows of qkv                        */
  int32_t rope_style;    /* awq_rope_style                                      */
  int32_t steps;         /* 0: automatic                                        */
  float rope_theta;      /* base of the rotation rates (> 0 unless NONE)        */
  float softmax_scale;   /* 0: 1/sqrt(D)                                        */
} awq_attn_desc;

/* Workspace bytes of awq_attention_decode for `desc` (the counters and states
 * described above; 0 for B = 0). */
int awq_attention_workspace_bytes(const awq_attn_desc* desc, size_t* bytes);
/* The work split a call with `desc` uses: workgroups per unit (a unit is a
 * sequence, kv head and tile of 16 query heads) and 32-position blocks per
 * wave. Either pointer may be NULL. */
int awq_attention_plan(const awq_attn_desc* desc, int32_t* workgroups_per_unit, int32_t* steps);
/* One generation step of attention (TinyChat README "Speed Benchmarks": fused
 * MHA/GQA/MQA with the positional embedding, pre-allocated key-value cache),
 * as described above. */
int awq_attention_decode(const awq_attn_desc* desc, const uint16_t* qkv, uint16_t* k_cache,
                         uint16_t* v_cache, const int32_t* lengths, uint16_t* out,
                         void* workspace, size_t workspace_bytes, void* stream);
/* awq_attention_decode with hipEvent_t handles recorded at the start and end
 * of its kernel, as in awq_linear_timed (either may be NULL). */
int awq_attention_decode_timed(const awq_attn_desc* desc, const uint16_t* qkv, uint16_t* k_cache,
                               uint16_t* v_cache, const int32_t* lengths, uint16_t* out,
                               void* workspace, size_t workspace_bytes, void* stream,
                               void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_MI355X_AWQ_H */
