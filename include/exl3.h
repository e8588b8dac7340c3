/*
 * exl3.h -- C ABI of the MI355X (gfx950) EXL3 trellis-quantized linear layer.
 *
 * Pages cited by title:
 *   "radiance_escha.py"      -- vLLM quantization method for escha (EXL3 trellis) W2 checkpoints on gfx1201.
 *                               Module docstring (forward formula), `_TILE`/`_HAD` constants,
 *                               `escha_linear_into`, `_ensure_scratch`, `EschaLinearMethod.apply`,
 *                               `process_weights_after_loading`.
 *   "vllm-quantpack 0.1.0"   -- wheel diff, exl3/linear.py: module docstring and `Exl3LinearMethod._forward`.
 *   "dspark/worker/exl3/bank.py" -- class `Exl3Bank` (expert bank layout, `allocate`, `views`, `tables`).
 *   "vLLM PR #190: [GG] Add EXL3 Trellis backend for rank-sliced MoE checkpoints" -- commit messages.
 *
 * The layer ("radiance_escha.py", module docstring):
 *     out[:, col0 : col0+OC] = bf16( Had128( Had128((x * s_in) * rin) @ W ) * rout * s_out )
 * where W = decode(code) is [IC, OC] and Had128 is the orthonormal Sylvester Walsh-Hadamard transform of
 * every consecutive 128-block (input side along IC, output side along OC).  rin is a pre-scale and rout a
 * post-scale; no bias is applied.
 *
 * Trellis layout (`_TILE = 16`, "code tensor is [IC//16, OC//16, 16*K]"): code[a][b][0 .. 16K) holds the
 * 16x16 tile W[16a .. 16a+16, 16b .. 16b+16) as a tail-biting 256K-bit stream (bit j = bit j%16 of word
 * j/16).  State i of a tile is the 16-bit window at stream bit i*K (circular, least significant bit
 * first); it sets W[16a + i%16][16b + i/16] to the fp16 number with bit pattern
 * ((state * 0x9E37) mod 2^16) & 0x8F80 | 0x3000.  The pages do not print EXL3's own codebooks; this one
 * is fixed here and checkpoints coded with another codebook decode to different values.
 *
 * Conventions (all entry points):
 *   - Every pointer is a device pointer unless stated otherwise; the caller owns every buffer.  The
 *     library never allocates, frees or synchronises, so each call is legal inside stream capture
 *     ("radiance_escha.py", `_ensure_scratch`: a lazy allocation inside the launch would land in graph
 *     capture).  `stream` is a hipStream_t (NULL = the legacy default stream).
 *   - Workspace: `ws` must hold at least the bytes the matching *_workspace_bytes() function returns,
 *     be 256-byte aligned, and be zero-filled once before its first use.  Kernels leave their counters
 *     zero again on exit, so later calls need no clearing.  One workspace serves one stream at a time:
 *     calls that may overlap (different streams) need different workspaces.
 *   - Host-side validation happens before any launch; a rejected call launches nothing and returns a
 *     negative status.  exl3_last_error() then names the offending argument (thread-local text).
 *   - M == 0 (or T == 0) is a valid no-op returning EXL3_OK ("radiance_escha.py", `escha_linear_into`).
 */
#ifndef EXL3_H
#define EXL3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EXL3_OK = 0,
  EXL3_EINVAL = -1,      /* bad shape, K, alignment, null pointer or flag */
  EXL3_EWORKSPACE = -2,  /* workspace missing or smaller than required */
  EXL3_EUNSUPPORTED = -3,/* valid request outside what the library implements */
  EXL3_ELAUNCH = -4      /* a kernel launch failed (message carries the HIP error) */
} exl3_status;

/* flags */
enum {
  EXL3_ACT_INT8 = 1u << 0,   /* per-row 8-bit activations: sc = max|xh| / 127, q = clamp(rne(xh / sc), +-127),
                                 Y = sc * (q . W); dispatched by M like the 16-bit path (the codes and scales
                                 are written by a pre-pass in either phase) */
  EXL3_FORCE_GEMV = 1u << 1, /* force the decode-phase (streaming split-K) kernel whatever M is */
  EXL3_FORCE_MFMA = 1u << 2, /* force the prefill-phase (tiled MFMA GEMM) kernel whatever M is */
  EXL3_GEMM_NO_SPLIT = 1u << 3, /* never split the GEMM's input features (exl3_gemm_splits): one fixed-order
                                 reduction per output element, so a row's result does not depend on M */
  EXL3_BATCH_INVARIANT = 1u << 4 /* a row's result depends on that row alone, at every M and across the
                                 decode/prefill crossover ("vLLM PR #190" commit message: the fused dense
                                 kernel's output does not change with the batch size).  The 16-bit path runs
                                 the decode-phase kernel at every M: its reduction order per output element
                                 (waves' feature ranges summed in wave order, then the input-feature splits
                                 in split order) does not depend on M, since every 16-row group of a launch
                                 is reduced alike and the split count is a function of (IC, OC, K) only.
                                 Costs nothing up to the crossover (exl3_gemv_max_rows); above it runs at the
                                 decode-phase kernel's rate, e.g. ~0.75 ms for a 5120 -> 7168 K=3
                                 projection at M=128 against ~0.04 ms on the GEMM.  The 8-bit path runs the
                                 unsplit GEMM (as EXL3_GEMM_NO_SPLIT).  Not with EXL3_FORCE_MFMA. */
};

/* Text of the last failure on the calling thread ("" if none). */
const char* exl3_last_error(void);

/* ABI version (major * 100 + minor). */
int exl3_version(void);

/* Largest M served by the decode-phase path (launches of up to 32 rows) when no FORCE flag is given,
 * for a call whose widest shard has OC output columns: 16 * clamp(10240 / OC, 2, 8), the measured
 * crossover against the (feature-split) MFMA GEMM over a 5120/17408 decoder's projections. */
int64_t exl3_gemv_max_rows(int64_t OC);

/* Number of input-feature splits the prefill-phase GEMM uses for M rows of an IC -> OC shard when no
 * FORCE flag is given: 1 once the shard has 1024 output tiles of 128 x 128 (one wave each fills the
 * chip), otherwise about 1024 / tiles, each split keeping at least 512 input features.  The splits'
 * fp32 partial tiles are summed in split order by a second launch, so the result is deterministic but
 * differs in rounding from the unsplit GEMM (EXL3_GEMM_NO_SPLIT), and a row's result depends on M
 * through the split count.  1 for invalid shapes. */
int exl3_gemm_splits(int64_t M, int64_t IC, int64_t OC);

/* Splits of the GEMM's tail round when exl3_gemm_splits is 1.  Blocks of 4 waves (128 rows x 512
 * columns) run 256 at a time; when the last round of a shard's blocks is at most half full, its blocks
 * (the last ones in launch order) run with their input features split this many ways after the other
 * blocks ran unsplit, so that round takes a fraction of the time; a second launch sums their partial
 * tiles in split order.  Those tiles differ in rounding from the unsplit GEMM.  1 when there is no such
 * tail (or with EXL3_GEMM_NO_SPLIT, which the library honours for both kinds of split). */
int exl3_gemm_tail_splits(int64_t M, int64_t IC, int64_t OC);

/* --------------------------------------------------------------------------------------------------
 * One projection written into its column slice ("radiance_escha.py", `escha_linear_into`: one escha
 * projection written into out[:, col0:col0+OC]; merged modules run one call per source tensor,
 * `EschaLinearMethod.apply`).
 *
 *   out    bf16 [M, ldo] row-major.  Only columns [col0, col0 + OC) are written; others are untouched.
 *   x      bf16 [M, IC] row-major, contiguous.
 *   code   int16 [IC/16, OC/16, 16K], contiguous, 16-byte aligned.
 *   s_in, rin    fp16 [IC];  rout, s_out   fp16 [OC].
 *   K      bits per weight, 1..8.
 * Requirements: IC % 128 == 0 and OC % 128 == 0 (the transform is blocked at 128, `create_weights`),
 * OC / 128 <= 4096, col0 >= 0, col0 + OC <= ldo, out/x/code 16-byte aligned, s_in/rin 4-byte aligned,
 * rout/s_out 2-byte aligned, IC*OC*K/8 < 2 GiB.
 * Precision: x * s_in * rin and the Hadamard in fp32, the rotated activations rounded once to fp16, fp16 x
 * fp16 products accumulated in fp32, output transform and scales in fp32, one round-to-nearest-even to
 * bf16.  M <= exl3_gemv_max_rows(OC) runs the decode-phase kernel, larger M the MFMA GEMM (the two agree
 * to rounding, not bitwise), split over the input features when the shard is small (exl3_gemm_splits).
 * For a given split count a row's result does not depend on the other rows; on the GEMM with
 * EXL3_GEMM_NO_SPLIT it does not depend on M at all.  Decode-phase launches of 5..32 rows rotate the
 * activations once per call into the workspace (16 or 32 rows x IC fp16 per distinct (s_in, rin)) before
 * the decode kernel; smaller ones rotate inside the kernel.  Both rotations give the same bits.
 * 8-bit path (EXL3_ACT_INT8): a pre-pass writes the row maxima and then the codes q as fp16 numbers, exact,
 * in the operand layout of the phase that runs (decode-phase launches of 1..4 rows form the same codes in
 * the kernel's own pre-pass from the row maxima), so the decode-phase kernel serves small M here too; every q * W product is exact in fp32, so the contraction is the integer dot product up
 * to fp32 summation; in both phases the row scale multiplies the result after the output Hadamard and
 * before rout * s_out.  The decode-phase path needs 16 or 32 rows x IC fp16 of codes, the row scales and
 * the row maxima (rows x IC/128 fp32) in the workspace per distinct (s_in, rin).
 * Returns EXL3_OK, EXL3_EINVAL, EXL3_EWORKSPACE, EXL3_EUNSUPPORTED, EXL3_ELAUNCH.
 * ------------------------------------------------------------------------------------------------ */
size_t exl3_linear_workspace_bytes(int64_t M, int64_t IC, int64_t OC, unsigned flags);

int exl3_linear_into(void* out, int64_t ldo, int64_t col0,
                     const void* x, int64_t M, int64_t IC,
                     const int16_t* code, int64_t OC, int K,
                     const void* s_in, const void* rin,
                     const void* rout, const void* s_out,
                     unsigned flags, void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------------------
 * Several shards of one merged projection in one call: every shard reads the same x and writes its own
 * column slice [col0_i, col0_i + OC_i) ("radiance_escha.py", module docstring: gate K=2 and up K=3 cannot
 * be one GEMM, each keeps its own code/rout/s_out; `apply`: one output buffer, each shard writes its own
 * columns).  The result is bitwise identical to one exl3_linear_into call per shard.
 *   shards    host array of n_shards descriptors (read during the call only); 1 <= n_shards <= 16.
 * Workspace: exl3_linear_multi_workspace_bytes with the same shard list.
 * ------------------------------------------------------------------------------------------------ */
typedef struct {
  const int16_t* code;   /* int16 [IC/16, OC/16, 16K] */
  int64_t OC;
  int32_t K;
  int32_t reserved;
  int64_t col0;
  const void* s_in;      /* fp16 [IC] */
  const void* rin;       /* fp16 [IC] */
  const void* rout;      /* fp16 [OC] */
  const void* s_out;     /* fp16 [OC] */
} exl3_shard;

size_t exl3_linear_multi_workspace_bytes(int64_t M, int64_t IC, int n_shards, const exl3_shard* shards,
                                         unsigned flags);

int exl3_linear_multi_into(void* out, int64_t ldo, const void* x, int64_t M, int64_t IC,
                           int n_shards, const exl3_shard* shards,
                           unsigned flags, void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------------------
 * The same call without a workspace argument, for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid allocation).  The workspace is a static
 * device array of exl3_static_scratch_bytes() (16 MiB) that the library holds on every GPU it runs on
 * until the process ends; nothing is allocated or freed per call.  A call whose workspace need
 * (exl3_linear_multi_workspace_bytes) exceeds that size launches nothing and returns EXL3_EWORKSPACE;
 * decode-phase calls of the usual shapes fit (the 4096 -> 2 x 14336 gate_up needs 3.8 MB at 16 rows, 7.6 at 32),
 * most prefill-phase calls do not.
 * The first call on a device (with that device current) looks up the array's address and clears its
 * counter head with a kernel on `stream`; make that first call outside stream capture.  Every call on a
 * device shares the one array: calls that may overlap on one device (other streams or threads without
 * ordering between them) race.  Results are bitwise those of exl3_linear_multi_into.
 * ------------------------------------------------------------------------------------------------ */
size_t exl3_static_scratch_bytes(void);

int exl3_linear_multi_into_static(void* out, int64_t ldo, const void* x, int64_t M, int64_t IC,
                                  int n_shards, const exl3_shard* shards, unsigned flags, void* stream);

/* --------------------------------------------------------------------------------------------------
 * MoE expert bank (layout of "dspark/worker/exl3/bank.py", `Exl3Bank` and `allocate`): the slot order
 * sorts the experts by bit width, so equal-K experts occupy one run of slots; one int16 array holds each
 * slot's w1 words followed by its w3 words, a second one each slot's w2 words, and the fp16 sign/scale
 * vectors are indexed by slot.
 *
 *   out[t] = bf16( sum_j topk_w[t, j] * E_{topk_ids[t, j]}(x[t]) )          (j in top-k order)
 *   E_e(v) = L_w2( silu(L_w1(v)) * L_w3(v) ),   silu(h) = h / (1 + exp(-h)),
 *   L_P(v) = svh * Had128( Had128(v * suh) @ W_P )      (suh plays s_in*rin, svh plays rout*s_out)
 *
 * Slot p (= perm[logical id]) holds w1 at w13 + off_w1[p] as [H/16, I/16, 16 k_gu], w3 at w13 + off_w3[p]
 * (same shape), w2 at w2 + off_w2[p] as [I/16, H/16, 16 k_d]; offsets count int16 elements and each
 * must make the address 16-byte aligned.  Groups are contiguous slot ranges [lo, hi) sharing (k_gu, k_d)
 * ("bank.py", `tables`: one GroupTables per K group); they must cover slots 0 .. E-1 in order.
 * The device tables (perm, off_w*) are trusted: the host cannot read them without synchronising.  A perm
 * entry outside [0, E) drops the expert like an out-of-range id; offsets must address the banks.
 * Limits: 1 <= E <= 1024, H and I multiples of 128 up to 65536, 1 <= n_groups <= 64, k_gu, k_d in 1..8,
 * 1 <= topk <= E, T * topk <= 2^24; w13/w2, w13_suh, x and out 16-byte aligned, other vectors 2-byte aligned, offset
 * tables 8-byte and perm/topk arrays 4-byte aligned.
 * Precision: each projection as in exl3_linear_into (fp16 operands, fp32 accumulation); h1, h3 and
 * silu(h1) * h3 stay in fp32 until w2's rotation rounds them to fp16; the top-k sum is taken in fp32 in
 * top-k order with one bf16 rounding.  Deterministic: every reduction has a fixed order.
 * Workspace: exl3_moe_workspace_bytes(bank, T, topk, flags); it holds the per-(token, expert) rotated
 * activations, w2 operands and expert outputs, so it grows linearly with T * topk.
 * ------------------------------------------------------------------------------------------------ */
typedef struct { int32_t k_gu, k_d, lo, hi; } exl3_group;

typedef struct {
  int32_t E, H, I;                     /* experts, hidden, intermediate (multiples of 128) */
  int32_t n_groups;                    /* 1 .. 64 */
  const int16_t* w13;                  /* flat int16 bank of w1 | w3 */
  const int16_t* w2;                   /* flat int16 bank of w2 */
  const void* w13_suh;                 /* fp16 [E, 2, H]  (slot order) */
  const void* w13_svh;                 /* fp16 [E, 2, I] */
  const void* w2_suh;                  /* fp16 [E, I] */
  const void* w2_svh;                  /* fp16 [E, H] */
  const int64_t* off_w1;               /* device int64 [E], slot order */
  const int64_t* off_w3;               /* device int64 [E] */
  const int64_t* off_w2;               /* device int64 [E] */
  const int32_t* perm;                 /* device int32 [E]: logical expert -> slot */
  const exl3_group* groups;            /* HOST array [n_groups], covering slots 0 .. E-1 in order */
} exl3_bank;

size_t exl3_moe_workspace_bytes(const exl3_bank* bank, int64_t T, int topk, unsigned flags);

/*   out      bf16 [T, H];  x  bf16 [T, H]
 *   topk_ids int32 [T, topk] logical expert ids in [0, E) (device);  topk_w float32 [T, topk] (device).
 * An id outside [0, E) is ignored (contributes nothing).
 * Plans: below 128 routed pairs per expert on average (T * topk < 128 E) the call streams every expert's
 * weights once per chunk of up to 32 of its rows (the decode-sized plan); from there on it runs grouped
 * tiles of 64 rows x 128 columns on MFMA (the prefill plan), as long as T * topk * (max(H, I) + 64) * 2 <
 * 2^31.  flags: 0, EXL3_FORCE_GEMV (the decode-sized plan at any T) or EXL3_FORCE_MFMA (the prefill plan at
 * any T; EXL3_EUNSUPPORTED past the size limit); the two are exclusive.  Both plans give the same results
 * up to fp32 summation order inside each projection.  EXL3_ACT_INT8 answers EXL3_EUNSUPPORTED.
 * Returns EXL3_OK / EXL3_EINVAL / EXL3_EWORKSPACE / EXL3_EUNSUPPORTED / EXL3_ELAUNCH. */
int exl3_moe_bank_forward(void* out, const void* x, int64_t T,
                          const int32_t* topk_ids, const float* topk_w, int topk,
                          const exl3_bank* bank, unsigned flags, void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------------------------------------------------------
 * Dense MLP block ("vllm-quantpack 0.1.0", exl3/linear.py module docstring: gate and up are two shards of
 * one fused gate_up layer, each its own EXL3 tensor of any K, whose outputs are concatenated; the model's
 * activation takes silu(gate) * up and feeds down_proj):
 *
 *   gu  = [gate(x) | up(x)]          one exl3_linear_multi_into call, bf16 [M, 2I] in the workspace
 *   h   = bf16(silu(g) * u)          as exl3_silu_mul computes it (fp32 arithmetic)
 *   out = down(h)                    as one exl3_linear_into call on h, bf16 [M, H]
 * down's activation pre-pass reads g and u and forms h itself, so h is not written to memory (except on
 * the 8-bit path, whose pre-pass reads it).
 *
 *   out   bf16 [M, H] row-major, 16-byte aligned;  x  bf16 [M, H] row-major, 16-byte aligned.
 *   gate, up   shard descriptors over IC = H with OC = I (their col0 is ignored: gate fills columns
 *              [0, I) of gu and up [I, 2I));  down   a shard descriptor over IC = I with OC = H (col0 ignored).
 *   flags      as for exl3_linear_into, applied to every projection.
 *   ws         exl3_mlp_workspace_bytes(M, H, I, gate, up, flags) bytes, 256-byte aligned, zeroed once
 *              before first use (the projections' counter area sits at its start); the calls it makes are
 *              stream-ordered, so they share it.
 * H and I positive multiples of 128.  The result is bitwise identical to the three calls made one by one.
 * M == 0 is a no-op.  Returns EXL3_OK / EXL3_EINVAL / EXL3_EWORKSPACE / EXL3_EUNSUPPORTED / EXL3_ELAUNCH
 * (from the first step that fails; the message names the argument).
 * ------------------------------------------------------------------------------------------------ */
size_t exl3_mlp_workspace_bytes(int64_t M, int64_t H, int64_t I, const exl3_shard* gate, const exl3_shard* up,
                                unsigned flags);
int exl3_mlp_forward(void* out, const void* x, int64_t M, int64_t H, int64_t I, const exl3_shard* gate,
                     const exl3_shard* up, const exl3_shard* down, unsigned flags, void* ws, size_t ws_bytes,
                     void* stream);

/* The block's activation on its own: h bf16 [M, I] (16-byte aligned, row-major) = bf16(silu(g) * u) with
 * g = gu[m, j] and u = gu[m, I + j] of a bf16 [M, 2I] input (16-byte aligned); silu(g) = g / (1 + exp(-g))
 * in fp32, one round-to-nearest-even to bf16.  I a positive multiple of 8; M == 0 is a no-op.
 * Returns EXL3_OK / EXL3_EINVAL / EXL3_ELAUNCH. */
int exl3_silu_mul(void* h, const void* gu, int64_t M, int64_t I, void* stream);

/* --------------------------------------------------------------------------------------------------
 * int8 embedding rows gathered by token id and dequantized ("vllm-quantpack 0.1.0", exl3/embedding.py,
 * `Exl3EmbeddingMethod.embedding`: the table is kept as int8 codes plus one scale per row; only the
 * requested rows are converted to the scale's dtype and scaled, and no bf16 copy of the table exists).
 *
 *   out    bf16 [T, H] row-major, 16-byte aligned: out[t, :] = bf16(table[ids[t], :] * scale[ids[t]]).
 *   table  int8 [V, H] row-major, 16-byte aligned.
 *   scale  bf16 [V], one scale per row.
 *   ids    int32 [T] device array of token ids; ids outside [0, V) give zero rows (the page's
 *          tensor-parallel cut masks the ids a rank does not hold).
 * Requirements: V >= 1, H a positive multiple of 16.  The product of an int8 code and a bf16 scale is
 * exact in fp32, so the result is bit-exact: one round-to-nearest-even to bf16.  T == 0 is a no-op.
 * Returns EXL3_OK, EXL3_EINVAL, EXL3_ELAUNCH.
 * ------------------------------------------------------------------------------------------------ */
int exl3_embed_int8(void* out, const int8_t* table, const void* scale, int64_t V, int64_t H, const int32_t* ids,
                    int64_t T, void* stream);

/* --------------------------------------------------------------------------------------------------
 * The same int8 table as the output head (tied embedding / lm_head; "vllm-quantpack 0.1.0",
 * exl3/embedding.py, `Exl3EmbeddingMethod.apply`: the table is multiplied by its row scales in bf16, so
 * every weight is rounded once, then mapped linearly onto x).
 *
 *   out    bf16 [M, V] with row stride ldo (elements); written 8 bytes at a time when out is 8-byte
 *          aligned and ldo a multiple of 4, element by element otherwise:
 *          out[m, v] = bf16(sum_h x[m, h] * bf16(table[v, h] * scale[v])), summed in fp32.
 *   x      bf16 [M, H] row-major, 16-byte aligned.
 *   table  int8 [V, H] row-major, 16-byte aligned;  scale  bf16 [V].
 * Requirements: V >= 1; H a positive multiple of 64; ldo >= V.  No bias (a tied head
 * has none).  M == 0 is a no-op.  Every 64 rows of x stream the table once (one launch per 64 rows).
 * The weights are the page's bf16(q * s) bit for bit; the sum order differs from any library GEMM, so
 * results agree with an exact sum to the bf16 rounding of the output.
 * Returns EXL3_OK, EXL3_EINVAL, EXL3_ELAUNCH.
 * ------------------------------------------------------------------------------------------------ */
int exl3_lm_head_int8(void* out, int64_t ldo, const void* x, int64_t M, const int8_t* table, const void* scale,
                      int64_t V, int64_t H, void* stream);

/* --------------------------------------------------------------------------------------------------
 * Test hook: the decoded weight, fp16 [IC, OC] row-major, produced by the same device decode routine
 * the GEMM kernels use.  IC, OC multiples of 16; K in 1..8.
 * ------------------------------------------------------------------------------------------------ */
int exl3_decode_tiles(void* w_out, const int16_t* code, int64_t IC, int64_t OC, int K, void* stream);

/* Test hook: the rotated activations the GEMM kernels consume for x [M, IC] (fp16 [M, IC], natural
 * feature order) or, with EXL3_ACT_INT8, int8 codes [M, IC] into q_out and float32 row scales [M] into
 * scale_out.  Same kernels as exl3_linear_into. */
int exl3_rotate_activations(void* q_out, float* scale_out, const void* x, int64_t M, int64_t IC,
                            const void* s_in, const void* rin, unsigned flags, void* stream);

/* --------------------------------------------------------------------------------------------------
 * Measurement hooks, not part of the layer: what the chip delivers, as secondary roofline denominators
 * beside the published peaks (8 TB/s HBM; 2.5 PFLOP/s dense f16; 5 POP/s dense int8).
 *   exl3_probe_read   reads `bytes` (a multiple of 16) at `src` (16-byte aligned) once with 16-byte loads
 *                     over `blocks` workgroups of 256 threads, 4 (variant 0) or 8 (variant 1; variant 2:
 *                     non-temporal) loads in flight per thread; sink: uint32 [blocks] (an XOR per block).
 *   exl3_probe_mfma   `blocks` workgroups of 4 waves, each wave issuing back-to-back independent MFMAs for
 *                     `iters` iterations: kind 0 f16 16x16x32 (8 per iteration, 16384 FLOP each), kind 1
 *                     f16 32x32x16 (4, 32768 FLOP each), kind 2 i8 16x16x64 (8, 32768 OP each), kind 3 i8
 *                     32x32x32 (4, 65536 OP each); sink: float [blocks * 256].
 * Operations per call: blocks * 4 * iters * 131072 for kinds 0 and 1, * 262144 for kinds 2 and 3.
 * Return EXL3_OK / EXL3_EINVAL / EXL3_ELAUNCH.
 * ------------------------------------------------------------------------------------------------ */
int exl3_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, int variant, void* stream);
int exl3_probe_mfma(float* sink, int kind, int iters, int blocks, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* EXL3_H */
