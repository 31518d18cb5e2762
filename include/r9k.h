/*
 * r9k: block-scaled fp8 GEMMs for one AMD Instinct MI355X (gfx950).
 *
 * C ABI of libr9k.so.  What the library computes is the dense fp8 block GEMM
 * of LLM decode and prefill described on the r9700-stack release pages:
 *   - release v0.3.1, "What changed for someone running it": the dense fp8
 *     block GEMM r9k_gemm_fp8_block_qa, whose per-token-group-128 activation
 *     quant runs inside the GEMM's A-load with operands bit-identical to the
 *     split form (a separate quant launch, then the GEMM);
 *   - release v0.3.2, same section: fp8 kernels for up to 255 rows and the
 *     tiled fp8 GEMMs above that; weights quantised once at load;
 *   - release v0.3.3, same section: the fused MoE decode path (silu(gate)*up in
 *     the gate_up GEMM's epilogue, the fp8 row quant in the down GEMM's A-load),
 *     bit-identical to the three-launch path.
 *
 * Number formats (the workload's stated rules; the pages say only "fp8"):
 *   fp8   = OCP e4m3fn codes (uint8_t), largest finite value 448;
 *   bf16  = uint16_t bit patterns (the top half of an IEEE binary32);
 *   scale = fp32.
 * Group quantisation rule, used for activations (a row's 128 consecutive K
 * values) and weights (a 128x128 block): s = max(amax, 1e-10f) / 448 in fp32,
 * code = e4m3(fp32(a / s)), rounding to nearest even and saturating at +-448.
 * The GEMM computes C[m,n] = bf16( sum_g P(m,n,g) * as[m,g] * ws[n/128,g] ),
 * P = sum over the group's 128 k of dec(aq[m,k]) * dec(w[n,k]), accumulated in
 * fp32, rounded to bf16 with ties to even.
 *
 * Layouts: every tensor is dense row-major with no strides.
 *   A  [M][K] bf16        Aq [M][K] fp8     As [M][K/128] fp32
 *   W  [N][K] fp8         Ws [N/128][K/128] fp32        (out x in)
 *   C  [M][N] bf16
 * K and N must be multiples of 128.  Every pointer passed to a compute call is
 * a device pointer on the current HIP device; every base pointer must be 16-byte
 * aligned.  `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *
 * Ownership and behaviour common to every call:
 *   - the caller owns every buffer, including workspaces; the library never
 *     allocates device memory, never synchronises and never reads device data
 *     on the host;
 *   - calls are asynchronous on `stream` and capturable in a HIP graph; launch
 *     grids depend only on the shapes, never on device data;
 *   - arguments are checked on the host before any launch; a failed check
 *     returns a negative code and launches nothing;
 *   - M == 0 (or T == 0, n == 0) returns R9K_OK without launching;
 *   - faults inside a kernel surface at the caller's next synchronisation;
 *   - unchecked precondition: inputs are finite.
 */
#ifndef R9K_H
#define R9K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every function declared here is exported from libr9k.so; the library's
 * internal symbols are not (it is built with hidden visibility). */
#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility push(default)
#endif

#define R9K_ABI_VERSION 8

/* Return codes: 0 or negative, as the pages' kernels return them (release
 * v0.3.0, its validation record: a test failing "with the kernel's -7").
 * The values below are this library's own. */
#define R9K_OK 0
#define R9K_ERR_NULLPTR (-1)   /* a required pointer is NULL */
#define R9K_ERR_SHAPE (-2)     /* a size is out of range (see each call) */
#define R9K_ERR_ALIGN (-3)     /* a base pointer is not 16-byte aligned */
#define R9K_ERR_DEVICE (-4)    /* no HIP device, or the current device is not gfx950 */
#define R9K_ERR_LAUNCH (-5)    /* a kernel launch failed (hipGetLastError) */
#define R9K_ERR_WORKSPACE (-6) /* the workspace is smaller than the query returned */
#define R9K_ERR_ARG (-7)       /* an enumerated argument has an unknown value */

/* The ABI version this library implements (R9K_ABI_VERSION; 4 added the MoE
 * routing and the shared-expert fold, 5 the bf16-activation variant, 6 the
 * mid-width kernel in the plan query, 7 the allocation-free GEMM entry point, 8 the tiled-plan
 * control and R9K_ENGINE_SPLITK).  Callers refuse
 * a library whose version differs from the header they were built against:
 * the convention of the pages' plugin, which refuses an older libr9k.so
 * (release v0.2.2, "Upgrading").  Host only; cannot fail. */
int r9k_abi_version(void);

/* Static text for a return code (the codes above; release v0.3.0's validation
 * record for the convention); never NULL, also for unknown codes.  Host only. */
const char *r9k_strerror(int code);

/* ------------------------------------------------------------------------ */
/* Quantisation                                                              */
/* ------------------------------------------------------------------------ */

/* Per-token group-128 activation quant (the split form's first launch, and the
 * definition the fused A-load reproduces bit for bit; release v0.3.1, "What
 * changed for someone running it").
 *   a  [M][K] bf16 in; aq [M][K] fp8 out; as [M][K/128] fp32 out.
 * Errors: NULLPTR; SHAPE if M < 0, K <= 0 or K % 128 != 0; ALIGN; DEVICE; LAUNCH. */
int r9k_quant_act(const uint16_t *a, int64_t M, int64_t K, uint8_t *aq, float *as, void *stream);

/* Weight quant at load time, one fp32 scale per 128x128 block (release v0.3.2,
 * "What changed for someone running it": weights quantised once, bf16 copies
 * freed).  w [N][K] bf16 in; wq [N][K] fp8 out; ws [N/128][K/128] fp32 out.
 * Errors: NULLPTR; SHAPE if N or K <= 0 or not multiples of 128; ALIGN;
 * DEVICE; LAUNCH. */
int r9k_quant_weight(const uint16_t *w, int64_t N, int64_t K, uint8_t *wq, float *ws, void *stream);

/* Elementwise fp32 -> e4m3fn with the library's device encoder: round to
 * nearest even, saturate at +-448 (inf too), sign of zero kept.  NaN inputs
 * give an unspecified code.  x [n] fp32 in; codes [n] out.
 * Errors: NULLPTR; SHAPE if n < 0; ALIGN; DEVICE; LAUNCH. */
int r9k_encode_e4m3(const float *x, int64_t n, uint8_t *codes, void *stream);

/* ------------------------------------------------------------------------ */
/* Dense block-scaled GEMM                                                   */
/* ------------------------------------------------------------------------ */

/* Workspace bytes that r9k_gemm_fp8_block and r9k_gemm_fp8_block_qa need for
 * this shape, under any dispatch setting (release v0.3.1, "What changed for
 * someone running it": the split form's separate quant launch writes the
 * activation codes somewhere; release v0.3.2, same section: the tiled GEMMs
 * above the decode widths quantise their activations).  0 for M = 0.
 * Host only; touches no device.
 * The workspace holds the activation codes and scales of a call that
 * quantises once before the GEMM (or the transposed scales the tiled and
 * mid-width kernels read), and the fp32 partial sums of a K split (decode,
 * mid-width, skinny and tiled kernels); every call writes what it reads, so the contents
 * need no initialisation.  Calls that share a workspace must not overlap in time
 * (same stream, or ordered by events).
 * Errors: NULLPTR (bytes); SHAPE as for the GEMM. */
int r9k_gemm_fp8_block_workspace(int64_t M, int64_t K, int64_t N, size_t *bytes);

/* Block GEMM on pre-quantised activations: the split form, selected on the
 * pages by turning the fused quant off (release v0.3.1), and the bitwise
 * reference for the fused form.
 *   aq [M][K] fp8, as [M][K/128] fp32, w [N][K] fp8, ws [N/128][K/128] fp32
 *   -> c [M][N] bf16.
 * Errors: NULLPTR; SHAPE if M < 0, K or N <= 0, or K, N not multiples of 128;
 * ALIGN; WORKSPACE; DEVICE; LAUNCH. */
int r9k_gemm_fp8_block(const uint8_t *aq, const float *as, int64_t M, int64_t K, const uint8_t *w,
                       const float *ws, int64_t N, uint16_t *c, void *workspace, size_t ws_bytes,
                       void *stream);

/* The fused form r9k_gemm_fp8_block_qa (release v0.3.1): bf16 activations are
 * quantised per token in groups of 128 inside the GEMM, with codes and scales
 * bit-identical to r9k_quant_act; the result is bit-identical to
 * r9k_quant_act followed by r9k_gemm_fp8_block under the same dispatch.
 * The dispatcher picks the engine by M (release v0.3.2: the decode kernels to
 * 255 rows, the tiled GEMMs above).  Under R9K_ENGINE_AUTO:
 *   M > skinny_max_m (default 255)       -> the LDS-tiled MFMA engine;
 *   else, where the decode kernel covers all of K in each CTA (up to 64 rows,
 *   enough column tiles to fill the chip) -> the decode kernel, with the
 *   activation quant in its A-load, one launch; from 17 rows only where its
 *   estimated time (the busiest compute unit's weight bytes and repeated
 *   quant) is below the mid-width kernel's (that unit's bytes of codes);
 *   else from 17 rows on -> the mid-width kernel on activations quantised
 *   once per call (a quant launch, then the GEMM launch): all of K per CTA,
 *   or up to 64 rows at K >= 8192 a K split whose fp32 partials a reduce
 *   launch sums in ascending split order; except above 64 rows where K >= 8192
 *   with N * K > 2^24, or where ceil(M / 64) * (N / 64) > 256 (its 64 x 64
 *   blocks would need more than one CTA per compute unit), which take the
 *   tiled engine;
 *   else the decode kernel with a K split (partials summed by a second launch);
 *   else, from 8 rows, the mid-width kernel with its K split; else the split-K
 *   skinny kernel (large K and N below 8 rows).
 * r9k_gemm_fp8_block_plan names the kernel a shape runs.
 *   a [M][K] bf16, w [N][K] fp8, ws [N/128][K/128] fp32 -> c [M][N] bf16.
 * Errors: as r9k_gemm_fp8_block. */
int r9k_gemm_fp8_block_qa(const uint16_t *a, int64_t M, int64_t K, const uint8_t *w, const float *ws,
                          int64_t N, uint16_t *c, void *workspace, size_t ws_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the fused
 * GEMM r9k_gemm_fp8_block_qa (packed = 0) or r9k_gemm_fp8_block_qa_packed
 * (packed = 1) with the same arguments and result bits, but no workspace
 * argument.  Its scratch is a device array inside the library, of
 * R9K_NOALLOC_SCRATCH_BYTES on each GPU the call runs on, held until the
 * process ends; the call allocates nothing (no hipMalloc, no library
 * allocation).  Shapes whose workspace (r9k_gemm_fp8_block_workspace) exceeds
 * that size are rejected.  Every call on one GPU shares the one array and
 * leaves its contents behind (nothing in it needs to start at zero): calls on
 * one GPU that overlap in time, on different streams or threads, race and give
 * wrong results; order them (one stream, or events).
 * Errors: NULLPTR; SHAPE as r9k_gemm_fp8_block_qa; ARG if packed is not 0 or 1;
 * ALIGN; WORKSPACE if the shape needs more than R9K_NOALLOC_SCRATCH_BYTES;
 * DEVICE (also if the scratch's address cannot be taken); LAUNCH. */
#define R9K_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int r9k_gemm_fp8_block_qa_noalloc(const uint16_t *a, int64_t M, int64_t K, const uint8_t *w, const float *ws,
                                  int64_t N, uint16_t *c, int packed, void *stream);

/* Fragment-order weights.  The r9700-stack release v0.3.1 notes ("What
 * changed for someone running it") keep fragment-order copies of the fp8
 * decode weights; this is that copy for gfx950's 16x16x128 fp8 MFMA.  The
 * codes and scales are unchanged (same values, same [N/128][K/128] scales);
 * only the byte order of W differs: for 16-row tile t = n / 16 and K-group
 * g = k / 128, the 2 KiB block at byte (t * K/128 + g) * 2048 holds, at
 * h * 1024 + 16 * l (h = 0, 1; l = 0..63), the 16 bytes of row 16 t + l % 16
 * starting at column 128 g + 64 h + 16 (l / 16).  A 16-row tile's groups are
 * thus consecutive, and every 16-byte load instruction of the GEMMs reads
 * 1 KiB of consecutive bytes.  Pack once at load time, after r9k_quant_weight.
 *   wq [N][K] fp8 row-major -> wp [N*K] fp8 in fragment order (same size).
 * Errors: NULLPTR; SHAPE if N or K is not a positive multiple of 128; ALIGN;
 * ARG if wp overlaps wq (no in-place packing); DEVICE; LAUNCH. */
int r9k_pack_weight(const uint8_t *wq, int64_t N, int64_t K, uint8_t *wp, void *stream);

/* r9k_gemm_fp8_block and r9k_gemm_fp8_block_qa on fragment-order weights wp
 * (r9k_pack_weight); same arguments otherwise and the same workspace query.
 * The result is the row-major calls' on the unpacked weights bit for bit when
 * both run the same launch; at decode widths the planner may slice K
 * differently for each layout (its fastest launch), and then the fp32 partial
 * sums are added in another order, so that a few outputs differ by one bf16
 * ulp.  r9k_gemm_fp8_block_plan reports the kernel and K split of each.
 * Errors: as the row-major calls. */
int r9k_gemm_fp8_block_packed(const uint8_t *aq, const float *as, int64_t M, int64_t K, const uint8_t *wp,
                              const float *ws, int64_t N, uint16_t *c, void *workspace, size_t ws_bytes,
                              void *stream);
int r9k_gemm_fp8_block_qa_packed(const uint16_t *a, int64_t M, int64_t K, const uint8_t *wp, const float *ws,
                                 int64_t N, uint16_t *c, void *workspace, size_t ws_bytes, void *stream);

/* Dispatch control (release v0.3.2, "What changed for someone running it":
 * the fp8 decode kernels are used to 255 rows, a setting that restores the
 * earlier boundary, and the tiled fp8 GEMMs above it).  skinny_max_m: the
 * largest M the skinny engine takes (default 255, the pages' boundary; env
 * R9K_FP8_SKINNY_MAXM).  engine:
 * R9K_ENGINE_AUTO (by M), R9K_ENGINE_SKINNY or R9K_ENGINE_TILED (forced, for
 * tests; env R9K_FP8_ENGINE=auto|skinny|tiled), or R9K_ENGINE_SPLITK: up to
 * skinny_max_m rows, the split-K skinny kernel itself, which the weight-
 * streaming engine otherwise takes only where neither the decode nor the
 * mid-width kernel fits (tests and tuning).  The setting is process-wide;
 * change it only while no GEMM call is being issued.
 * Errors: SHAPE if skinny_max_m < 0; ARG for an unknown engine. */
#define R9K_ENGINE_AUTO 0
#define R9K_ENGINE_SKINNY 1
#define R9K_ENGINE_TILED 2
#define R9K_ENGINE_SPLITK 3
int r9k_set_dispatch(int skinny_max_m, int engine);
int r9k_get_dispatch(int *skinny_max_m, int *engine);

/* Tiled-engine plan control (release v0.3.0, "What changed for someone
 * running it": the tiled fp8 GEMMs of prefill widths), for tuning and tests:
 * every later call that runs the tiled engine uses this tile shape and K
 * split.  shape: R9K_TILE_AUTO (the planner's choice) or one of the CTA tiles
 * rows x columns below; ksplit: 0 (the planner's) or the number of CTAs that
 * share one output tile along K (clamped to K/128 by the call; the 256 x 256
 * tile takes none, and a forced split is ignored for it).  The environment
 * variables R9K_TILED_CFG (c, b, 1, 2 for the four tiles) and R9K_TILED_KSPLIT
 * give the initial values.  The setting is process-wide, changes the
 * workspace a shape needs (query again after a change), and must change only
 * while no GEMM call is being issued.
 * Errors: ARG for an unknown shape or a negative ksplit; NULLPTR (get). */
#define R9K_TILE_AUTO 0
#define R9K_TILE_256X256 1
#define R9K_TILE_256X128 2
#define R9K_TILE_128X64 3
#define R9K_TILE_256X64 4
int r9k_set_tiled_plan(int shape, int ksplit);
int r9k_get_tiled_plan(int *shape, int *ksplit);

/* The bf16-activation variant at decode widths (release v0.3.1, "What changed
 * for someone running it": the decode GEMMs of fp8 weights run as bf16
 * matrix products against the unquantised activations), with the weight block
 * scales applied per 128-K group:
 *   C[m][n] = bf16( sum_g ws[n/128][g] * sum_{k in g} a[m][k] * dec(w[n][k]) ),
 * fp32 accumulation.  No activation quant: a [M][K] bf16 is used as given.
 * w [N][K] codes (row-major) and ws [N/128][K/128] as for r9k_gemm_fp8_block.
 * No workspace; every CTA covers all of K.
 * Errors: NULLPTR; SHAPE if M < 0 or M > 16, if K or N is not a positive
 * multiple of 128, or if K/128 is not wk * gs with wk <= 8 and gs one of 1, 2,
 * 4, 8, 16 (every K/128 up to 8; even ones up to 16; multiples of 4 up to 32,
 * of 8 up to 64, of 16 up to 128: K = 4096, 7168 and 14336 among them);
 * ALIGN; DEVICE; LAUNCH.  M = 0 launches nothing. */
int r9k_gemm_fp8_block_bf16a(const uint16_t *a, int64_t M, int64_t K, const uint8_t *w, const float *ws, int64_t N,
                             uint16_t *c, void *stream);

/* r9k_gemm_fp8_block_bf16a on fragment-order weights (r9k_pack_weight); the
 * same result bits.  Errors: as r9k_gemm_fp8_block_bf16a. */
int r9k_gemm_fp8_block_bf16a_packed(const uint16_t *a, int64_t M, int64_t K, const uint8_t *wp, const float *ws,
                                    int64_t N, uint16_t *c, void *stream);

/* The kernel a GEMM call of this shape runs under the current dispatch
 * setting (host only, launches nothing, needs no device): kernel receives
 * R9K_KERNEL_DECODE (the whole-row weight-streaming kernel of the decode
 * widths), R9K_KERNEL_SKINNY (the split-K skinny kernel), R9K_KERNEL_TILED
 * (the LDS-tiled MFMA GEMM), R9K_KERNEL_MID (the mid-width kernel, 17 to 255
 * rows) or R9K_KERNEL_NONE (M = 0: nothing is launched);
 * ksplit receives the number of CTAs that share one output tile along K
 * (1: no K split, and no reduction launch follows).  packed (0 or 1) says
 * whether the weight is in the fragment order of r9k_pack_weight; the same
 * answer holds with and without the activation quant in the call.
 * Errors: NULLPTR (kernel, ksplit); SHAPE as for r9k_gemm_fp8_block; ARG if
 * packed is neither 0 nor 1. */
#define R9K_KERNEL_NONE 0
#define R9K_KERNEL_DECODE 1
#define R9K_KERNEL_SKINNY 2
#define R9K_KERNEL_TILED 3
#define R9K_KERNEL_MID 4
int r9k_gemm_fp8_block_plan(int64_t M, int64_t K, int64_t N, int packed, int *kernel, int *ksplit);

/* ------------------------------------------------------------------------ */
/* MoE decode                                                                */
/* ------------------------------------------------------------------------ */

/* Workspace bytes for r9k_moe_fp8_decode (host only): the intermediates of
 * release v0.3.3's three-launch path (gu, h and its codes and scales, y), which
 * the fused path partly keeps in registers.  Needs no initialisation; calls
 * sharing one must not overlap in time.
 * Errors: NULLPTR (bytes); SHAPE as for the call. */
int r9k_moe_fp8_decode_workspace(int64_t T, int64_t H, int64_t E, int64_t I, int64_t topk, size_t *bytes);

/* Routed MoE decode (release v0.3.3, "What changed for someone running it").
 * For token t and slot j, expert e = topk_ids[t][j]:
 *   gu  = bf16(block GEMM of quant(x[t]) against w13[e])    rows [0,I) gate, [I,2I) up
 *   h   = bf16(silu(gate) * up)                              fp32 arithmetic
 *   y   = block GEMM of quant(h) (group 128 along I) against w2[e], fp32
 *   out[t] = bf16(sum_j topk_w[t][j] * y(t,j)), j ascending.
 * A slot whose id lies outside [0,E) contributes nothing; ids need not be
 * distinct within a row (a repeated expert is computed once per slot).
 * fused = 1: silu(gate)*up in the gate_up kernel's epilogue and h's row quant
 * in the down kernel's A-load; fused = 0: the three-launch path (gate_up,
 * silu*up + quant, down), bit-identical.  Both end with the ordered combine.
 *   x [T][H] bf16; topk_ids [T][topk] int32; topk_w [T][topk] fp32;
 *   w13 [E][2I][H] fp8, w13_s [E][2I/128][H/128] fp32;
 *   w2 [E][H][I] fp8, w2_s [E][H/128][I/128] fp32 -> out [T][H] bf16.
 * The workspace holds, at byte offsets r9k_moe_ws_offset() reports, the
 * intermediates per pair p = t*topk + j: gu [T*topk][2I] bf16 (unfused only),
 * h [T*topk][I] bf16, y [T*topk][H] fp32.
 * Errors: NULLPTR; SHAPE if T < 0, T > 256, H or I not positive multiples of
 * 128, E <= 0, topk < 1 or topk > E; ALIGN; WORKSPACE; ARG (fused not 0/1);
 * DEVICE; LAUNCH. */
int r9k_moe_fp8_decode(const uint16_t *x, int64_t T, int64_t H, const int32_t *topk_ids, const float *topk_w,
                       int64_t topk, const uint8_t *w13, const float *w13_s, const uint8_t *w2,
                       const float *w2_s, int64_t E, int64_t I, uint16_t *out, void *workspace,
                       size_t ws_bytes, int fused, void *stream);

/* r9k_moe_fp8_decode on fragment-order expert weights: w13p = r9k_pack_weight
 * of w13 viewed as [E * 2I][H], w2p = r9k_pack_weight of w2 viewed as
 * [E * H][I] (2I and H are multiples of 128, so no 16-row tile straddles two
 * experts).  Same arguments, workspace and result bits as the row-major call.
 * Errors: as r9k_moe_fp8_decode. */
int r9k_moe_fp8_decode_packed(const uint16_t *x, int64_t T, int64_t H, const int32_t *topk_ids,
                              const float *topk_w, int64_t topk, const uint8_t *w13p, const float *w13_s,
                              const uint8_t *w2p, const float *w2_s, int64_t E, int64_t I, uint16_t *out,
                              void *workspace, size_t ws_bytes, int fused, void *stream);

/* Options of r9k_moe_fp8_decode_ex. */
typedef struct r9k_moe_opts {
    int fused;                /* 1: the fused path, 0: the three-launch path (as for r9k_moe_fp8_decode) */
    int packed;               /* 1: w13 and w2 in fragment order (as for r9k_moe_fp8_decode_packed), 0: row-major */
    const uint16_t *shared;   /* NULL, or the shared expert's output s [T][H] bf16 (device) */
    const float *shared_w;    /* NULL (weight 1), or its weight g [T] fp32 (device); needs shared */
} r9k_moe_opts;

/* r9k_moe_fp8_decode with the shared expert folded into the combine: the
 * fused top-k sum with the shared expert (release v0.3.0, "What changed for
 * someone running it").  With opts->shared set,
 *   out[t][n] = bf16( sum_j topk_w[t][j] * y(t,j)[n]  +  g[t] * s[t][n] ),
 * j ascending in fp32, the shared term added last, one rounding; g[t] =
 * shared_w[t], or 1 when shared_w is NULL.  Without it, the same result bits
 * as r9k_moe_fp8_decode (opts->packed = 0) or r9k_moe_fp8_decode_packed (1).
 * The caller computes s (e.g. with r9k_gemm_fp8_block_qa) and g.
 * Errors: as r9k_moe_fp8_decode; NULLPTR also for opts, or for shared_w
 * without shared; ALIGN also for shared and shared_w; ARG for a fused or
 * packed flag other than 0 or 1. */
int r9k_moe_fp8_decode_ex(const uint16_t *x, int64_t T, int64_t H, const int32_t *topk_ids, const float *topk_w,
                          int64_t topk, const uint8_t *w13, const float *w13_s, const uint8_t *w2,
                          const float *w2_s, int64_t E, int64_t I, uint16_t *out, void *workspace,
                          size_t ws_bytes, const r9k_moe_opts *opts, void *stream);

/* MoE routing in one launch (release v0.3.0, "What changed for someone running
 * it": one-launch MoE routing).  For each token t, the topk experts with the
 * largest logits[t][e], a larger logit first and equal logits in ascending e
 * (the softmax is increasing, so these are the topk largest probabilities);
 * their weights are the softmax probabilities renormalised over the chosen
 * experts, w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) with l_0 the largest
 * logit, in fp32 with HIP's expf.  The output feeds r9k_moe_fp8_decode.
 *   logits [T][E] fp32 (finite) -> topk_ids [T][topk] int32, topk_w [T][topk] fp32.
 * One wave per token, no workspace.
 * Errors: NULLPTR; SHAPE if T < 0, E < 1, E > 65536, topk < 1, topk > E or
 * topk > 64; ALIGN; DEVICE; LAUNCH.  T = 0 launches nothing. */
int r9k_moe_route(const float *logits, int64_t T, int64_t E, int64_t topk, int32_t *topk_ids, float *topk_w,
                  void *stream);

/* Byte offset inside the MoE workspace of an intermediate of the three-launch
 * path (release v0.3.3, "What changed for someone running it"; for tests):
 * which = 0 gu [P][2I] bf16, 1 h [P][I] bf16, 2 y [P][H] fp32, 3 hq [P][I] fp8,
 * 4 hs [P][I/128] fp32 (P = T*topk; gu, hq and hs are written by the
 * three-launch path only).  Host only.  Errors: NULLPTR; SHAPE; ARG. */
int r9k_moe_ws_offset(int64_t T, int64_t H, int64_t E, int64_t I, int64_t topk, int which, size_t *offset);

#if defined(__GNUC__) || defined(__clang__)
#pragma GCC visibility pop
#endif

#ifdef __cplusplus
}
#endif

#endif /* R9K_H */
