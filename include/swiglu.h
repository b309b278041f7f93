/*
 * swiglu.h -- C ABI of the MI355X (gfx950) fused SwiGLU MLP GEMM library.
 *
 * Computes  Y = SiLU(A x W1) (.) (A x W2)  with bf16 inputs, fp32 accumulation
 * and a bf16 result, in which the Gate (A x W1) and Up (A x W2) products never
 * leave the chip.  The operation is defined on the gist.science page
 * "Riepilogo Tecnico: Sovrapposizione delle Attivazioni a Livello di Tile per
 * l'Inferenza Efficiente di LLM" (summary of arXiv 2607.02521), cited as [RT]:
 *   [RT §Definizione del Problema]  the gated MLP formula, two independent
 *                                   GEMMs followed by an element-wise gate;
 *   [RT §Metodologia, Kernel-1]     "sync": the Gate tile is finished first,
 *                                   SiLU is applied to its register-resident
 *                                   accumulator while the Up weight tiles are
 *                                   being loaded, the product is formed and
 *                                   stored in the epilogue (large batches);
 *   [RT §Metodologia, Kernel-2]     "interleave": W1 and W2 are stored as one
 *                                   [K, 2N] matrix with Gate in even and Up in
 *                                   odd columns, one [M, 2N, K] GEMM runs and
 *                                   the epilogue multiplies SiLU(even column)
 *                                   by the odd column (small batches);
 *   [RT §Definizione del Problema]  the unfused baseline that writes Gate and
 *                                   Up to HBM before a separate activation.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All functions are extern "C", never throw and never exit; they return a
 *    swiglu_status_t.  Argument checks run synchronously before anything is
 *    enqueued; on any error nothing is enqueued.
 *  - Tensors are device pointers (memory from hipMalloc or any allocator that
 *    returns device-accessible memory, e.g. torch), dense and row-major with
 *    no strides, holding bf16 values (raw 16-bit patterns).
 *      A       [M, K]           activations
 *      W1, W2  [K, N]           Gate and Up weights   (SWIGLU_LAYOUT_SEPARATE)
 *      W_fused [K, 2N]          W_fused[k, 2n] = W1[k, n], [k, 2n+1] = W2[k, n]
 *                               (SWIGLU_LAYOUT_INTERLEAVED; passed as W1, W2
 *                               must then be NULL)
 *      Y       [M, N]           output, bf16 rounded to nearest even from fp32
 *  - The caller owns every buffer and keeps it alive until the stream work has
 *    completed.  The library never allocates device memory, never frees or
 *    retains caller pointers.  Y must not overlap any input.
 *  - Shapes: M, N, K >= 0.  M == 0 or N == 0 is a no-op (pointers may then be
 *    NULL).  K == 0 writes Y = 0 (empty sums).  The kernels need N % 8 == 0,
 *    K % 8 == 0 and 16-byte aligned pointers; other shapes or alignments give
 *    SWIGLU_ERR_UNSUPPORTED.  Ragged row tiles are masked, so M needs no
 *    multiple; M is bounded by the tensor-size rule below and, for the
 *    split-K streaming configurations (family 1, chosen for small M or forced
 *    by id), by 65535 row blocks of `bm` rows (bm = 16 ... 64, so M up to
 *    1,048,560 ... 4,194,240): a larger M on such a configuration gives
 *    SWIGLU_ERR_UNSUPPORTED before anything is enqueued.
 *    Every byte offset must fit in 31 bits (each tensor < 2 GiB), otherwise
 *    SWIGLU_ERR_UNSUPPORTED.
 *  - Execution is asynchronous on the given stream (0 = the null stream of the
 *    current device); SWIGLU_OK means "enqueued".  Each kernel is launched
 *    with hipLaunchKernel and judged by that call's own return value: a
 *    failed launch gives SWIGLU_ERR_LAUNCH.  An error left pending on the
 *    calling thread by an earlier HIP call is neither cleared nor reported
 *    (hipGetLastError still returns it to the caller).
 *  - A handle holds host state only, is immutable after creation and may be
 *    used from several host threads and streams at once.  It is bound to the
 *    device it was created for; that device must be current when calling.
 */
#ifndef SWIGLU_H
#define SWIGLU_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct swiglu_ctx* swiglu_handle_t;

typedef enum {
  SWIGLU_OK = 0,
  SWIGLU_ERR_INVALID_ARG = 1, /* NULL pointer, negative size, unknown enum   */
  SWIGLU_ERR_UNSUPPORTED = 2, /* shape/alignment/config the kernels cannot take */
  SWIGLU_ERR_DEVICE = 3,      /* no device, bad ordinal or not gfx950         */
  SWIGLU_ERR_LAUNCH = 4,      /* the HIP launch reported an error             */
  SWIGLU_ERR_ALLOC = 5        /* host allocation of the handle failed         */
} swiglu_status_t;

typedef enum {
  SWIGLU_LAYOUT_SEPARATE = 0,   /* W1, W2 each [K, N]                          */
  SWIGLU_LAYOUT_INTERLEAVED = 1, /* W1 = W_fused [K, 2N], W2 = NULL            */
  SWIGLU_LAYOUT_PACKED = 2      /* W1 = W_fused in MFMA fragment order (see
                                   swiglu_pack_fragments), W2 = NULL           */
} swiglu_layout_t;

typedef enum {
  SWIGLU_VARIANT_AUTO = 0,       /* table choice for the layout and shape      */
  SWIGLU_VARIANT_SYNC = 1,       /* Kernel-1 family: separate layout           */
  SWIGLU_VARIANT_INTERLEAVE = 2, /* Kernel-2 family: interleaved layout        */
  SWIGLU_VARIANT_GEMM = 3,       /* plain bf16 GEMM (unfused baseline only)    */
  SWIGLU_VARIANT_FP8 = 4,        /* config descriptions: Kernel-2 order on FP8
                                    inputs (swiglu_forward_fp8, INTERLEAVE)    */
  SWIGLU_VARIANT_FP8_SYNC = 5,   /* config descriptions: Kernel-1 order on FP8
                                    inputs (swiglu_forward_fp8, SYNC)          */
  SWIGLU_VARIANT_MXFP8 = 6,      /* Kernel-2 order on MXFP8 inputs
                                    (swiglu_forward_mx; swiglu_query_fp8)      */
  SWIGLU_VARIANT_PACKED = 7,     /* Kernel-2 order on fragment-ordered W_fused
                                    (PACKED layout)                            */
  SWIGLU_VARIANT_FP8_PACKED = 8, /* Kernel-2 order on FP8 inputs with
                                    fragment-ordered W8 (swiglu_forward_fp8)   */
  SWIGLU_VARIANT_MXFP8_PACKED = 9, /* Kernel-2 order on MXFP8 inputs with
                                    fragment-ordered W8 (swiglu_forward_mx_packed;
                                    swiglu_query_fp8)                          */
  SWIGLU_VARIANT_MXFP8_SYNC = 10, /* Kernel-1 order on MXFP8 inputs, the same W8
                                    and scales (swiglu_forward_mx with a config
                                    of this variant; swiglu_query_fp8)         */
  SWIGLU_VARIANT_PACKED_SPLITK = 11 /* PACKED with K also split over workgroups
                                    (swiglu_forward_packed_splitk only)        */
} swiglu_variant_t;

/* Description of one compiled kernel configuration. */
typedef struct swiglu_tile {
  int32_t id;          /* index in [0, swiglu_config_count())                */
  int32_t variant;     /* swiglu_variant_t: SYNC, INTERLEAVE, GEMM, FP8 or
                          FP8_SYNC                                            */
  int32_t family;      /* 0 = LDS-tiled MFMA 32x32x16 (FP8: 32x32x64 with
                          unit block scales), 1 = split-K streaming
                          MFMA 16x16x32 (weights straight to registers),
                          2 = LDS-tiled on one persistent workgroup per
                          CU looping over tiles, the next tile's loads
                          issued under the current tile's last K steps,
                          3 = streaming as 1 with K also split over
                          workgroups (fp32 partials in a workspace)        */
  int32_t bm;          /* output rows per workgroup                           */
  int32_t bn;          /* output (Y or G) columns per workgroup               */
  int32_t bk;          /* K depth of one pipeline stage                       */
  int32_t waves;       /* waves (64 lanes) per workgroup                      */
  int32_t split_k;     /* waves of one workgroup that split K (1 = none)      */
  int32_t lds_bytes;   /* LDS per workgroup                                   */
  int32_t tail_split;  /* 0, or 4: when the tiles leave a last round of
                          workgroups at most a quarter full, each of its tiles
                          runs as four (bm/2 x bn/2) tiles in the same launch */
} swiglu_tile_t;

/* Create a handle for HIP device `device`.  Checks that the device exists and
 * is gfx950; reads its compute-unit count; the first handle on a device also
 * resolves that device's address of the fixed scratch array of
 * swiglu_forward_unfused_static (making the device current for that lookup
 * and restoring the caller's current device).  *out is set to NULL on error.
 * Errors: INVALID_ARG (out NULL), DEVICE (also: the scratch address could not
 * be resolved), ALLOC. */
swiglu_status_t swiglu_create(swiglu_handle_t* out, int device);

/* Release a handle (NULL is accepted).  No call using it may be executing. */
swiglu_status_t swiglu_destroy(swiglu_handle_t h);

/* Fused forward [RT §Metodologia]: SEPARATE layout runs the sync family
 * (Kernel-1: from M = 65 a Gate and an Up wave group share each A k-tile and
 * SiLU(Gate) is applied to the Gate group's register-resident accumulator;
 * the phase tiles that run the Gate and then the Up K loop are selectable by
 * config id), INTERLEAVED runs the interleave family (Kernel-2), PACKED runs
 * the Kernel-2 order on fragment-ordered W_fused (split-K weight streaming, any
 * M; made for decode-sized batches); the tile configuration comes from the
 * per-shape table. */
swiglu_status_t swiglu_forward(swiglu_handle_t h, const void* A, const void* W1,
                               const void* W2, void* Y, int64_t M, int64_t N,
                               int64_t K, swiglu_layout_t layout, hipStream_t stream);

/* As swiglu_forward with an explicit variant and configuration (config_id < 0
 * uses the table).  The variant must match the layout (SYNC <-> SEPARATE,
 * INTERLEAVE <-> INTERLEAVED, INTERLEAVE or PACKED <-> PACKED) and a given
 * config must belong to the layout's family (variant SYNC, INTERLEAVE or
 * PACKED), otherwise INVALID_ARG.  Used by tuning sweeps and tests. */
swiglu_status_t swiglu_forward_ex(swiglu_handle_t h, const void* A, const void* W1,
                                  const void* W2, void* Y, int64_t M, int64_t N,
                                  int64_t K, swiglu_layout_t layout,
                                  swiglu_variant_t variant, int32_t config_id,
                                  hipStream_t stream);

/* Bytes of caller-owned device workspace the unfused baseline needs: Gate and
 * Up as bf16 [M, N] each, i.e. 4*M*N (0 for negative sizes). */
int64_t swiglu_unfused_workspace_bytes(int64_t M, int64_t N);

/* Unfused baseline [RT §Definizione del Problema]: G = A W1 and U = A W2 are
 * written to `workspace` as bf16 ([M, N] G followed by [M, N] U, 16-byte
 * aligned, at least swiglu_unfused_workspace_bytes(M, N) bytes), then a
 * separate element-wise kernel computes Y = bf16(SiLU(G) * U) in fp32.  Three
 * launches; separate layout only.  gemm_config_id < 0 uses the table's GEMM
 * configuration (config ids of variant GEMM only). */
swiglu_status_t swiglu_forward_unfused(swiglu_handle_t h, const void* A,
                                       const void* W1, const void* W2,
                                       void* workspace, void* Y, int64_t M,
                                       int64_t N, int64_t K, int32_t gemm_config_id,
                                       hipStream_t stream);

/* Size of the fixed device scratch array of swiglu_forward_unfused_static:
 * 128 MiB on each device the library runs on (Gate and Up of M * N <= 2^25
 * outputs, e.g. the Qwen2.5-1.5B MLP at M = 2048). */
#define SWIGLU_STATIC_SCRATCH_BYTES (128LL * 1024 * 1024)

/* The unfused baseline with no allocation of any kind, for callers that
 * cannot allocate device memory: code running under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The same launches and
 * result as swiglu_forward_unfused, but G and U live in a fixed array of
 * SWIGLU_STATIC_SCRATCH_BYTES that the library holds on each device from its
 * first swiglu_create there until the process ends, instead of a caller
 * workspace.  The caller still passes A, W1, W2 and Y (separate layout).
 * 4 * M * N > SWIGLU_STATIC_SCRATCH_BYTES gives SWIGLU_ERR_UNSUPPORTED with
 * nothing enqueued; the other argument rules and errors are those of
 * swiglu_forward_unfused.  Every call on one device shares that device's
 * array, which keeps the last call's Gate and Up (nothing in it has to start
 * at zero): calls that can overlap on one device -- on different streams, from
 * different host threads or handles -- race on it, and the caller must order
 * them (one stream, or events). */
swiglu_status_t swiglu_forward_unfused_static(swiglu_handle_t h, const void* A,
                                              const void* W1, const void* W2, void* Y,
                                              int64_t M, int64_t N, int64_t K,
                                              int32_t gemm_config_id, hipStream_t stream);

/* Build W_fused [K, 2N] from W1, W2 [K, N] [RT §Metodologia, Kernel-2]:
 * W_fused[k, 2n] = W1[k, n], W_fused[k, 2n+1] = W2[k, n].  A bit copy done
 * once per weight set, outside the forward.  N % 8 == 0 and 16-byte aligned
 * pointers required (else UNSUPPORTED); W_fused must not overlap W1 or W2. */
swiglu_status_t swiglu_pack_interleaved(swiglu_handle_t h, const void* W1,
                                        const void* W2, void* W_fused, int64_t K,
                                        int64_t N, hipStream_t stream);

/* ---- fragment-ordered W_fused (SWIGLU_LAYOUT_PACKED) ------------------------
 * W_fused [K, 2N] of [RT §Metodologia, Kernel-2] stored once, offline, in the
 * order the decode kernel's 16x16x32 MFMAs consume it, so that every load
 * instruction reads 1 KB contiguous and each workgroup streams one contiguous
 * span.  With S = ceil(2N / 128) slabs of 128 W_fused columns and
 * T = ceil(K / 32) steps of 32 k, P holds S * T * 4096 bf16 values:
 *   P[((s*T + t)*8 + c)*512 + (16*g + l)*8 + e] = W_fused[32t + 8g + e][128s + 8l + c]
 * for s < S, t < T, c < 8, g < 4, l < 16, e < 8, and 0 where the row is >= K
 * or the column >= 2N.  Each 16-byte run is 8 consecutive k of one column (a
 * k-contiguous layout: no transposition on the way to the MFMA). */

/* Bytes of the fragment-ordered W_fused for N, K: 2 * S * T * 4096 (0 when
 * N <= 0 or K <= 0 or a size is out of range). */
int64_t swiglu_packed_bytes(int64_t N, int64_t K);

/* Build the fragment-ordered W_fused P (swiglu_packed_bytes(N, K) bytes, padding
 * included) from W1, W2 [K, N].  A bit copy done once per weight set, outside
 * the forward.  N % 8 == 0, K % 8 == 0, 16-byte aligned pointers and tensors
 * under 2 GiB required (else UNSUPPORTED); P must not overlap W1 or W2
 * (INVALID_ARG).  K == 0 or N == 0 is a no-op. */
swiglu_status_t swiglu_pack_fragments(swiglu_handle_t h, const void* W1, const void* W2,
                                      void* P, int64_t K, int64_t N, hipStream_t stream);

/* ---- decode with K split over workgroups (PACKED layout, 1 <= M <= 16) ----
 * For decode shapes whose weight slabs are too few to give every CU work (a
 * narrow N, such as one GPU's share of a tensor-parallel MLP), S workgroups
 * share each slab part: each streams a contiguous range of its K steps and
 * writes fp32 partial sums to a caller workspace; the last of the S to finish
 * adds them in K order (fixed, so results are reproducible) and applies SiLU
 * and the pair product [RT §Metodologia, Kernel-2 pairing; §Risultati: split
 * sums kept in FP32 and reduced before the activation].  No workgroup waits
 * for another.
 *
 * Workspace: swiglu_packed_splitk_workspace_bytes(N, K, S) bytes, 16-byte
 * aligned, caller-owned, **all zero before its first use**: it holds a counter
 * per slab part, and every call leaves those back at zero when it completes,
 * so a workspace zeroed once can serve any number of calls in stream order.
 * Calls that may run at the same time on the GPU need workspaces of their own;
 * a call that did not complete (an aborted launch) leaves it to be zeroed
 * again. */

/* Bytes of the split-K workspace for N, K and S pieces of K: a 256-byte
 * aligned block of counters (ceil(2N/128) * 16 bytes, rounded up) plus
 * ceil(2N/128) * S * 8192 bytes of fp32 partials.  0 for N <= 0, K < 0,
 * S outside [1, 64] or sizes out of range. */
int64_t swiglu_packed_splitk_workspace_bytes(int64_t N, int64_t K, int32_t ksplit);

/* The configuration (variant PACKED_SPLITK) and S the library picks for the
 * shape on this handle's device (either out-pointer may be NULL).
 * UNSUPPORTED for M > 16. */
swiglu_status_t swiglu_packed_splitk_plan(swiglu_handle_t h, int64_t M, int64_t N, int64_t K,
                                          int32_t* config_id, int32_t* ksplit);

/* Y = SiLU(A W1) * (A W2) for 1 <= M <= 16 on the fragment-ordered W_fused P
 * (swiglu_pack_fragments), K split into S = ksplit pieces over workgroups.
 * config_id < 0 or ksplit < 1: the plan's choice for that argument.  The
 * arguments are checked as for swiglu_forward with the PACKED layout; also
 * INVALID_ARG for a config of another variant, a NULL or too small workspace,
 * or one overlapping A, P or Y; UNSUPPORTED for M > 16, S > 64 or a
 * workspace not 16-byte aligned. */
swiglu_status_t swiglu_forward_packed_splitk(swiglu_handle_t h, const void* A, const void* P,
                                             void* Y, int64_t M, int64_t N, int64_t K,
                                             int32_t config_id, int32_t ksplit, void* workspace,
                                             int64_t workspace_bytes, hipStream_t stream);

/* What swiglu_forward / _ex(AUTO) would run for this shape and layout, and
 * which layout the table recommends for the shape (the per-batch choice of
 * kernel family [RT §Contributi Chiave, item 2]): PACKED up to M = 64 (up to
 * M = 16 when N >= 16384 on 256 CUs), INTERLEAVED above (measured on
 * MI355X).  Any out-pointer may be NULL.
 * For variant GEMM pass layout SEPARATE to ask for the unfused GEMM config. */
swiglu_status_t swiglu_query(swiglu_handle_t h, int64_t M, int64_t N, int64_t K,
                             swiglu_layout_t layout, swiglu_variant_t* chosen,
                             swiglu_tile_t* tile, swiglu_layout_t* recommended_layout);

/* Same question for the unfused baseline's GEMM configuration. */
swiglu_status_t swiglu_query_unfused(swiglu_handle_t h, int64_t M, int64_t N,
                                     int64_t K, swiglu_tile_t* tile);

/* Tuned per-shape configurations.  A tuned file (written by the package's
 * tuner, python -m gemm_epilogues_mlp_amd.tune) is text:
 *   swiglu-tuned <signature: 16 hex digits> <arch>        first non-comment line
 *   <variant> <M> <N> <K> <config id> [ignored provenance]    one per shape
 * (variant: a swiglu_variant_t value, the one of the config)
 * with '#' comment lines.  The signature (swiglu_config_signature) identifies
 * the list of compiled configurations; a file written for a library with a
 * different list is refused, so an id can never name the wrong kernel.
 * Entries only add exact shapes: every other shape keeps the built-in table
 * [RT §Contributi Chiave, item 2: the per-batch choice of kernel]. */
uint64_t swiglu_config_signature(void);

/* Read and validate a tuned file without a device.  *n_entries (may be NULL)
 * receives the number of entries.  Errors: INVALID_ARG (NULL path, unreadable
 * or malformed file, a config id that does not exist or is not of the entry's
 * variant, more than 4096 entries), UNSUPPORTED (signature of another build). */
swiglu_status_t swiglu_tuned_check(const char* path, int32_t* n_entries);

/* swiglu_create plus the entries of a tuned file (path NULL: none), which then
 * take precedence over the built-in table for their exact (variant, M, N, K)
 * in swiglu_forward, _ex with config_id < 0, _unfused, _fp8 and _mx with
 * config_id < 0, and the queries.  The
 * file is read once here; the handle stays immutable.  Errors: those of
 * swiglu_tuned_check, then those of swiglu_create. */
swiglu_status_t swiglu_create_tuned(swiglu_handle_t* out, int device, const char* path);

/* ---- FP8 inputs -----------------------------------------------------------
 * [RT §Definizione del Problema] names FP8 quantisation as what makes the
 * memory-bound activation a larger share of the MLP, and the page
 * "Ottimizzazione delle GEMM: la chiave per l'efficienza dei Large Language
 * Models" (§Impatto sui deployment on-premise) benchmarks MXFP8 GEMMs; neither
 * fixes the format.  Taken here: OCP FP8 E4M3 codes (one byte: sign, 4
 * exponent bits with bias 7, 3 mantissa bits; no infinities; S.1111.111 is
 * NaN; largest finite 448) with one fp32 scale per tensor, a code q standing
 * for scale * value(q).
 *   A8  [M, K]   E4M3 activations, row-major
 *   W8  [2N, K]  E4M3 weights with k contiguous: row 2n is column n of W1
 *                (Gate), row 2n+1 column n of W2 (Up) -- the Kernel-2 pairing
 *                [RT §Metodologia], each W_fused column stored as a row
 * The FP8 calls need N % 8 == 0, K % 16 == 0, 16-byte aligned pointers and
 * tensors under 2 GiB (else UNSUPPORTED); otherwise the conventions above. */

/* Y = bf16(SiLU(g) * u) with g = fp32(scale_a * scale_w1) * (A8 x W1) and
 * u = fp32(scale_a * scale_w2) * (A8 x W2): the E4M3 products are exact and
 * accumulate in fp32; the scales apply to the finished sums, before SiLU.
 * Both kernel orders read the same W8: variant INTERLEAVE (or AUTO) runs one
 * GEMM over the paired rows with the pair-multiply epilogue [RT §Metodologia,
 * Kernel-2]; SYNC runs the Gate rows over the whole K, applies SiLU in
 * registers while the Up tiles load, then the Up rows [RT §Metodologia,
 * Kernel-1]; FP8_PACKED runs the Kernel-2 order with W8 passed in fragment
 * order (swiglu_pack_fp8_fragments; a streaming kernel made for decode-sized
 * batches); any other variant is INVALID_ARG.  config_id < 0 uses the table;
 * a given id must be of variant FP8 (INTERLEAVE), FP8_SYNC (SYNC) or
 * FP8_PACKED, else INVALID_ARG.  Y must not overlap A8 or W8. */
swiglu_status_t swiglu_forward_fp8(swiglu_handle_t h, const void* A8, const void* W8, void* Y,
                                   int64_t M, int64_t N, int64_t K, float scale_a,
                                   float scale_w1, float scale_w2, swiglu_variant_t variant,
                                   int32_t config_id, hipStream_t stream);

/* Q[i] = E4M3(fp32(X[i] * inv_scale)) for `count` bf16 values X: round to
 * nearest even; magnitudes >= 448 and infinities saturate to +-448; NaN gives
 * the NaN code; the sign of zero is kept.  count % 16 == 0; Q (count bytes)
 * must not overlap X.  Quantises activations per forward or weights once. */
swiglu_status_t swiglu_quantize_fp8(swiglu_handle_t h, const void* X, void* Q, int64_t count,
                                    float inv_scale, hipStream_t stream);

/* W8 [2N, K] from E4M3 W1, W2 [K, N] (row-major): W8[2n, k] = W1[k, n],
 * W8[2n+1, k] = W2[k, n].  A bit copy done once per weight set.  W8 must not
 * overlap W1 or W2. */
swiglu_status_t swiglu_pack_fp8(swiglu_handle_t h, const void* W1, const void* W2, void* W8,
                                int64_t K, int64_t N, hipStream_t stream);

/* Fragment-ordered W8 (variant FP8_PACKED): the W8 pairing above cut into
 * blocks of 16 rows and steps of 128 k, each 2048-byte block the B operand of
 * one 16x16x128 MFMA for 64 lanes, stored as two 1 KB halves.  With
 * T = ceil(K / 128):
 *   P8[((rb*T + t)*2 + h)*1024 + (16*g + i)*16 + e] = W8[16*rb + i][128*t + 64*h + 16*g + e]
 * for rb < ceil(2N / 16), h < 2, g < 4, i < 16, e < 16, and 0 where the row
 * is >= 2N or the byte >= K.  Every load instruction then reads 1 KB
 * contiguous.  swiglu_fp8_packed_bytes gives its size (0 when N <= 0 or
 * K <= 0 or a size is out of range). */
int64_t swiglu_fp8_packed_bytes(int64_t N, int64_t K);

/* P8 (swiglu_fp8_packed_bytes(N, K) bytes, padding included) from W8 [2N, K].
 * A byte copy done once per weight set.  N % 8 == 0, K % 16 == 0, 16-byte
 * aligned pointers and tensors under 2 GiB (else UNSUPPORTED); P8 must not
 * overlap W8 (INVALID_ARG).  K == 0 or N == 0 is a no-op. */
swiglu_status_t swiglu_pack_fp8_fragments(swiglu_handle_t h, const void* W8, void* P8,
                                          int64_t K, int64_t N, hipStream_t stream);

/* ---- MXFP8 inputs ----------------------------------------------------------
 * The OCP Microscaling format with E4M3 elements, which the TorchInductor/
 * CuteDSL page (§Impatto sui deployment on-premise) benchmarks: every 32
 * consecutive k of a row share one E8M0 scale byte e standing for 2^(e-127)
 * (e = 255: NaN), so element k of a row is 2^(e[k/32] - 127) * value(q[k]).
 *   A8 [M, K] + SA [M, ks]       activations and their scales
 *   W8 [2N, K] + SW [2N, ks]     the k-major paired weights (row 2n Gate
 *                                column n, row 2n+1 Up column n) and scales
 * Scale rows have a stride of ks bytes, ks a multiple of 16 and >= K/32;
 * bytes past K/32 (the row padding) may be loaded with their 16-byte chunk
 * but never affect the result, whatever they hold.  The forward needs K % 64 == 0,
 * N % 8 == 0, 16-byte aligned pointers and every tensor under 2 GiB (else
 * UNSUPPORTED). */

/* Y = bf16(SiLU(g) * u), g = A x W1 and u = A x W2 on the MX values: the MFMA
 * applies the block scales to exact E4M3 products, fp32 accumulation.
 * config_id < 0 uses the table (the interleave order, [RT §Metodologia,
 * Kernel-2]); a given id must be of variant MXFP8 or MXFP8_SYNC (else
 * INVALID_ARG).  A MXFP8_SYNC configuration runs the sync order on the same
 * W8 and scales ([RT §Metodologia, Kernel-1]: each output tile's Gate rows
 * first, SiLU on the register-resident Gate sums while the Up rows' tiles and
 * scales are in flight, then the Up rows); swiglu_query_fp8 with
 * SWIGLU_VARIANT_MXFP8_SYNC reports the table's choice of it.  Y must not
 * overlap any input. */
swiglu_status_t swiglu_forward_mx(swiglu_handle_t h, const void* A8, const void* SA,
                                  const void* W8, const void* SW, void* Y, int64_t M, int64_t N,
                                  int64_t K, int64_t ks, int32_t config_id, hipStream_t stream);

/* MX quantisation of bf16 rows X [rows, K] (k contiguous, K % 32 == 0) into
 * Q [rows, K] E4M3 and S [rows, ks] E8M0 (ks % 16 == 0, ks >= K/32; bytes
 * past K/32 are written as 0).  Per block of 32: shared exponent =
 * floor(log2 max |x|) - 8 (E4M3's largest normal is 1.75 * 2^8), clamped to
 * [-127, 127] (-127 for a block of zeros or subnormals; NaN is left out of the
 * maximum, an infinity counts as 2^128); elements x * 2^-shared rounded to
 * nearest even E4M3, saturating at +-448, NaN kept.  Outputs must not overlap
 * X or each other. */
swiglu_status_t swiglu_quantize_mx(swiglu_handle_t h, const void* X, void* Q, void* S,
                                   int64_t rows, int64_t K, int64_t ks, hipStream_t stream);

/* The MXFP8 forward of swiglu_forward_mx with W8 passed in the fragment order
 * of a streaming kernel made for decode-sized batches (any M; the weights are
 * read once per 32 rows of A).  The order is that of the 32x32x64 scaled MFMA's
 * sources: W8 cut into blocks of 32 rows and steps of 64 k (K % 64 == 0), each
 * 2048-byte block stored as two 1 KB halves, with T = K / 64:
 *   P8[((rb*T + t)*2 + v)*1024 + (i + 32*h)*16 + e] = W8[32*rb + i][64*t + 32*v + 16*h + e]
 * for rb < ceil(2N / 32), v < 2, h < 2, i < 32, e < 16, and 0 for rows >= 2N.
 * SA, SW and ks are those of swiglu_forward_mx (the scales are not reordered).
 * config_id < 0 uses the table; a given id must be of variant MXFP8_PACKED.
 * Errors and other conventions as swiglu_forward_mx. */
swiglu_status_t swiglu_forward_mx_packed(swiglu_handle_t h, const void* A8, const void* SA,
                                         const void* P8, const void* SW, void* Y, int64_t M,
                                         int64_t N, int64_t K, int64_t ks, int32_t config_id,
                                         hipStream_t stream);

/* Bytes of that P8: ceil(2N / 32) * (K / 64) * 2048 (0 when N <= 0, K <= 0,
 * K % 64 != 0 or a size is out of range). */
int64_t swiglu_mx_packed_bytes(int64_t N, int64_t K);

/* P8 (swiglu_mx_packed_bytes(N, K) bytes) from E4M3 W8 [2N, K], a byte copy
 * done once per weight set.  N % 8 == 0, K % 64 == 0, 16-byte aligned
 * pointers and tensors under 2 GiB (else UNSUPPORTED); P8 must not overlap
 * W8 (INVALID_ARG).  K == 0 or N == 0 is a no-op. */
swiglu_status_t swiglu_pack_mx_fragments(swiglu_handle_t h, const void* W8, void* P8, int64_t K,
                                         int64_t N, hipStream_t stream);

/* bf16 Wt [2N, K] from W1, W2 [K, N]: Wt[2n, k] = W1[k, n], Wt[2n+1, k] =
 * W2[k, n] (the k-major pairing, a bit copy), the input of swiglu_quantize_mx
 * for the weights.  K % 8 == 0, N % 8 == 0; Wt must not overlap W1 or W2. */
swiglu_status_t swiglu_pack_kmajor(swiglu_handle_t h, const void* W1, const void* W2, void* Wt,
                                   int64_t K, int64_t N, hipStream_t stream);

/* The configuration swiglu_forward_fp8 (variant AUTO, INTERLEAVE, SYNC or
 * FP8_PACKED), swiglu_forward_mx (variant MXFP8) or swiglu_forward_mx_packed
 * (variant MXFP8_PACKED) with config_id < 0 runs for a shape. */
swiglu_status_t swiglu_query_fp8(swiglu_handle_t h, int64_t M, int64_t N, int64_t K,
                                 swiglu_variant_t variant, swiglu_tile_t* tile);

/* Number of compiled kernel configurations and their descriptions. */
int32_t swiglu_config_count(void);
swiglu_status_t swiglu_config_info(int32_t config_id, swiglu_tile_t* out);

/* Static string for a status code ("unknown status" for other values). */
const char* swiglu_status_str(swiglu_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_H */
