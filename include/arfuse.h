/*
 * arfuse — the epilogue of a one-shot all-reduce fused with the residual add,
 * RMSNorm and an optional block-scaled FP4 quantization, for AMD Instinct
 * MI355X (gfx950). C ABI.
 *
 * The operation (per token row r, column j; N rank partials p_0..p_{N-1}):
 *
 *   acc       = p_0 + p_1 + ... + p_{N-1}     fp32, in this rank order
 *   h         = acc + residual                 fp32, residual added last
 *   residual_out = bf16(h)                      round to nearest even
 *   y         = h / sqrt(mean_j(h^2) + eps) * gamma_j
 *               (mean of squares and inverse root in fp64; the inverse is
 *               rounded to fp32 and y = (h * inv) * gamma_j in fp32)
 *   out       = bf16(y)                         optional
 *   FP4       = per 16 consecutive elements of y: scale s = E4M3(max|y| / 6),
 *               code = sign | E2M1(|y| / s)     optional
 *   FP8       = sign | E4M3(|y * inv_scale|)    optional (arfuse_rmsnorm_ex)
 *
 * The fusion patterns of the pages' fused operator are selected by which
 * pointers are given: no residual (h = the rank sum), and no gamma (no
 * RMSNorm: residual_out = bf16(sum [+ residual]) is then the plain all-reduce
 * result and the only output).
 *
 * Where the pages define it:
 *  - The all-reduce of tensor parallelism sums same-shaped partial products of
 *    the row-parallel layer ("Optimizing Tensor Parallelism Communication
 *    Overhead ...", "The Anatomy of the Tensor Parallelism Bottleneck";
 *    "Deep Dive: AllReduce and AllReduce Fusion in TensorRT-LLM", §2.1.1 and
 *    §2.7). Here the N partials are N buffers in this GPU's HBM; they stand in
 *    for the peer slots a one-shot kernel reads after the push (Deep Dive
 *    §5.2, ONESHOT).
 *  - A fixed summation order gives the same bits on every rank
 *    ("Collectives, topology, custom all-reduce", the one-shot kernel and the
 *    determinism section); fp32 accumulation is the fp32_acc option of the
 *    fused call in the same page and the Fp32Acc template flag (Deep Dive
 *    §3.1.5).
 *  - Residual add, residual store, RMSNorm with gamma and eps, normalized
 *    store and quantization follow the fused operator of Deep Dive §6.3 and
 *    §6.5; eps is the layer norm's variance epsilon (Deep Dive §6.2).
 *  - The LL layout (8 bytes of payload and an 8-byte flag in one 16-byte word,
 *    the reader checking the flag) is the LL protocol of "Every µs Matters",
 *    section on signalling without barriers; the sentinel layout (a value
 *    real data never takes marks an element not yet written, the buffer is
 *    reset to it before reuse) is its sentinel mode and the one-shot
 *    kernel's arrival test of Deep Dive §5.2, whose triple-buffered slots are
 *    reset two calls ahead (the `reset` option).
 *  - The pattern list (all-reduce only, with or without residual, FP8 or FP4
 *    output, with or without the bf16 norm output) is Deep Dive §6.3.
 *
 * Conventions for every entry point:
 *  - Pointers marked (device) are HIP device pointers; (host) are host memory.
 *  - bf16 tensors are row-major [t][d] arrays of 16-bit bfloat16.
 *  - The caller owns every buffer. The library allocates no memory, keeps no
 *    pointer after it returns and holds no global state, apart from the
 *    static exchange slots of arfuse_rmsnorm_noalloc; calls are reentrant.
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *    work; they never synchronize, so they are legal under stream capture.
 *  - Argument errors are returned before anything is enqueued. A failed
 *    launch returns ARFUSE_ERR_LAUNCH. Data-dependent errors (LL flags,
 *    sentinel slots, a split row's exchange) are written to a device status
 *    word instead (arfuse_ll_status); a call that can wait for data or for
 *    another workgroup is rejected without one (see arfuse_rmsnorm_ex).
 *  - t == 0 is a no-op: only the shape, eps and the options are validated and
 *    the buffer pointers may be NULL.
 */
#ifndef ARFUSE_H
#define ARFUSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ARFUSE_VERSION 4

/* Largest supported rank count and row width. */
#define ARFUSE_MAX_PARTIALS 8
#define ARFUSE_MAX_D 65536
/* Largest accepted opts->max_polls: bounds how long a row can wait on data
 * that never arrives (each re-read follows a sleep of about 60 ns). */
#define ARFUSE_MAX_POLLS (1u << 20)

typedef enum {
  ARFUSE_OK = 0,
  /* null or misaligned pointer, n_partials outside [1, 8], t < 0, d <= 0,
   * d % 16 != 0, eps negative or not finite, overlapping buffers (other than
   * residual_out == residual), bad option values */
  ARFUSE_ERR_INVALID_ARG = 1,
  /* valid arguments without a compiled kernel (d > ARFUSE_MAX_D, a launch
   * override that does not cover the row) */
  ARFUSE_ERR_UNSUPPORTED = 2,
  /* the HIP runtime refused the launch; the returned value also carries the
   * runtime's hipError_t in bits 8 and up (status & 0xFF == 3) */
  ARFUSE_ERR_LAUNCH = 3,
  /* device side only (arfuse_ll_status.code): something a row waits for
   * did not arrive within its bounded wait (an LL word still carried
   * another flag, or a sentinel vector still held the pattern, after
   * max_polls re-reads; or a split row's partner share never came) */
  ARFUSE_ERR_FLAG_TIMEOUT = 4
} arfuse_status;

/* Input layouts of the partials. */
#define ARFUSE_LAYOUT_PLAIN 0 /* bf16 [t][d], t*d*2 bytes per partial */
#define ARFUSE_LAYOUT_LL 1    /* [t][d/4] 16-byte words: bytes 0..7 hold four
                                 bf16 elements (element 4w first, little
                                 endian), bytes 8..15 a little-endian uint64
                                 flag; t*d*4 bytes per partial */
#define ARFUSE_LAYOUT_SENTINEL 2 /* bf16 [t][d] like PLAIN; a 16-byte vector (8
                                   elements) holding the sentinel pattern in
                                   any element has not arrived yet */

/* Default sentinel: a negative NaN bf16 pattern, which finite data never
 * takes. (+0.0 or any finite value must not be used as a sentinel.) */
#define ARFUSE_SENTINEL_DEFAULT 0xFFFFu

/* Outputs of one call (the epilogue), as bit flags. */
#define ARFUSE_EPI_BF16 1 /* out: bf16 y */
#define ARFUSE_EPI_FP4 2  /* fp4_out + fp4_scales */
#define ARFUSE_EPI_FP8 4  /* opts->fp8_out (not together with FP4) */
/* A mask of 0 is the all-reduce alone (no gamma): only residual_out. */

/* Device-side status of a call (LL or sentinel layout, split rows). The
 * caller zeroes it before the call (the library only ever ORs into code and
 * adds to the counters, so one word can collect several calls, e.g. a
 * captured chain). */
typedef struct {
  uint32_t code;      /* 0, or ARFUSE_ERR_FLAG_TIMEOUT: something a row waits
                         for did not arrive within its bounded wait */
  uint32_t exchange_timeouts; /* split rows: partner slots that did not
                         carry this call's token within the bounded wait;
                         that row's outputs are unspecified */
  uint64_t bad_words; /* LL words whose flag never matched, or, in the
                         sentinel layout, 16-byte vectors that still held the
                         sentinel after the last re-read */
} arfuse_ll_status;

/* Split rows: largest number of workgroups per row, and the largest
 * t * split a call may launch (every workgroup of a row must be resident at
 * once for the exchange). */
#define ARFUSE_MAX_SPLIT 8
#define ARFUSE_MAX_SPLIT_BLOCKS 256
/* opts->split value that lets the library choose the split for the shape
 * (arfuse_query_launch reports the choice and the workspace it needs). */
#define ARFUSE_SPLIT_AUTO 0xFFFFFFFFu

/* Options of arfuse_rmsnorm_ex. Zero-initialise it for the defaults
 * (plain layout, library-chosen launch). */
typedef struct {
  int32_t layout;             /* ARFUSE_LAYOUT_PLAIN, _LL or _SENTINEL */
  uint32_t max_polls;         /* LL / SENTINEL: re-reads of a word or vector
                                 that has not arrived, with a short sleep
                                 between them, before it counts as bad
                                 (0: check once); at most ARFUSE_MAX_POLLS */
  uint64_t ll_flag;           /* LL: the flag every word must carry */
  arfuse_ll_status* status;   /* (device) status word, 8-byte aligned,
                                 overlapping no other buffer. Required (else
                                 ARFUSE_ERR_INVALID_ARG) by every call that
                                 can wait: the LL and sentinel layouts, and
                                 split rows with a norm. NULL otherwise */
  int32_t block_threads;      /* launch override: threads per row block,
                                 a multiple of 64 in [64, 1024]; 0 = auto */
  int32_t vpt;                /* launch override: 16-byte vectors per thread
                                 per partial, 1, 2, 4 or 8; 0 = auto */
  uint32_t sentinel;          /* SENTINEL: 16-bit pattern of a not-yet-
                                 written element; 0 = ARFUSE_SENTINEL_DEFAULT */
  uint32_t split;             /* workgroups per row: 0 or 1 = one; 2, 4 or 8
                                 divide each row's columns between that many
                                 workgroups on different CUs, which exchange
                                 the row's sum of squares through workspace
                                 (decode shapes, where a row is bound by one
                                 CU's fetch). Needs workspace,
                                 d % (16 * split) == 0 and
                                 t * split <= ARFUSE_MAX_SPLIT_BLOCKS; a
                                 slice of more than 16,384 elements (or a vpt
                                 override above 2) is ARFUSE_ERR_UNSUPPORTED.
                                 ARFUSE_SPLIT_AUTO: the smallest split whose
                                 slices take at most 256 threads and 16 KiB
                                 of partial reads per workgroup, used where
                                 it removes at least three waves per SIMD or
                                 the whole row reads 128 KiB or more, else
                                 1; the all-reduce alone (no exchange)
                                 splits whenever the row reads 32 KiB or
                                 more. A pure function of (n_partials, t, d,
                                 layout, whether the call normalizes) */
  void* const* reset;         /* SENTINEL: (host) array of n_partials (device)
                                 bf16 [t][d] buffers, 16-byte aligned, that this
                                 call fills with the sentinel (the slot set a
                                 later call reuses); or NULL. For t <= 128
                                 extra workgroups of the same launch write
                                 them, otherwise each row's workgroup does */
  uint8_t* fp8_out;           /* (device) uint8 [t][d] FP8 E4M3 codes of
                                 y * fp8_inv_scale (sign bit 7, saturating at
                                 448), 16-byte aligned; or NULL */
  float fp8_inv_scale;        /* per-tensor reciprocal FP8 scale, finite */
  uint32_t reserved2;         /* must be 0 */
  void* workspace;            /* split rows: (device) 256 bytes per row
                                 position, t rounded up to a multiple of 8
                                 (two 128-byte lines of slots per row;
                                 arfuse_query_launch gives the size),
                                 16-byte aligned (128-byte alignment keeps
                                 each row's slots in lines of their own, the
                                 fast case). Each slice tags its slot with a
                                 token of the kernel dispatch (the dispatch's
                                 index in its hardware queue and the queue),
                                 so any earlier contents read as "not yet
                                 written": the workspace needs no clearing,
                                 before the first call or when t or the
                                 split changes. Calls sharing a workspace
                                 must not overlap. NULL when split <= 1 */
} arfuse_opts;

/* The launch the library would use for a call. */
typedef struct {
  int64_t grid;         /* workgroups: t (one per row), or with split rows
                           split times t rounded up to a multiple of 8 (the
                           rows past t are padding that exits at once), plus,
                           in the sentinel layout with a reset set and
                           t <= 128, the blocks that write the reset */
  int32_t block;        /* threads per workgroup */
  int32_t vpt;          /* 16-byte vectors per thread per partial */
  int32_t split;        /* workgroups per row (1 unless opts->split > 1,
                           the choice for ARFUSE_SPLIT_AUTO) */
  int32_t stream_stores; /* 1: the outputs are written through to memory
                           (calls whose rows take several rounds of
                           workgroups: t * vpt >= 1536, not LL); 0: they
                           stay in the caches for the next call (whole
                           rows: default-policy stores, written back at
                           the end of the kernel; split rows: non-temporal
                           stores) */
  int64_t workspace_bytes; /* bytes of opts->workspace a split call needs */
} arfuse_launch_info;

/*
 * arfuse_rmsnorm — the fused call on plain-layout partials.
 *
 *  partials      (host) array of n_partials pointers; each (device) bf16
 *                [t][d], 16-byte aligned. Summed in array order.
 *  n_partials    1..8
 *  residual      (device) bf16 [t][d], 16-byte aligned; NULL: no residual
 *                add (h is the rank sum)
 *  gamma         (device) fp32 [d], 16-byte aligned; NULL: no RMSNorm (the
 *                plain all-reduce); then out and the FP4/FP8 outputs must be
 *                NULL and residual_out must be given
 *  eps           finite, >= 0; added to the mean square inside the root
 *  out           (device) bf16 [t][d] normalized output, 16-byte aligned;
 *                or NULL
 *  residual_out  (device) bf16 [t][d] = bf16(h); may equal residual (in place)
 *                but must not otherwise overlap any other buffer; may be NULL
 *                when gamma is given and another output is requested
 *  fp4_out       (device) uint8 [t][d/2] E2M1 codes, element 2k in the low
 *                nibble of byte k; 16-byte aligned; or NULL
 *  fp4_scales    (device) uint8 [t][d/16] E4M3 codes of the block scales;
 *                NULL exactly when fp4_out is NULL
 *  t, d          rows (tokens) and row width; d % 16 == 0, d <= 65536
 *  stream        hipStream_t
 * Returns an arfuse_status.
 */
int arfuse_rmsnorm(const void* const* partials, int n_partials, const void* residual,
                   const float* gamma, float eps, void* out, void* residual_out,
                   uint8_t* fp4_out, uint8_t* fp4_scales, int64_t t, int64_t d,
                   void* stream);

/*
 * arfuse_rmsnorm_ex — as arfuse_rmsnorm, with options (opts may be NULL).
 * With opts->layout == ARFUSE_LAYOUT_LL every partial is (device) LL words
 * [t][d/4][16 bytes]; each word's flag is compared with opts->ll_flag and a
 * word that does not match is re-read up to opts->max_polls times. With
 * ARFUSE_LAYOUT_SENTINEL the partials are plain bf16 and a 16-byte vector
 * holding opts->sentinel in any element is re-read the same way; opts->reset,
 * if given, names buffers the call fills with the sentinel. Words or vectors
 * that never arrive are counted into opts->status (if given); the rows
 * holding them get unspecified outputs. The kernel never waits without
 * bound, and since a wait that gives up is reported only there, these
 * layouts (and split rows with a norm, below) need opts->status: without it
 * the call returns ARFUSE_ERR_INVALID_ARG and enqueues nothing (a bounded
 * wait that gives up must be observable: "Optimizing Tensor Parallelism
 * Communication Overhead ...", production pitfalls, the timeout break in the
 * spin loop). opts->fp8_out requests the FP8 output.
 *
 * opts->split > 1 divides every row's columns between that many workgroups
 * (on different CUs of one XCD where the workgroups of a launch are placed on
 * the XCDs in turn: a row's slices are workgroups 8 apart). Each computes its
 * columns' share of the sum of squares, writes it with its dispatch's token
 * to its slot of opts->workspace and waits (bounded) for the row's other
 * slots to carry the same token; the shares are added in slice order, so the
 * result is deterministic (it may differ in
 * the last bits from the unsplit call, whose sum runs in another order).
 * residual_out, the FP4 and the FP8 outputs are produced per slice exactly as
 * without the split. The operation is unchanged (the mean square is over the
 * whole row, Deep Dive §6.3); only the division of the work differs. A share
 * that does not arrive is counted into opts->status (exchange_timeouts),
 * which such a call therefore needs. The wait for a share is
 * bounded (2^18 re-reads, a fraction of a second); a split row's workgroups
 * only ever wait for each other, so work running beside the call on other
 * streams can delay them but not stall them. The all-reduce alone (gamma
 * NULL) has no norm and splits without a workspace.
 */
int arfuse_rmsnorm_ex(const void* const* partials, int n_partials, const void* residual,
                      const float* gamma, float eps, void* out, void* residual_out,
                      uint8_t* fp4_out, uint8_t* fp4_scales, int64_t t, int64_t d,
                      void* stream, const arfuse_opts* opts);

/*
 * arfuse_rmsnorm_noalloc — arfuse_rmsnorm_ex for callers that cannot
 * allocate device memory or be handed a workspace: code under stream or
 * graph capture, tight serving loops, harnesses that forbid allocation.
 * Split rows exchange their sums of squares through a static array of
 * ARFUSE_NOALLOC_BYTES (32 KiB) inside the library instead of
 * opts->workspace, which must be NULL (else ARFUSE_ERR_INVALID_ARG). Every
 * split the library accepts fits it (t * split <= ARFUSE_MAX_SPLIT_BLOCKS;
 * larger requests are ARFUSE_ERR_UNSUPPORTED, as for arfuse_rmsnorm_ex).
 * Each GPU the library runs on holds its own copy of the array until the
 * process ends; the first call on a device (any call, t == 0 included) looks
 * up its address there once, with no allocation and nothing enqueued, so a
 * caller that captures can make a t == 0 call on that device beforehand.
 * The slots are never cleared and need not be: each call tags them with a
 * token of its own kernel dispatch. All calls on one GPU share the array,
 * so calls that overlap in time on one GPU (concurrent streams) race and
 * their split rows' outputs are unspecified; calls ordered on one stream,
 * or otherwise serialized, do not. Arguments, outputs, the status word
 * rule and errors are otherwise those of arfuse_rmsnorm_ex, and the results
 * are the same bits.
 */
#define ARFUSE_NOALLOC_BYTES 32768
int arfuse_rmsnorm_noalloc(const void* const* partials, int n_partials, const void* residual,
                           const float* gamma, float eps, void* out, void* residual_out,
                           uint8_t* fp4_out, uint8_t* fp4_scales, int64_t t, int64_t d,
                           void* stream, const arfuse_opts* opts);

/*
 * arfuse_quantize_fp4 — the FP4 epilogue alone, on fp32 y [t][d] (device,
 * 16-byte aligned), with the same device code as the fused call. codes:
 * (device) uint8 [t][d/2], 16-byte aligned; scales: (device) uint8 [t][d/16].
 * d % 16 == 0. (Deep Dive §6.5: quantization of the normalized output.)
 */
int arfuse_quantize_fp4(const float* y, int64_t t, int64_t d, uint8_t* codes,
                        uint8_t* scales, void* stream);

/*
 * arfuse_quantize_fp4_ll — test entry: the FP4 epilogue of LL-layout calls
 * alone, on fp32 y [t][d] (device, 16-byte aligned). In that layout a lane
 * holds groups of 4 elements and the 4 lanes of a quad hold one 16-element
 * block; this runs the same device code with thread i on group i (elements
 * 4i..4i+3 of the flattened y). codes: (device) uint8 [t][d/2], 2-byte
 * aligned; scales: (device) uint8 [t][d/16]; not overlapping y or each
 * other. d % 16 == 0. The format is arfuse_quantize_fp4's (Deep Dive §6.5).
 */
int arfuse_quantize_fp4_ll(const float* y, int64_t t, int64_t d, uint8_t* codes,
                           uint8_t* scales, void* stream);

/*
 * arfuse_query_launch — fill *info with the launch a call with these
 * arguments would use. Host only, enqueues nothing. epilogue is a mask of
 * ARFUSE_EPI_* flags. Returns an arfuse_status.
 */
int arfuse_query_launch(int n_partials, int64_t t, int64_t d, int epilogue,
                        const arfuse_opts* opts, arfuse_launch_info* info);

/*
 * arfuse_launch_floor — measurement aid: enqueue an empty kernel with the
 * same grid, block and argument block as the fused call would use, to
 * measure the per-launch floor (a single launch or a node of a captured
 * chain). Returns an arfuse_status.
 */
int arfuse_launch_floor(int n_partials, int64_t t, int64_t d, int epilogue,
                        const arfuse_opts* opts, void* stream);

/*
 * arfuse_stream_copy — measurement aid: copy `bytes` (a multiple of 16) from
 * src to dst (device, 16-byte aligned, not overlapping) with the same
 * 16-byte streaming loads and stores the fused kernel uses; a reference for
 * achievable HBM bandwidth and for scaling hardware byte counters.
 */
int arfuse_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);

/*
 * arfuse_stream_mix — measurement aid: the fused call's byte mix without its
 * arithmetic, in its launch shape. For every row r < t, reads row r of each
 * of the n_in input planes (device, [t][d] 16-bit elements, 16-byte aligned)
 * and writes the XOR of them to row r of each of the n_out output planes
 * (device, [t][d], 16-byte aligned, overlapping no other plane). One
 * workgroup per row with the block and vectors per thread the fused call
 * uses for that t and d, non-temporal loads, and the fused call's
 * write-through stores where its rows take several rounds of workgroups,
 * else non-temporal stores; every load of a row is issued before the first
 * store. The time of a call is a reference for the fused call's memory
 * traffic at that shape: the same bytes without the arithmetic (Deep Dive
 * §6.1, §6.4: the fused kernel's cost is its HBM transactions). n_in in
 * [1, 9], n_out in [1, 3]; d % 16 == 0, d <= ARFUSE_MAX_D.
 */
int arfuse_stream_mix(const void* const* in, int n_in, void* const* out, int n_out, int64_t t,
                      int64_t d, void* stream);

/*
 * arfuse_round_bf16 — test entry: the fused kernel's fp32 -> bf16 rounding
 * (round to nearest even) applied to x (device fp32 [n], 8-byte aligned),
 * written to out (device bf16 bits [n], 4-byte aligned). n even.
 */
int arfuse_round_bf16(const float* x, int64_t n, uint16_t* out, void* stream);

/*
 * arfuse_round_fp8 — test entry: the fused kernel's FP8 conversion with
 * inv_scale 1 (E4M3FN, round to nearest even, sign kept, magnitudes above 448
 * saturating to 448) applied to x (device fp32 [n], 16-byte aligned), written
 * to out (device uint8 [n], 4-byte aligned). n a multiple of 4; x finite.
 */
int arfuse_round_fp8(const float* x, int64_t n, uint8_t* out, void* stream);

/*
 * arfuse_round_fp4 — test entry: the conversion the fused kernel's FP4
 * epilogue takes its E2M1 codes from where both ends of its reciprocal
 * envelope agree (gfx950's FP4 conversion with scale 1: nearest even,
 * saturating at 6, sign kept), applied to x (device fp32 [n], 8-byte
 * aligned), written to out (device uint8 [n/2]: x[2i] in the low nibble of
 * byte i, x[2i+1] in the high one). n even.
 */
int arfuse_round_fp4(const float* x, int64_t n, uint8_t* out, void* stream);

/* Static description of a status code. */
const char* arfuse_status_string(int status);

/* ARFUSE_VERSION of the built library. */
int arfuse_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ARFUSE_H */
