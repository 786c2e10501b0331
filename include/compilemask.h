/*
 * compilemask.h -- C ABI of the MI355X (gfx950) CompileMask hot path.
 *
 * What the library computes (CompileMask paper summary):
 *   - a MaskSpec groups query rows into Regions, each with a row guard and a
 *     visibility rule (section 3.2 "Offline Mask Specification and
 *     Compilation", section 3.2.1 "Mask Specification");
 *   - the spec is lowered once, offline, to visible-interval endpoints; the
 *     number of interval slots is derived per Region from its rule (section
 *     3.2.2 "Symbolic Lowering to Visible Intervals");
 *   - every batch, a preprocess kernel evaluates the endpoints against the
 *     batch metadata and writes an Execution Descriptor for the forward and
 *     the backward pass (section 3.3 "Online Efficient Mask Attention
 *     Execution"): an Interval Table of visible [start,end) intervals padded
 *     with zero-length intervals, plus two-bit-per-tile state bitmaps
 *     (section 3.3.1 "Execution Descriptor");
 *   - the attention kernels skip empty tiles, run full tiles without a mask
 *     and check visibility with unsigned endpoint compares only in partial
 *     tiles, replacing invisible scores by -inf before the online softmax
 *     (section 3.3.2 "Descriptor-Guided Attention Execution").
 *
 * Conventions shared by every entry point:
 *   - Ownership: the caller owns every device buffer (tensors, metadata, the
 *     descriptor buffer, the backward workspace) and the stream.  The library
 *     owns only the opaque host handles cm_spec and cm_desc.  It never
 *     allocates device memory.
 *   - Streams: `cm_stream` is a hipStream_t (NULL = the default stream).  The
 *     hot calls (cm_build_descriptor, cm_attn_fwd, cm_attn_bwd and
 *     cm_attn_bwd_stage) only enqueue kernels on it; they never synchronise.
 *     (cm_attn_bwd on short grids also uses a library stream, forked from
 *     and joined back to the caller's by events; see there.)
 *   - Errors: every call returns a cm_status.  A negative status means the
 *     call did nothing (no kernel launched, no output written); the detail is
 *     in cm_last_error() (thread-local, valid until the next call on the same
 *     thread).  No C++ exception crosses this boundary.
 *   - Errors found in the metadata on the device are not reported by the
 *     status: the preprocess kernel sets bits in the descriptor's header word
 *     13 and in sample_err[b], and gives that sample no visible pair at all.
 *
 * Descriptor byte layout (uint32 words, every section at a multiple of 256
 * bytes, gaps zero; Tq_f = ceil(N/fwd_q), Tk_f = ceil(N/fwd_k),
 * Tk_b = ceil(N/bwd_k), Tq_b = ceil(N/bwd_q)):
 *   header[16]     0x31444D43, B, N, K_r, K_c, fwd_q, fwd_k, bwd_k, bwd_q,
 *                  Tq_f, Tk_f, Tk_b, Tq_b, OR of sample_err, seg_cap, 0
 *   sample_err[B]  CM_MD_* bits of each sample's metadata
 *   row_tkmax[B][Tq_f]   largest run count among a forward query tile's rows
 *   col_tkmax[B][Tk_b]   largest run count among a backward key tile's columns
 *   fbm[B][Tq_f][ceil(Tk_f/16)]  forward Tile-State Bitmap (query tile major)
 *   bbm[B][Tk_b][ceil(Tq_b/16)]  backward Tile-State Bitmap (key tile major)
 *   row_iv[B][N][K_r][2]  per query row: visible key runs [start,end)
 *   col_iv[B][N][K_c][2]  per key column: visible query-row runs [start,end)
 * Tile codes: 0 empty, 1 full, 2 partial; tile c sits at bits 2*(c%16) of word
 * c/16.  Runs are maximal, ascending, and padded with (0,0) at the tail.  The
 * descriptor is per sample and shared by all heads.
 */
#ifndef COMPILEMASK_H
#define COMPILEMASK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct cm_spec cm_spec;  /* compiled MaskSpec (host, immutable)        */
typedef struct cm_desc cm_desc;  /* host handle over a caller-owned descriptor */
typedef void* cm_stream;         /* hipStream_t                                */

typedef enum cm_status {
  CM_OK = 0,
  CM_ERR_NULL = -1,        /* a required pointer is NULL                      */
  CM_ERR_INVALID = -2,     /* an argument is out of range                     */
  CM_ERR_PARSE = -3,       /* the spec text does not parse or lower           */
  CM_ERR_MISMATCH = -4,    /* descriptor and spec/arguments do not belong together */
  CM_ERR_UNSUPPORTED = -5, /* no kernel for this head dim / tile shape        */
  CM_ERR_SIZE = -6,        /* a caller buffer is too small                    */
  CM_ERR_HIP = -7          /* the HIP runtime reported an error               */
} cm_status;

/* Metadata error bits (descriptor header word 13 and sample_err[b]). */
#define CM_MD_NSEG 1u          /* n_seg outside [0, seg_cap]                   */
#define CM_MD_BOUNDS_ORDER 2u  /* a used boundary is smaller than the one before */
#define CM_MD_BOUNDS_RANGE 4u  /* a used boundary lies outside [0, N]          */
#define CM_MD_REF_RANGE 8u     /* a used reference lies outside [-1, n_seg)    */
#define CM_MD_CU_SEQLENS 16u   /* packed batch: cu_seqlens is not 0 = c[0] <= c[1]
                                  <= ... <= c[n] = total length                 */

#define CM_DESC_MAGIC 0x31444D43u

/* Tile shapes of the two descriptor grids.  Forward grid: fwd_q query rows x
 * fwd_k keys.  Backward grid: bwd_k keys x bwd_q query rows.  The preprocess
 * accepts any positive sizes; the attention kernels accept (fwd_q, fwd_k) in
 * {(64,64), (128,64)} and (bwd_k, bwd_q) in {(64,64), (128,64)}. */
typedef struct cm_tiles {
  int32_t fwd_q, fwd_k, bwd_k, bwd_q;
} cm_tiles;

/* Batch metadata: device int32 arrays, caller-owned, read by
 * cm_build_descriptor (CompileMask paper summary, section 1: mask boundaries
 * depend on sequence lengths and segment boundaries).
 *   scalars    [B][n_scalars]  the spec's `param` values, in declaration order
 *   seg_bounds [B][seg_cap+1]  segment s of sample b is
 *                              [seg_bounds[b][s], seg_bounds[b][s+1]), s < n_seg[b]
 *   n_seg      [B]
 *   refs       [B][seg_cap][n_refs]  referenced segment ids, -1 = none
 *   cu_seqlens [B+1]           packed batches only (else NULL): sample b holds
 *                              tokens [cu_seqlens[b], cu_seqlens[b+1]) of one
 *                              packed sequence
 * A pointer may be NULL when its array is empty (n_scalars == 0, seg_cap == 0
 * or n_refs == 0).  In a packed batch every sample's scalars and boundaries
 * are in the sample's own coordinates (its first token is 0 and its length
 * plays the part of N). */
typedef struct cm_metadata {
  const int32_t* scalars;
  const int32_t* seg_bounds;
  const int32_t* n_seg;
  const int32_t* refs;
  int32_t n_scalars;
  int32_t n_refs;
  const int32_t* cu_seqlens;
} cm_metadata;

/* Attention shapes.  q, k, v, o, dO, dq, dk, dv are bf16 [B][H][N][d] with
 * the last dimension contiguous and element strides stride_b, stride_h,
 * stride_n (all three 0 = contiguous [B,H,N,d]); lse is fp32 [B][H][N]
 * contiguous.  scale 0 means 1/sqrt(d).  causal = 1 selects the maskless
 * causal path (row i sees keys 0..i, tile states from indices, no descriptor:
 * desc may be NULL); causal = 0 uses the descriptor.  Size limits (else
 * CM_ERR_UNSUPPORTED): B * H * N <= 2^27 rows per call, and one head's rows,
 * ((N - 1) * stride_n + d) bf16, span less than 4 GiB. */
typedef struct cm_attn_args {
  int32_t B, H, N, d;
  int64_t stride_b, stride_h, stride_n;
  float scale;
  int32_t causal;
  int32_t check;      /* partial-tile visibility check, CM_CHECK_*; 0 = the default */
  int32_t precision;  /* P / dS operand precision, CM_PRECISION_*; 0 = the default */
} cm_attn_args;

/* Precision of the attention probabilities P and score gradients dS where
 * they enter a matrix product (O = P V forward; dV = P^T dO, dK = dS^T Q,
 * dQ = dS K backward).  The pages fix the result as plain masked softmax
 * attention (paper summary, sections 2.1 and 3.3.2); the inputs are bf16 and
 * every product accumulates in fp32.
 *   CM_PRECISION_BF16 (the default): P and dS rounded once to bf16 (a
 *     relative error of up to 2^-9 per element), as tiled attention kernels
 *     usually do.
 *   CM_PRECISION_SPLIT: P and dS enter as the sum of two bf16 values, hi =
 *     bf16(x) and lo = bf16(x - hi) (about 2^-17 relative error), so every
 *     product carries fp32 P and dS up to the order of accumulation; the
 *     four products take two matrix instructions per operand pair.  Only
 *     with CM_CHECK_RUN_BITS (else CM_ERR_UNSUPPORTED). */
#define CM_PRECISION_BF16 0
#define CM_PRECISION_SPLIT 1

/* Partial-tile visibility checks (cm_attn_args.check).  All give identical
 * results; they differ only in the instructions the kernels spend on it.
 *   CM_CHECK_RUN_BITS (the default): per partial tile, each visible run's
 *     endpoints are compared once against the tile's index range, giving
 *     the range of the lane's elements the run covers; the ranges form one
 *     visibility word, and each element costs a bit extract and a bit
 *     select, however many runs the row or column has.
 *   CM_CHECK_UNSIGNED: visible runs, one subtraction (hoisted per row) and one
 *     unsigned compare per run and element (paper summary, section 3.3.2).
 *   CM_CHECK_ORDINARY_MASKED: the ablation of section 4.4 / Table 3 there:
 *     masked intervals (the complement of the visible runs) with two ordinary
 *     compares and their conjunction per interval.  For measurement only. */
#define CM_CHECK_RUN_BITS 0
#define CM_CHECK_ORDINARY_MASKED 1
/*   CM_CHECK_PREDICATE: the predicate baseline (see cm_build_blockmask); the
 *     descriptor must come from cm_build_blockmask. */
#define CM_CHECK_PREDICATE 2
#define CM_CHECK_UNSIGNED 3

/* ---- offline: MaskSpec -> symbolic endpoints (section 3.2.2) ------------ */

/* Parse and lower a MaskSpec text (grammar in the package's spec docs: one
 * `forward` and one `backward` section of `region NAME: GUARD => RULE`
 * lines).  Lowering: AST, negation pushed to atoms, DNF, one interval per
 * conjunct, canonicalisation (redundant bounds dropped, provably empty
 * conjuncts dropped, conjuncts with the same interval merged, adjacent
 * intervals merged when provable over the whole Region).  On success *out
 * owns a new spec (free with cm_spec_free); it is immutable and may be
 * shared by threads.  CM_ERR_PARSE on any syntax or lowering error. */
cm_status cm_spec_compile(const char* text, cm_spec** out);
void cm_spec_free(cm_spec* spec);

/* Interval-table widths the spec needs for a segment capacity: K_row (query
 * rows, forward) and K_col (key columns, backward) = the largest slot count
 * of any Region of that direction; an `exists` slot counts seg_cap slots.
 * Also the number of scalars and references the metadata must carry. */
cm_status cm_spec_info(const cm_spec* spec, int32_t seg_cap, int32_t* K_row, int32_t* K_col,
                       int32_t* n_scalars, int32_t* n_refs);

/* Human-readable listing of the lowered program (regions, slots, bounds,
 * conditions) into buf (NUL-terminated, truncated to len).  *needed gets the
 * full length + 1 when non-NULL. */
cm_status cm_spec_dump(const cm_spec* spec, char* buf, size_t len, size_t* needed);

/* Evaluate one index on the host (inspection aid; not used by any other
 * entry point): the visible runs of query row `index` (direction 0) or key
 * column `index` (direction 1) of ONE sample whose metadata is given in host
 * arrays (scalars[n_scalars], seg_bounds[seg_cap+1], refs[seg_cap][n_refs]).
 * Writes up to `cap` pairs to runs[2*cap] and their count to *n_runs.
 * Metadata errors give *md_err != 0 and no runs. */
cm_status cm_spec_eval_host(const cm_spec* spec, int32_t direction, int32_t N, int32_t index,
                            const int32_t* scalars, int32_t n_scalars, const int32_t* seg_bounds,
                            int32_t n_seg, int32_t seg_cap, const int32_t* refs, int32_t n_refs,
                            uint32_t* runs, int32_t cap, int32_t* n_runs, uint32_t* md_err);

/* ---- descriptor memory (caller-owned) ---------------------------------- */

/* Bytes of a descriptor for (spec, B, N, seg_cap, tiles): the Execution
 * Descriptor of paper summary section 3.3.1 (interval tables padded to the
 * spec's slot counts, two-bit tile states per direction) in the layout at the
 * top of this header.  Host only; CM_ERR_INVALID for sizes out of range. */
cm_status cm_desc_size(const cm_spec* spec, int32_t B, int32_t N, int32_t seg_cap,
                       const cm_tiles* tiles, size_t* bytes);

/* Bind a caller-owned device buffer of at least cm_desc_size() bytes to a new
 * descriptor handle and zero it (synchronously, once).  The handle does not
 * own dev_buf; free the handle with cm_desc_free and the buffer yourself.
 * The descriptor is bound to one spec, batch shape and tile shape and is
 * rebuilt from each batch's metadata (paper summary sections 3.1 and 3.3: the
 * spec is compiled once, the descriptor is produced online per batch).
 * CM_ERR_SIZE when bytes is too small, CM_ERR_INVALID when dev_buf is not
 * 256-byte aligned. */
cm_status cm_desc_init(const cm_spec* spec, int32_t B, int32_t N, int32_t seg_cap,
                       const cm_tiles* tiles, void* dev_buf, size_t bytes, cm_desc** out);
void cm_desc_free(cm_desc* desc);

/* Packed variable-length batches (cu_seqlens style).  n_samples sequences
 * are laid end to end as one sequence of T tokens; a token attends only to
 * its own sample's keys, under the spec's rules in the sample's coordinates.
 * The descriptor covers that one sequence (its header has B = 1, N = T and
 * word 15 = n_samples; sample_err has n_samples words), so attention runs
 * with cm_attn_args B = 1, N = T on [1][H][T][d] tensors (or [T][H][d] via
 * the strides); tiles that straddle two samples are partial.  Build it with
 * cm_build_descriptor and metadata whose cu_seqlens is set.  Same ownership
 * and errors as cm_desc_size / cm_desc_init. */
cm_status cm_desc_size_packed(const cm_spec* spec, int32_t n_samples, int32_t T, int32_t seg_cap,
                              const cm_tiles* tiles, size_t* bytes);
cm_status cm_desc_init_packed(const cm_spec* spec, int32_t n_samples, int32_t T, int32_t seg_cap,
                              const cm_tiles* tiles, void* dev_buf, size_t bytes, cm_desc** out);

/* Byte offsets of the descriptor sections, in layout order: header,
 * sample_err, row_tkmax, col_tkmax, fbm, bbm, row_iv, col_iv; then the
 * total size.  offsets must hold 9 entries. */
cm_status cm_desc_offsets(const cm_desc* desc, size_t* offsets);

/* Spec-specialised preprocess (paper summary, sections 1 and 3.1: the spec
 * is compiled once, every batch reuses the result).  cm_spec_specialize
 * generates a preprocess kernel in which this spec's lowered program is a
 * compile-time constant, compiles it with hipRTC for gfx950 (about a second)
 * and loads it on the current device; from then on cm_build_descriptor with
 * this spec on that device launches it instead of the interpreting kernel.
 * The descriptor is bit-identical.  Synchronous, host side; a repeated call
 * for the same device returns at once.  Threads may call it, and use the spec
 * in other calls, concurrently.  The modules are unloaded by cm_spec_free.  CM_ERR_HIP
 * (with the compiler log in cm_last_error) if hipRTC or the loader fails.
 * cm_spec_codegen returns the generated source (same conventions as
 * cm_spec_dump). */
cm_status cm_spec_specialize(cm_spec* spec);
cm_status cm_spec_codegen(const cm_spec* spec, char* buf, size_t len, size_t* needed);

/* ---- online, every batch (section 3.3) --------------------------------- */

/* One preprocess kernel launch (paper summary section 3.3 "Online Efficient
 * Mask Attention Execution", with the descriptor contents of section 3.3.1):
 * evaluate the compiled endpoints of `spec` against `md` and write the whole
 * descriptor (header, both interval tables, both bitmaps, per-tile run
 * maxima, error words).  desc must come from
 * cm_desc_init (md->cu_seqlens NULL) or cm_desc_init_packed (md->cu_seqlens
 * set) with the same spec.  Asynchronous on `stream`. */
cm_status cm_build_descriptor(const cm_spec* spec, const cm_metadata* md, cm_desc* desc,
                              cm_stream stream);

/* ---- predicate baseline (for measurement; paper summary, sections 1, 4.2) */

/* The masking the CompileMask pages compare against (FlexAttention style):
 * the mask as a predicate of (row i, key j), a block mask built per batch by
 * evaluating it at every element, and the predicate evaluated again at every
 * element of a partial tile, reading its inputs (each token's segment, a
 * segment's references) from memory.  Families (CM_PRED_*), as the workloads
 * define them, with s = metadata scalars[b][0]:
 *   CM_PRED_CAUSAL         j <= i
 *   CM_PRED_HSTU           i < s ? j <= i : (j < s || j == i)
 *   CM_PRED_SHARED_PROMPT  i < s ? j <= i : (j < s || (seg(i) >= 0 && seg(j) == seg(i) && j <= i))
 *   CM_PRED_RETRIEVAL      i < s ? j <= i : (j < s || seg(i) >= 0 && seg(j) >= 0 &&
 *                          ((seg(j) == seg(i) && j <= i) || seg(j) is a reference of seg(i)))
 *                          (at most 2 references per segment)
 * cm_build_blockmask writes both tile bitmaps, the error words and the
 * header of a descriptor from cm_desc_init (any spec; padded batches; tiles
 * of at most 128 rows/keys) and keeps each token's segment in its row_iv
 * section; the interval tables are not built.  The descriptor then refers to
 * md's scalars and refs: they must stay unchanged until the attention calls
 * that use it (with check = CM_CHECK_PREDICATE) have run.  Two launches on
 * `stream`; the bitmaps equal those cm_build_descriptor makes for the same
 * mask. */
#define CM_PRED_CAUSAL 0
#define CM_PRED_HSTU 1
#define CM_PRED_SHARED_PROMPT 2
#define CM_PRED_RETRIEVAL 3
cm_status cm_build_blockmask(int32_t family, const cm_metadata* md, cm_desc* desc, cm_stream stream);

/* Forward (paper summary section 3.3.2 "Descriptor-Guided Attention
 * Execution": empty tiles skipped, full tiles unmasked, endpoint checks in
 * partial tiles, invisible scores set to -inf before the online softmax):
 * o (bf16) and lse (fp32, natural log; -inf for a row with no visible key,
 * whose o row is 0).  q, k, v, o follow args' layout; every pointer is a
 * caller-owned device pointer, 16-byte aligned.  Requires d in {64, 128} and
 * a descriptor whose forward tiles are supported (CM_ERR_UNSUPPORTED), built
 * for args' B and N (CM_ERR_MISMATCH).  Asynchronous on `stream`. */
cm_status cm_attn_fwd(const cm_attn_args* args, const void* q, const void* k, const void* v,
                      const cm_desc* desc, void* o, float* lse, cm_stream stream);

/* Bytes of fp32 workspace cm_attn_bwd needs: per row, rowsum(dO * O) and
 * the row's lse in log2 units (2 * B * H * N floats). */
cm_status cm_attn_bwd_workspace(const cm_attn_args* args, size_t* bytes);

/* Backward from the forward's o and lse: dq, dk, dv (bf16).  Training
 * throughput counts forward and backward (paper summary section 1), and the
 * backward follows its own descriptor direction (section 3.3: per key column,
 * with the backward spec's intervals).  Three kernels: D = rowsum(dO * O);
 * dK/dV per key tile over the query tiles that the backward bitmap marks
 * non-empty (column runs in partial tiles); dQ per query tile over the
 * forward bitmap (row runs).  Deterministic (no atomics).  All of it is
 * ordered after earlier work on `stream` and before later work on it: when
 * B * H * N <= 131072 the library runs dQ beside dK/dV on a stream of its
 * own (one per device, created on the first such call outside a graph
 * capture; a capture takes the fork and join along), with the same results.
 * The workspace (caller-owned device memory of cm_attn_bwd_workspace bytes,
 * else CM_ERR_SIZE) holds D and the log2 lse between the kernels; same
 * argument checks as cm_attn_fwd. */
cm_status cm_attn_bwd(const cm_attn_args* args, const void* q, const void* k, const void* v,
                      const void* o, const float* lse, const void* dO, const cm_desc* desc,
                      void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                      cm_stream stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, allocation-free serving loops, harnesses that forbid hipMalloc):
 * cm_attn_bwd with the workspace taken from a fixed array inside the library
 * instead of a caller buffer.  The array holds D and the log2 lse of
 * CM_NOALLOC_MAX_ROWS rows (16 MiB); every GPU the library runs on keeps its
 * own copy until the process ends.  Its device address is looked up on the
 * first call on each device; the call allocates and frees nothing.  Calls on
 * one GPU share the array: two calls that overlap in time on the same GPU
 * (other streams, other threads) race and give wrong results; calls in order
 * on one stream are safe.  Every row the kernels read is written by the same
 * call first, so nothing needs clearing.  CM_ERR_SIZE when B * H * N exceeds
 * CM_NOALLOC_MAX_ROWS; otherwise the same arguments, checks, kernels and
 * results as cm_attn_bwd, all three kernels on `stream` (no library stream). */
#define CM_NOALLOC_MAX_ROWS (1 << 21)
cm_status cm_attn_bwd_noalloc(const cm_attn_args* args, const void* q, const void* k, const void* v,
                              const void* o, const float* lse, const void* dO, const cm_desc* desc,
                              void* dq, void* dk, void* dv, cm_stream stream);

/* One of the three backward kernels alone, same arguments as cm_attn_bwd
 * (stage 0: D, stage 1: dK/dV, stage 2: dQ), for per-kernel timing.  Running
 * stages 0, 1, 2 in order equals cm_attn_bwd. */
cm_status cm_attn_bwd_stage(int32_t stage, const cm_attn_args* args, const void* q, const void* k,
                            const void* v, const void* o, const float* lse, const void* dO,
                            const cm_desc* desc, void* dq, void* dk, void* dv, void* workspace,
                            size_t workspace_bytes, cm_stream stream);

/* ---- test and debug (synchronising) ------------------------------------ */

/* Copy the whole descriptor (cm_desc_offsets' total) into host memory:
 * enqueued on `stream` after the work already there, then the stream is
 * synchronised.  The descriptor of paper summary section 3.3.1, in the byte
 * layout at the top of this header.  CM_ERR_SIZE when bytes is smaller than
 * the descriptor; CM_ERR_HIP if the copy fails.  Not for the hot path. */
cm_status cm_desc_download(const cm_desc* desc, void* host, size_t bytes, cm_stream stream);

/* The metadata errors the preprocess found (paper summary section 3.1: the
 * descriptor is built on the device from each batch's metadata, so errors
 * there are found on the device): *flags = header word 13, the OR of the
 * CM_MD_* bits of every sample (0 = valid metadata); with per_sample non-NULL
 * also each sample's word (B words, or n_samples for a packed descriptor;
 * n_per_sample gives that count when non-NULL).  Reads after the work already
 * on `stream` and synchronises it.  Not for the hot path. */
cm_status cm_desc_errors(const cm_desc* desc, uint32_t* flags, uint32_t* per_sample, int32_t* n_per_sample,
                         cm_stream stream);

/* ---- diagnostics -------------------------------------------------------- */
const char* cm_status_str(cm_status status);
const char* cm_last_error(void);
/* Library version string and the gfx target it was built for. */
const char* cm_version(void);

#ifdef __cplusplus
}
#endif
#endif /* COMPILEMASK_H */
