/*
 * deltalog.h -- C ABI of the MI355X (gfx950) decode-time recurrent-state
 * library for gated delta-rule linear attention.
 *
 * The operation (the DeltaLog page, "DeltaLog: Deferred Materialization of
 * Recurrent States for Linear Attention Decoding", Technical Summary):
 *
 *   Problem:   every decode step folds one token's compact update (q, k, v,
 *              a decay and, for delta-rule operators, a write strength beta)
 *              into a fixed-size per-head state; eager decoding rewrites the
 *              whole dense state to HBM each step.
 *   Operators (Kernel Implementation): head-wise scalar decay with the
 *              delta-rule correction (Gated DeltaNet), per-key decay with the
 *              correction (KDA), per-key decay with raw-value updates (RWKV6).
 *   Core Mechanism: the live state is a dense base plus a bounded log of
 *              compact updates; appends leave the base untouched, and a
 *              periodic merge materialises base + log into a new base.
 *
 * With S the d_v x d_k state of one (sequence, head) -- row i = value
 * channel, column j = key channel -- and alpha = exp(g):
 *
 *   GDN    S' = alpha S (I - beta k k^T) + beta v k^T
 *   KDA    S' = S diag(alpha) (I - beta k k^T) + beta v k^T
 *   RWKV6  S' = S diag(w) + v k^T          (w = exp(g), per key channel)
 *   GDN2   S' = S diag(alpha) (I - (e * k) k^T) + (w * v) k^T
 *          (the gated form of the Gated DeltaNet-2 and FG2-GDN abstracts:
 *          KDA's beta split into a channel-wise erase gate e on the key
 *          channels and a write gate w on the value channels; KDA when both
 *          are the same scalar)
 *   every step reads out o = S' q.
 *
 * Memory.  The caller owns all device memory (e.g. torch tensors): one state
 * block of dl_state_bytes() bytes, and every input and output.  The handle
 * holds host metadata only; the memory must outlive it.
 *
 * Streams.  Every call that launches work is asynchronous on `stream` (a
 * hipStream_t passed as void*, NULL = the null stream) and never
 * synchronises, except dl_state_check.  Use one handle from one stream at a
 * time.
 *
 * Rows.  A step call processes `rows` sequences at once.  Input row r
 * updates state unit slot_idx[r] (a device int32 array), or unit r when
 * slot_idx is NULL (then rows <= units).  Two rows of one call must not
 * name the same unit (undefined result).  A slot index outside [0, units)
 * makes that row write NaN to its outputs, leave every state untouched and
 * raise DL_FLAG_BAD_SLOT.
 *
 * Errors.  Host-side validation failures return a non-zero dl_status
 * without launching anything; dl_last_error() describes the latest one on
 * the calling thread.  Conditions only the GPU can see set bits in a device
 * flag word that dl_state_check() reads.  Faults in device code surface at
 * the caller's next synchronisation.  No C++ exception crosses this ABI.
 */
#ifndef DELTALOG_H
#define DELTALOG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DL_OK = 0,
    DL_ERR_INVALID = 1,      /* null or misaligned pointer, bad count, argument wrong for the variant */
    DL_ERR_UNSUPPORTED = 2,  /* well-formed but not built: d_k != d_v, d not in {64, 128}, L > 64,
                              * a GDN2 log in the WY form, an INT8 base without a
                              * factor-form log of a delta-rule variant, an eager step
                              * on an INT8 base */
    DL_ERR_SIZE = 3,         /* caller memory smaller than dl_state_bytes() */
    DL_ERR_LAUNCH = 4,       /* the HIP runtime rejected a launch or copy */
    DL_ERR_STATE = 5         /* dl_state_check found device flags set */
} dl_status;

typedef enum {
    DL_GDN = 0,              /* head-wise decay, delta rule */
    DL_KDA = 1,              /* per-key decay, delta rule */
    DL_RWKV6 = 2,            /* per-key decay, raw-value updates */
    DL_GDN2 = 3              /* per-key decay, delta rule with a channel-wise erase
                              * gate e (key channels) and write gate w (value
                              * channels); DeltaLog only with DL_LOG_FACTORS */
} dl_variant;
typedef enum { DL_F32 = 0, DL_BF16 = 1 } dl_dtype;

/* What the log stores per pending step (dl_desc.log_form). */
typedef enum {
    DL_LOG_WY = 0,           /* bit copies of (k, v), beta, the decay and the
                              * key-side factors R of the compact WY readout */
    DL_LOG_FACTORS = 1       /* the additive factors (a_t, b_t = k_t) and the
                              * decay: a_t = beta_t (v_t - S_{t-1}(alpha_t k_t)),
                              * fp32; RWKV6's raw-value log is already of this
                              * form (a_t = v_t), so both values give it the
                              * same log */
} dl_log_form;

typedef enum {
    DL_MERGE_FULL = 0,       /* merge units whose log holds exactly L entries */
    DL_MERGE_ALL = 1         /* merge every unit with a non-empty log (flush) */
} dl_merge_mode;

/* Device flag bits (dl_state_check). */
#define DL_FLAG_LOG_FULL   0x1  /* dl_decode_step_log met a full log: row skipped, o = NaN */
#define DL_FLAG_LOG_NONEMPTY 0x2 /* dl_decode_step_eager met a non-empty log: row skipped, o = NaN */
#define DL_FLAG_BAD_SLOT   0x4  /* a slot index outside [0, units): row skipped, o = NaN */
#define DL_FLAG_BAD_KEPT   0x8  /* kept-channel indices not increasing in [0, d_k): row skipped */

/* How the dense base is stored (dl_desc.base_format). */
typedef enum {
    DL_BASE_F32 = 0,         /* fp32 [units, H, d_v, d_k] */
    DL_BASE_I8 = 1           /* mixed precision (a reading of the DAMP abstract, "DAMP:
                              * Decay-Aware Mixed-Precision Recurrent-State
                              * Quantization", Jianchao Tan author page: most of the state
                              * in INT8, a few channels chosen offline kept at higher
                              * precision): kept_channels key channels per head stay
                              * fp32; every other entry is a symmetric INT8 code with one
                              * fp32 scale per value row, scale_i = max |S_ij| / 127 over
                              * the coded columns, code_ij = clip(rint(S_ij / scale_i),
                              * -127, 127) (fp32 divisions, ties to even; all codes 0 for
                              * a zero row), kept columns coded 0.  The base is quantised
                              * on dl_base_import and at every merge, from the fp32
                              * merged state; steps read it as code * scale.  Factor-form
                              * logs of the delta-rule variants only. */
} dl_base_format;

/* Shape of one state block. */
typedef struct {
    int32_t variant;   /* dl_variant */
    int32_t units;     /* state slots (sequences), >= 1 */
    int32_t heads;     /* heads per unit, >= 1 */
    int32_t d_k;       /* key channels: 64 or 128 */
    int32_t d_v;       /* value channels: must equal d_k */
    int32_t log_len;   /* L, log slots per (unit, head): 0 (eager only) .. 64 */
    int32_t in_dtype;  /* dl_dtype of q, k, v and of the logged k, v copies */
    int32_t merge_on_step; /* 0: a full log waits for dl_merge; 1: the log step
                            * that fills a log also merges it into the base in
                            * the same pass and leaves fill at 0 (that entry
                            * is not written to the log) */
    int32_t log_form;  /* dl_log_form */
    int32_t base_format;   /* dl_base_format (0: fp32) */
    int32_t kept_channels; /* DL_BASE_I8: key channels per head kept in fp32, 0 .. 16 */
} dl_desc;

/* Device pointers into a state block (all row-major, contiguous).
 *   base     [units, H, d_v, d_k] fp32  -- the dense state (eager) or base (DeltaLog)
 *   log_k    [units, H, L, d_k] in_dtype -- logged keys, bit copies of the inputs
 *   log_v    [units, H, L, d_v] in_dtype -- logged values; under DL_LOG_FACTORS
 *            (GDN, KDA) fp32 -- the factors a_t
 *   log_g    [units, H, L] (GDN) or [units, H, L, d_k] (KDA, RWKV6, GDN2) fp32 -- the
 *            log-decay accumulated from the log's first entry through each
 *            entry (Lam_j = Lam_{j-1} + g_j in fp32, Lam_{-1} = 0)
 *   log_beta [units, H, L] fp32 (NULL for RWKV6 and under DL_LOG_FACTORS)
 *   log_t    [units, H, L(L-1)/2] fp32 -- key-side factors of the log (delta-
 *            rule variants): the inverse R of the unit upper-triangular
 *            coupling matrix of the logged entries, column j (rows 0..j-1)
 *            at offset j(j-1)/2, written when entry j is appended and read
 *            by every readout (NULL for RWKV6, under DL_LOG_FACTORS and
 *            when L < 2)
 *   fill     [units, H] int32 -- entries in each log; every head of a unit
 *            advances together, one writer per counter
 *   flags    [1] int32 -- DL_FLAG_* bits
 *   base_codes [units, H, d_v, d_k] int8, base_scale [units, H, d_v] fp32,
 *   base_kept [units, H, d_v, M] fp32 (M = kept_channels), kept_idx [H, M]
 *            int32 -- the DL_BASE_I8 base (then `base` is NULL; these are NULL
 *            for DL_BASE_F32): codes, row scales, the kept channels' values
 *            and their column indices, strictly increasing in [0, d_k), the
 *            same for every unit of a head.  dl_state_alloc sets kept_idx to
 *            evenly spaced channels (m d_k / M + d_k / (2 M)); write other
 *            indices through this view before the first import or step.
 * log_* are NULL when L == 0. */
typedef struct {
    float *base;
    void *log_k;
    void *log_v;
    float *log_g;
    float *log_beta;
    float *log_t;
    int32_t *fill;
    int32_t *flags;
    int8_t *base_codes;
    float *base_scale;
    float *base_kept;
    int32_t *kept_idx;
} dl_state_ptrs;

typedef struct dl_state dl_state;   /* opaque host handle */

/* State block (the DeltaLog page, Technical Summary, Core Mechanism: Base +
 * Log -- the live state of each head is a dense base plus a bounded log of
 * compact updates with their log-decay metadata, with a per-log fill count).
 * One block holds, for every (unit, head), the fp32 base, the L log slots
 * and the fill counter, laid out as dl_state_ptrs describes.
 *
 * Bytes of device memory a state block of this shape needs (0 if the
 * descriptor is invalid or unsupported; dl_last_error() says why). */
size_t dl_state_bytes(const dl_desc *desc);

/* Bind a state block (Core Mechanism: Base + Log, as above) to caller
 * memory `dev_mem` (device memory, 256-byte aligned, at least
 * dl_state_bytes(desc) bytes; the caller keeps ownership and must keep it
 * alive until dl_state_free) and zero all of it on `stream` (base = 0, logs
 * empty, flags clear).  Write an initial base through dl_state_view after
 * this call (on the same stream, or after synchronising).  On success *out
 * owns a new host handle; free it with dl_state_free.  Errors: DL_ERR_INVALID
 * (NULL or misaligned memory, bad descriptor), DL_ERR_UNSUPPORTED, DL_ERR_SIZE
 * (bytes too small), DL_ERR_LAUNCH (the zeroing launch failed); *out is then
 * NULL and nothing was launched except, for DL_ERR_LAUNCH, the failed zeroing. */
dl_status dl_state_alloc(const dl_desc *desc, void *dev_mem, size_t bytes, void *stream,
                         dl_state **out);

/* Release the host handle of a state block (Core Mechanism: Base + Log); the
 * device memory stays the caller's.  NULL is accepted.  Launches already
 * issued with the handle keep running; the handle itself is no longer
 * touched by them. */
dl_status dl_state_free(dl_state *st);

/* Device pointers of the block's parts (Core Mechanism: Base + Log: the base,
 * the log's keys, values or factors, log-decay metadata, betas, key-side
 * factors and fill counts), written into the caller's dl_state_ptrs struct
 * (one struct instead of one out-parameter per part).  The pointers stay
 * valid as long as the caller's memory does.  Errors: DL_ERR_INVALID for a
 * NULL handle or out. */
dl_status dl_state_view(const dl_state *st, dl_state_ptrs *out);

/* Eager step (the "eager" decoding the DeltaLog page's Problem section
 * describes): for each row, read the dense state once, apply the operator,
 * write the whole state back and emit o = S' q.  The unit's log must be
 * empty (else DL_FLAG_LOG_NONEMPTY).
 *   q, k   [rows, H, d_k] in_dtype         v [rows, H, d_v] in_dtype
 *   g      [rows, H] (GDN) or [rows, H, d_k] (KDA, RWKV6, GDN2) fp32 log-decay
 *   beta   [rows, H] fp32 (GDN, KDA; ignored and may be NULL for RWKV6);
 *          GDN2: [rows, H, d_k + d_v] fp32, the erase gate then the write gate
 *   o      [rows, H, d_v] fp32 output (must not alias any input or the state)
 * q, k, v, g, o must be 16-byte aligned; beta and slot_idx 4-byte aligned
 * (beta 16-byte aligned for GDN2). */
dl_status dl_decode_step_eager(dl_state *st, int32_t rows, const int32_t *slot_idx,
                               const void *q, const void *k, const void *v, const float *g,
                               const float *beta, float *o, void *stream);

/* DeltaLog step (the page's Append Phase): append (k, v, g, beta) to slot
 * fill of each row's log without writing the base, then read out
 * o = S_logical q from the read-only base plus the log, the new entry
 * included.  Under DL_LOG_FACTORS the entry is (a_t, k_t, the decay), with
 * a_t read from base + log in the same pass; the readout is then base
 * (E q) plus one independent dot product per entry.  When the log now holds
 * L entries it is full: call dl_merge (DL_MERGE_FULL) before the unit's next
 * step, or that step is skipped with DL_FLAG_LOG_FULL.  Arguments as for
 * dl_decode_step_eager; needs L >= 1.  g must be finite: the log keeps the
 * decay accumulated since its first entry (log_g) in fp32, and the decay
 * between two entries is the exponential of a difference of those sums, so
 * its relative rounding error is about 6e-8 times the sum's magnitude (1e-5
 * at a sum of -170 over one log). */
dl_status dl_decode_step_log(dl_state *st, int32_t rows, const int32_t *slot_idx,
                             const void *q, const void *k, const void *v, const float *g,
                             const float *beta, float *o, void *stream);

/* The two steps above with the order of their workgroups given: workgroups
 * start in block order, and block b serves input row row_order[b] (all its
 * heads), so the caller decides which rows start first -- e.g. rows whose log
 * the step fills and, with merge_on_step, merges in place, whose workgroups
 * run longer, spread through the launch or placed ahead of the rest -- without
 * reordering any input or output in memory.  row_order is a device int32
 * array of `rows` entries, a permutation of 0 .. rows - 1, 4-byte aligned;
 * NULL gives input order (the plain calls above).  An entry outside
 * [0, rows) skips its block and raises DL_FLAG_BAD_SLOT; a repeated entry
 * (then some row is missing) is undefined, as for slot_idx.  Results do not
 * depend on the order.  This is a scheduling choice for the launches the
 * DeltaLog page's Kernel Implementation describes (one pass over the
 * batch's states per step). */
dl_status dl_decode_step_eager_ordered(dl_state *st, int32_t rows, const int32_t *slot_idx,
                                       const int32_t *row_order, const void *q, const void *k,
                                       const void *v, const float *g, const float *beta, float *o,
                                       void *stream);
dl_status dl_decode_step_log_ordered(dl_state *st, int32_t rows, const int32_t *slot_idx,
                                     const int32_t *row_order, const void *q, const void *k,
                                     const void *v, const float *g, const float *beta, float *o,
                                     void *stream);

/* Merge (the page's Merge Phase): materialise base + log into the base and
 * empty the log, for the selected rows' units (DL_MERGE_FULL: units whose
 * log holds L entries; DL_MERGE_ALL: every non-empty log).  The update is
 * applied in WY/UT form -- the logged rank-one transforms folded into one
 * triangular solve and two dense contractions on the matrix cores -- the
 * block form the CARVE page (abstract) and Gated DeltaNet-2 (chunkwise WY
 * algorithm) use.  Under DL_LOG_FACTORS the log already holds the solved
 * factors: base' = base diag(E_c) + sum_j a_j (k_j E_c / E_j)^T, one
 * contraction. */
dl_status dl_merge(dl_state *st, int32_t rows, const int32_t *slot_idx, int32_t mode,
                   void *stream);

/* Same result as dl_merge, computed by replaying the logged steps one by
 * one on the vector ALUs (a cross-check of the WY path; also a fallback for
 * callers who prefer its rounding).  Under DL_LOG_FACTORS there is nothing
 * to replay: the same contraction as dl_merge. */
dl_status dl_merge_replay(dl_state *st, int32_t rows, const int32_t *slot_idx, int32_t mode,
                          void *stream);

/* Write the bases of the rows' units from fp32 states src [rows, H, d_v, d_k]
 * (device, 16-byte aligned, read-only): a copy for DL_BASE_F32, the
 * quantisation described at DL_BASE_I8 otherwise (the dense base of the
 * DeltaLog page's Core Mechanism, stored as DL_BASE_I8 says).  Logs and
 * fill counts are left as they are: import into empty logs.  Errors as for
 * the step calls (DL_ERR_INVALID for NULL or misaligned pointers). */
dl_status dl_base_import(dl_state *st, int32_t rows, const int32_t *slot_idx, const float *src,
                         void *stream);

/* The bases of the rows' units as fp32 states dst [rows, H, d_v, d_k]
 * (device, 16-byte aligned): a copy, or code * scale with the kept channels'
 * values for DL_BASE_I8.  This is the base alone: after dl_merge with
 * DL_MERGE_ALL it is the logical state (the DeltaLog page, Core Mechanism:
 * the merge materialises base + log). */
dl_status dl_base_export(dl_state *st, int32_t rows, const int32_t *slot_idx, float *dst,
                         void *stream);

/* Readout without an update: o = S_logical q for each row's unit, from the
 * base and whatever the log holds (for an eager state, o = S q) -- the
 * readout o = S q of the DeltaLog page's Technical Summary (Problem), taken
 * here as a query of the current logical state with no token folded in (the
 * plainest reading of a readout call beside the step calls; the final state
 * itself is read after dl_merge with DL_MERGE_ALL, through dl_state_view).
 *   q [rows, H, d_k] in_dtype (16-byte aligned), o [rows, H, d_v] fp32
 *   (16-byte aligned, must not alias q or the state).  Errors as for the step
 * calls; a full or empty log is valid here. */
dl_status dl_readout(dl_state *st, int32_t rows, const int32_t *slot_idx, const void *q,
                     float *o, void *stream);

/* Synchronise `stream`, copy the device flag word to *flags_out (may be
 * NULL), clear it, and return DL_ERR_STATE if any bit was set. */
dl_status dl_state_check(dl_state *st, void *stream, int32_t *flags_out);

/* Profiling hook: the next kernel this handle launches records `start_event`
 * and `stop_event` (hipEvent_t values the caller created, with timing) at
 * its own dispatch begin and end, so hipEventElapsedTime between them is
 * that kernel's execution time alone, without launch gaps.  One-shot: the
 * next launching call consumes them (calls that launch nothing leave them
 * armed); NULL, NULL disarms.  The events must belong to the same device
 * and HIP runtime as the stream. */
dl_status dl_time_next_launch(dl_state *st, void *start_event, void *stop_event);

/* Message for the latest non-OK status on this thread ("" if none). */
const char *dl_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t dl_version(void);

/* Log length with the lowest modeled cost per state update for the shape in
 * `desc` (variant, d_k, d_v, in_dtype, merge_on_step, log_form;
 * desc->log_len and the unit and head counts are ignored).  The model is the
 * traffic the method must move per update -- the base read, the logged
 * entries read back, the append, the key-side factors and the amortised merge
 * (one base write per L steps, in place of that step's append, when
 * merge_on_step is set, else a separate read + write of the base and the
 * log) -- divided by the share of its bandwidth-bound rate the step
 * kernel keeps at that L: it needs four workgroups per CU, and fewer fit once
 * the staged log outgrows a quarter of the CU's 160 KiB LDS.  This is the
 * merge-interval trade-off of the DeltaLog page's Traffic Model, made
 * concrete for this kernel.  Candidates are 1..64; ties go to the smaller L.
 * Writes the choice to *L_out and, if bytes_out is not NULL, the modeled
 * bytes per update (before the occupancy factor) to *bytes_out.
 * Errors: DL_ERR_INVALID / DL_ERR_UNSUPPORTED as dl_state_bytes would report
 * for the descriptor with log_len = 1, or a NULL L_out. */
dl_status dl_suggest_log_len(const dl_desc *desc, int32_t *L_out, double *bytes_out);

/* Whether the kernels of a state with this descriptor move its base with
 * nontemporal (streaming) loads and stores: an eager state larger than the
 * 256 MiB Infinity Cache, or a base and log together larger than 384 MiB
 * (every log step reads both; streaming the base keeps the log entries
 * cached).  A cache policy only: results are identical either way.  Host
 * only, no GPU needed.  Writes 1 or 0 to *streams_out.  Errors:
 * DL_ERR_INVALID / DL_ERR_UNSUPPORTED as dl_state_bytes would report for the
 * descriptor, or a NULL streams_out. */
dl_status dl_state_streams(const dl_desc *desc, int32_t *streams_out);

/* Streaming-rate calibration, not part of the method: one launch that only
 * moves bytes, in the access pattern of the state kernels' largest stream
 * (16-byte nontemporal loads, 256 threads per workgroup), so that a kernel's
 * achieved rate can be set beside what a plain kernel reaches on this memory
 * system as well as beside the published peak.
 *   DL_PROBE_READ: reads `bytes` of `src` and writes, per 32 KiB of it, the
 *     float32 sum of that block's float32 values to `dst` (dst holds
 *     ceil(bytes / 32768) floats);
 *   DL_PROBE_COPY: copies `bytes` of `src` to `dst` (non-overlapping).
 * src and dst are device pointers (caller-owned, 16-byte aligned); bytes is
 * a positive multiple of 16.  `start_event` / `stop_event`, if given (both or
 * neither), are recorded at the kernel's own dispatch begin and end, as
 * dl_time_next_launch arms them.  Asynchronous on `stream`.  Errors:
 * DL_ERR_INVALID (mode, NULL or misaligned pointer, bytes, one event),
 * DL_ERR_UNSUPPORTED (more than 2^31 - 1 blocks of 32 KiB), DL_ERR_LAUNCH. */
typedef enum { DL_PROBE_READ = 0, DL_PROBE_COPY = 1 } dl_probe_mode;
dl_status dl_stream_probe(int32_t mode, const void *src, void *dst, size_t bytes, void *stream,
                          void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* DELTALOG_H */
