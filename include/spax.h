/*
 * spax.h -- C ABI of libspax: three-tier activation-sparse decoding GEMV on gfx950.
 *
 * What the library computes (batch-one decoding, one activation vector per call):
 *
 *   SpAx, "Activation Sparsity with Weight Approximation for Faster LLM Decoding on
 *   Offloaded Weights" (arXiv:2610.02598), Abstract: each weight is read in its original
 *   form, read from a compressed approximation, or not read; activations closest to zero
 *   skip their weights, smaller-magnitude ones read the approximation, the largest read
 *   the original.  The eigenradar commentary on SpAx ("The route outside GPU memory",
 *   first and third paragraphs) makes the unit one weight column per input channel, the
 *   approximation two-bit, and stores jointly accessed columns together.
 *
 *   TopK-Guided (arXiv:2610.01763), section 2.1 "TopK-Guided Masking": the tier mask may
 *   be a TopK, a threshold, or a threshold estimate clipped to +-delta around the target
 *   followed by TopK.
 *
 *   y[r] = sum_{j in FULL} x[j] * W[r][j]  +  sum_{j in APPROX} x[j] * What[r][j]
 *
 * Conventions shared by every entry point:
 *   - Return SPAX_OK (0) or a negative spax_status.  All argument validation happens on
 *     the host before anything is enqueued; on error nothing runs and no output buffer
 *     is touched.  spax_last_error() then holds a thread-local message.
 *   - "device pointer" means memory the GPU can address (hipMalloc).  The caller owns
 *     every buffer; the library never allocates device memory in these calls.
 *   - Work is enqueued on the given HIP stream and is asynchronous unless stated.
 *   - fp16 values are passed as uint16_t bit patterns; y is fp32.
 *   - No exceptions cross this boundary.
 */
#ifndef SPAX_H
#define SPAX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- status codes */
typedef enum spax_status {
  SPAX_OK = 0,
  SPAX_ERR_NULL = -1,        /* a required pointer is NULL                          */
  SPAX_ERR_SHAPE = -2,       /* layout sizes not supported (see spax_layout_init)    */
  SPAX_ERR_PARAM = -3,       /* tier parameters out of range                         */
  SPAX_ERR_ALIGN = -4,       /* a pointer is not aligned as required                 */
  SPAX_ERR_WORKSPACE = -5,   /* workspace too small                                  */
  SPAX_ERR_HIP = -6,         /* a HIP runtime call failed (message has the details)  */
  SPAX_ERR_UNSUPPORTED = -7, /* valid request the library does not implement         */
  SPAX_ERR_HOST = -8         /* host memory or a host thread could not be obtained   */
} spax_status;

/* ---------------------------------------------------------------- packed layout */
enum { SPAX_FMT_FP16 = 0, SPAX_FMT_INT4 = 1 };

#define SPAX_MAX_MATS 4
#define SPAX_MAX_DIN 32768     /* largest input vector one tier-mask workgroup holds */
#define SPAX_RECORD_ALIGN 128  /* column records are padded to one 128-byte line     */

/*
 * spax_layout: shape and byte layout of one packed weight blob.
 *
 * Pages: eigenradar commentary on SpAx, "The route outside GPU memory", third
 * paragraph (jointly accessed columns are placed together).  Matrices that multiply the
 * same activation vector (q|k|v, gate|up) are fused: the record of input channel j holds
 * column j of every matrix, concatenated along rows (matrix 0 rows first).
 *
 * Blob = region F (original tier) then region A (two-bit approximation); both are
 * column-major with one record per input channel, in channel order, each record
 * zero-padded to a multiple of 128 bytes:
 *   region F, record j at  j * stride_F:
 *     FP16: d_out_total fp16 values (little endian);
 *     INT4: d_out_total/2 bytes of codes (row 2k in bits [3:0], row 2k+1 in [7:4]) then
 *           d_out_total/base_group u32 words, fp16 scale in bits [15:0], fp16 zero in
 *           bits [31:16];
 *   region A, record j at  off_A + j * stride_A:
 *     d_out_total/4 bytes of two-bit codes (row 4k+i in bits [2i+1:2i]) then
 *     d_out_total/approx_group (scale, zero) u32 words as above.
 * A group of G rows reconstructs as w_hat = s*q + z (z = group minimum, s = (max-min)/L,
 * q = round-half-even((w - z)/s) clamped to [0, L], L = 3 for two-bit, 15 for int4;
 * every step in fp32 with round-to-nearest-even, s and z rounded to fp16).
 *
 * The caller fills the input fields; spax_layout_init fills the derived ones.
 */
typedef struct spax_layout {
  /* inputs */
  int32_t n_mats;                /* 1..SPAX_MAX_MATS matrices sharing one input       */
  int32_t d_in;                  /* input channels = columns, 1..SPAX_MAX_DIN          */
  int32_t d_out[SPAX_MAX_MATS];  /* rows of each matrix; each a multiple of every group */
  int32_t base_fmt;              /* SPAX_FMT_FP16 or SPAX_FMT_INT4                     */
  int32_t base_group;            /* INT4 group rows: 128                               */
  int32_t approx_group;          /* two-bit group rows: 64 or 128                      */
  int32_t reserved0;
  /* derived by spax_layout_init */
  int64_t d_out_total;           /* sum of d_out                                       */
  int64_t rec_F, rec_A;          /* unpadded record bytes                              */
  int64_t stride_F, stride_A;    /* padded record bytes (multiples of 128)             */
  int64_t off_A;                 /* byte offset of region A = d_in * stride_F          */
  int64_t total_bytes;           /* blob size                                          */
} spax_layout;

/* Validate the inputs of *L and fill its derived fields.  Host only; enqueues nothing.
 * Pages: eigenradar commentary on SpAx, "The route outside GPU memory", first paragraph (each
 * weight column has an original and a two-bit approximate form) and third paragraph (columns
 * used together are stored together); the SpAx Abstract's 16-bit and 4-bit weights give the
 * two base formats.
 * Errors: SPAX_ERR_NULL; SPAX_ERR_SHAPE if n_mats, d_in, a group size or the format is
 * out of range, or any d_out[m] is not a positive multiple of approx_group (and of
 * base_group for INT4). */
int spax_layout_init(spax_layout* L);

/*
 * Pack fp16 weights into the blob (offline, once per weight set).  Pages: eigenradar
 * commentary on SpAx, "The route outside GPU memory", first and third paragraphs (an original
 * and a two-bit form of every column, prepared ahead of decoding and stored together).
 *   W[m]   : host array of n_mats device pointers; W[m] is matrix m stored column-major
 *            as d_in records of d_out[m] fp16 values (the record of channel j is column j).
 *   packed : device pointer, total_bytes, 256-byte aligned; fully overwritten, padding
 *            included, so the result is a deterministic function of the weights.
 * Weights must be finite (non-finite input gives unspecified codes).
 * Errors: SPAX_ERR_NULL, SPAX_ERR_SHAPE (layout not initialised), SPAX_ERR_ALIGN
 * (packed not 256-byte aligned or a W[m] not 16-byte aligned), SPAX_ERR_HIP.
 */
int spax_pack_columns(const spax_layout* L, const uint16_t* const* W, void* packed,
                      hipStream_t stream);

/*
 * Offline placement of the column records (eigenradar commentary on SpAx, "The route outside
 * GPU memory", third paragraph: jointly accessed columns are placed together, so a token's
 * selection reads fewer, longer ranges).  Host only.
 *   tiers : host, n_tokens rows of d_in tier bytes (SPAX_TIER_*), the masks of calibration
 *           tokens (e.g. spax_build_tiers' tier output copied back).
 *   order : host, d_in entries: a permutation of [0, d_in) with channels in descending order of
 *           the bytes they made selected (stride_F per FULL, stride_A per APPROX), equal
 *           scores in channel order.  Position p of a placed blob holds channel order[p].
 * Errors: SPAX_ERR_NULL, SPAX_ERR_SHAPE (layout not initialised), SPAX_ERR_PARAM (n_tokens < 0,
 * a byte that is not a tier).
 */
int spax_placement_order(const spax_layout* L, const uint8_t* tiers, int32_t n_tokens,
                         int32_t* order);

/*
 * spax_pack_columns with a placement: record p of each region holds column perm[p] (perm:
 * device, d_in int32, a permutation such as spax_placement_order's order; entries are clamped
 * to [0, d_in) so a malformed one repeats a column but stays in bounds).  The activation vector
 * of a placed blob is permuted alike, x_placed[p] = x[perm[p]] (in a model, once, through the
 * rows of the layer that produces x); masks, lists and the product then work on positions, and
 * y is the product over the same columns.  Errors: as spax_pack_columns, plus SPAX_ERR_NULL
 * (perm) and SPAX_ERR_ALIGN (perm not 4-byte aligned).
 */
int spax_pack_columns_placed(const spax_layout* L, const uint16_t* const* W,
                             const int32_t* perm, void* packed, hipStream_t stream);

/* ---------------------------------------------------------------- tier masks */
enum { SPAX_TIER_SKIP = 0, SPAX_TIER_APPROX = 1, SPAX_TIER_FULL = 2 };
enum { SPAX_MODE_TOPK = 0, SPAX_MODE_THRESHOLD = 1, SPAX_MODE_TOPK_GUIDED = 2 };

/*
 * Tier-mask parameters.  Ranking: channel j outranks k iff key_j > key_k, or equal keys
 * and j < k, with key = (fp16 bits of x) & 0x7FFF (so NaN ranks above +Inf).
 *   TOPK         : ranks [0, n_full) FULL, the next n_approx APPROX, the rest SKIP.
 *   THRESHOLD    : FULL if |x| >= tau_full, else APPROX if |x| >= tau_skip, else SKIP.
 *   TOPK_GUIDED  : natural skip count c = #{|x| < tau}; n_skip = min(max(c, n_skip_lo),
 *                  n_skip_hi); kept = d - n_skip; n_approx = floor((approx_num*kept +
 *                  floor(approx_den/2)) / approx_den); then TOPK(kept - n_approx, n_approx).
 *                  (TopK-Guided section 2.1; spax_guided_bounds gives the +-delta band.)
 * Float thresholds are compared as fp16 keys: |x| >= tau  <=>  key >= K(tau), with K(tau)
 * from spax_key_threshold.
 */
typedef struct spax_tier_params {
  int32_t mode;
  int32_t n_full, n_approx;        /* TOPK                                   */
  int32_t n_skip_lo, n_skip_hi;    /* TOPK_GUIDED clip band on the skip count */
  int32_t approx_num, approx_den;  /* TOPK_GUIDED FULL/APPROX split of kept   */
  int32_t reserved0;
  double tau_skip, tau_full;       /* THRESHOLD                               */
  double tau;                      /* TOPK_GUIDED calibrated threshold        */
} spax_tier_params;

/*
 * Build one tier mask (one workgroup per vector).
 *   x          : device, d_in fp16 activations.
 *   tier       : device, d_in bytes of SPAX_TIER_* (may be NULL: not written).
 *   full_idx   : device, capacity d_in int32; ascending channel indices of the FULL tier.
 *   approx_idx : device, capacity d_in int32; ascending indices of the APPROX tier.
 *   counts     : device, 3 int32 = {n_full, n_approx, n_skip}.  Stays on the device.
 * List entries past their count are unspecified.  x, lists and counts 4-byte aligned.
 * Errors: SPAX_ERR_NULL, SPAX_ERR_SHAPE (d_in outside 1..SPAX_MAX_DIN), SPAX_ERR_PARAM
 * (unknown mode, counts out of range, n_skip_lo > n_skip_hi, approx_den outside
 * 1..65535, approx_num outside [0, approx_den], tau_skip > tau_full, NaN thresholds),
 * SPAX_ERR_ALIGN, SPAX_ERR_HIP.
 */
int spax_build_tiers(const uint16_t* x, int32_t d_in, const spax_tier_params* p,
                     uint8_t* tier, int32_t* full_idx, int32_t* approx_idx, int32_t* counts,
                     hipStream_t stream);

/* ---------------------------------------------------------------- tiered GEMV */

/* Workspace bytes spax_tiered_gemv needs for layout *L.  The current kernels need none and
 * return 0 (then ws may be NULL); callers should still size ws with this function.
 * Returns 0 also if *L is not initialised. */
size_t spax_gemv_workspace_bytes(const spax_layout* L);

/*
 * y = tiered product of one packed blob with one activation vector.  Pages: SpAx Abstract
 * (read the original weights of the largest activations, the compressed approximation for
 * smaller ones, nothing for those closest to zero); eigenradar commentary, "The route outside
 * GPU memory", third paragraph (the two-bit approximation is reconstructed on the GPU).
 *   packed      : device blob laid out by *L (spax_pack_columns), 256-byte aligned.
 *   x           : device, d_in fp16 activations (the same vector the mask was built from),
 *                 4-byte aligned; for odd d_in the kernels may read the two bytes that pad
 *                 x to a whole dword (never past that dword).
 *   full_idx, approx_idx, counts : device, as written by spax_build_tiers (or any
 *                 caller lists of distinct channels with counts[0], counts[1]).  Counts are
 *                 clamped to [0, d_in] and indices to [0, d_in) on the device, so malformed
 *                 lists give an unspecified y but never an out-of-bounds access.
 *   y           : device, d_out_total fp32, 16-byte aligned; fully overwritten (all zeros
 *                 if both lists are empty).  Rows follow the fused order of *L.
 *   ws, ws_bytes: device workspace of at least spax_gemv_workspace_bytes(L) bytes,
 *                 256-byte aligned (may be NULL when that size is 0).
 * Accumulation is fp32.  Column chunks handled by different workgroups meet in y through
 * fp32 atomic adds, so y can differ in the last bits between runs; the tier masks and
 * lists are bit-exact.  Enqueues a zero fill of y before the product when the launch
 * splits the column lists.
 * Errors: SPAX_ERR_NULL, SPAX_ERR_SHAPE, SPAX_ERR_ALIGN, SPAX_ERR_WORKSPACE, SPAX_ERR_HIP.
 */
int spax_tiered_gemv(const spax_layout* L, const void* packed, const uint16_t* x,
                     const int32_t* full_idx, const int32_t* approx_idx,
                     const int32_t* counts, float* y, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* ---------------------------------------------------------------- pinned-host path */

/*
 * Read ranges of one column list (host helper).  Pages: eigenradar commentary on SpAx, "The
 * route outside GPU memory", third paragraph (adjacent read ranges are merged; coarse
 * granularity can move more bytes than were selected).
 *   idx      : host array of n ascending, distinct, non-negative channel indices.
 *   gap      : runs of consecutive channels separated by at most `gap` unselected channels
 *              are merged into one range (the gap columns are moved too); 0 merges only
 *              adjacent channels.
 *   first, count : host arrays of capacity n receiving each range (may be NULL to count only).
 *   n_ranges : receives the number of ranges.
 * Errors: SPAX_ERR_NULL, SPAX_ERR_PARAM (n < 0, gap < 0, idx not ascending / distinct /
 * non-negative).
 */
int spax_column_ranges(const int32_t* idx, int32_t n, int32_t gap, int32_t* first,
                       int32_t* count, int32_t* n_ranges);

/* Byte ledger of one mask read from block storage (spax_storage_ledger). */
typedef struct spax_storage_stats {
  int64_t selected_bytes;  /* n_full * stride_F + n_approx * stride_A                         */
  int64_t moved_bytes;     /* bytes of the merged record ranges (selected + merged gaps)       */
  int64_t read_bytes;      /* bytes physically read: n_blocks * block_bytes                    */
  int64_t n_blocks;        /* blocks read, each range rounded out to block boundaries          */
  int32_t n_ranges;        /* merged ranges (FULL + APPROX) = read requests                    */
  int32_t reserved0;
} spax_storage_stats;

/*
 * Bytes selected against bytes physically read when the blob sits on block storage (host
 * helper).  Pages: eigenradar commentary on SpAx, "The route outside GPU memory", third
 * paragraph (coarse storage granularity can move more bytes than a selected column needs) and
 * last paragraph (for NVMe, selected bytes and bytes physically read are separate entries);
 * the SpAx Abstract reports the flash-offloaded case apart.
 * The blob (laid out by *L) starts on a block boundary; the selected columns of each region
 * are merged into ranges as by spax_column_ranges (gap); each range is one read request that
 * reads every block of block_bytes its bytes touch (a block touched by two requests is read
 * twice).
 *   full_idx, approx_idx : host, n_full / n_approx ascending distinct channels < d_in.
 *   out : host.
 * Errors: SPAX_ERR_NULL, SPAX_ERR_SHAPE (layout not initialised), SPAX_ERR_PARAM (lengths out
 * of range, gap < 0, block_bytes < 1, a list not ascending / distinct / inside [0, d_in)).
 */
int spax_storage_ledger(const spax_layout* L, const int32_t* full_idx, int32_t n_full,
                        const int32_t* approx_idx, int32_t n_approx, int32_t gap,
                        int64_t block_bytes, spax_storage_stats* out);

/* Byte account of one spax_tiered_gemv_pinned call. */
typedef struct spax_move_stats {
  int64_t selected_bytes;  /* n_full * stride_F + n_approx * stride_A                   */
  int64_t moved_bytes;     /* record bytes copied host -> device (selected + merged gaps) */
  int64_t list_bytes;      /* list bytes copied host -> device: 0 for SPAX_PINNED_GATHER
                              (the lists never leave the device); for SPAX_PINNED_MEMCPY and
                              SPAX_PINNED_HOSTGATHER one upload of the span of the two
                              compacted host lists (d_in entries each) that holds every used
                              entry                                                       */
  int32_t n_ranges;        /* merged ranges (FULL + APPROX)                               */
  int32_t n_full, n_approx;
  int32_t reserved0;
} spax_move_stats;

/* spax_tiered_gemv_pinned: how the ranges cross PCIe */
enum {
  /* the lists come back to the host (the call synchronizes `stream`), which merges the
   * ranges and issues one hipMemcpyAsync per range (host-driven DMA) */
  SPAX_PINNED_MEMCPY = 0,
  /* the ranges are merged on the device (one kernel, two workgroups) and one copy kernel
   * reads them from the mapped pinned blob (zero-copy) into the compacted staging area:
   * nothing waits for the host, so the call is asynchronous unless `stats` is requested */
  SPAX_PINNED_GATHER = 1,
  /* the lists come back to the host (the call synchronizes `stream`), which merges the
   * ranges; a pool of host threads (up to 16, started on first use) copies the records of
   * every range from the pinned blob into one library-owned pinned staging buffer (FULL
   * records, then APPROX records, back to back), which moves to the device in 8 MiB
   * hipMemcpyAsync chunks, each issued as soon as it is filled (CPU gather, one DMA stream
   * that overlaps the gathering) */
  SPAX_PINNED_HOSTGATHER = 2
};

/* Device workspace for spax_tiered_gemv_pinned: a compacted staging copy of the blob's
 * records (total_bytes, for the case that every column is selected), two compacted lists and
 * two slot -> column tables (4 * d_in bytes each) and 24 bytes of totals; 0 if *L is not
 * initialised. */
size_t spax_pinned_workspace_bytes(const spax_layout* L);

/*
 * Tiered GEMV with the packed blob in pinned host memory (allocated with hipHostMalloc).
 *   packed_host : the blob laid out by *L (e.g. a copy of spax_pack_columns' output).
 *   x, full_idx, approx_idx, counts, y : device, as for spax_tiered_gemv (the lists as
 *                 written by spax_build_tiers: ascending).
 *   gap   : range merging, as for spax_column_ranges.
 *   transfer : SPAX_PINNED_MEMCPY, SPAX_PINNED_GATHER or SPAX_PINNED_HOSTGATHER (same bytes
 *              moved, same result).
 *   ws    : device, >= spax_pinned_workspace_bytes(L) bytes, 256-byte aligned.
 *   stats : host, may be NULL (the byte account; requesting it synchronizes `stream`).
 * Merges the selected columns of each region into ranges (on the device for
 * SPAX_PINNED_GATHER; on the host, after reading counts and lists back, for
 * SPAX_PINNED_MEMCPY and SPAX_PINNED_HOSTGATHER), moves the ranges host -> device (see `transfer`) into a compacted
 * staging area of ws (a range's columns land in consecutive slots, ranges in order) with the
 * compacted lists (staging slot | channel << 16), then runs the tiered GEMV over the staged
 * records.  y equals spax_tiered_gemv's on a device copy of the blob up to the order of fp32
 * additions.  Returns with the work enqueued on `stream`; with `stats` it also waits for the
 * byte account.  SPAX_PINNED_MEMCPY and SPAX_PINNED_HOSTGATHER: library-owned pinned buffers
 * (allocated on first use and grown as needed) hold the lists and, for the host gather, the
 * staged records; a later call waits until the previous call's copies from them have completed
 * before reusing them.
 * SPAX_PINNED_GATHER on lists that are not strictly ascending gives an unspecified y (never
 * an access outside the blob or ws).
 * Errors: as spax_tiered_gemv, plus SPAX_ERR_PARAM (gap < 0, unknown transfer, packed_host
 * not pinned host memory mapped for the device, and for the host-merged transfers lists read
 * back not ascending) and SPAX_ERR_WORKSPACE.
 */
int spax_tiered_gemv_pinned(const spax_layout* L, const void* packed_host, const uint16_t* x,
                            const int32_t* full_idx, const int32_t* approx_idx,
                            const int32_t* counts, float* y, int32_t gap, int32_t transfer,
                            void* ws, size_t ws_bytes, spax_move_stats* stats,
                            hipStream_t stream);

/* ---------------------------------------------------------------- decode step */

/*
 * One group of projections that share an activation vector (q|k|v, o, gate|up, down).
 * All pointers are device pointers as in spax_build_tiers / spax_tiered_gemv.
 */
typedef struct spax_phase {
  const spax_layout* layout;   /* host pointer to an initialised layout */
  const void* packed;
  const uint16_t* x;
  spax_tier_params params;
  uint8_t* tier;               /* may be NULL */
  int32_t* full_idx;
  int32_t* approx_idx;
  int32_t* counts;
  float* y;
} spax_phase;

/* spax_step.flags */
enum {
  /* one fused mask+GEMV launch per phase whose d_in <= 16384 (and whose lists fit in LDS):
   * one 1024-thread workgroup per compute unit, each finding the boundaries itself; other
   * phases take the two launches of SPAX_STEP_SEPARATE.  Same outputs either way.  Kernel
   * launches only (no copy, no memset), so the step can be captured into a HIP graph. */
  SPAX_STEP_DEFAULT = 0,
  /* one stand-alone mask launch (spax_build_tiers' kernel, which also clears y) and one
   * GEMV launch (spax_tiered_gemv's kernel) per phase */
  SPAX_STEP_SEPARATE = 1,
  /* every phase's mask in one launch, then every phase's GEMV in one persistent launch per
   * base format present (fp16 phases, then int4 phases).
   * Only for phases that are independent: all x ready when the step is enqueued, and no
   * phase's outputs (tier, lists, counts, y) overlapping another phase's inputs or outputs
   * (checked; SPAX_ERR_PARAM).  Needs ws of spax_step_workspace_bytes bytes (per-phase
   * descriptor tables, copied from a library-owned pinned ring of host buffers, so not
   * capturable in a graph).  events: [0, 1] bracket the mask launch, [2, 3] the GEMV launches
   * (one phase: [0, 1] bracket both).  Cannot be combined with SPAX_STEP_SEPARATE. */
  SPAX_STEP_BATCHED = 2,
  /* (with SPAX_STEP_DEFAULT or SPAX_STEP_SEPARATE) y identical bit for bit from run to run: a
   * phase's column chunks store their partial sums in ws instead of adding them into y with
   * atomics, and one more launch per phase adds the chunks in a fixed order.  Needs ws of
   * spax_step_workspace_bytes bytes, disjoint from every phase's buffers; y need not be
   * cleared (it is overwritten).  Not with SPAX_STEP_BATCHED, nor through
   * spax_decode_step_projections_noalloc (SPAX_ERR_UNSUPPORTED). */
  SPAX_STEP_DETERMINISTIC = 4
};

typedef struct spax_step {
  int32_t n_phases;            /* e.g. 32 layers x 4 groups = 128               */
  int32_t flags;
  const spax_phase* phases;    /* host array of n_phases                        */
  void* ws;                    /* device workspace, see spax_step_workspace_bytes */
  size_t ws_bytes;
  /* Optional timing hook (NULL: none): 2 * n_phases caller-created events.  events[2i] and
   * events[2i+1] are recorded on the stream right before and right after phase i's fused
   * mask+GEMV launch (its GEMV launch when the phase takes two launches), so they bracket
   * exactly that kernel. */
  hipEvent_t* events;
} spax_step;

/* Workspace bytes for spax_decode_step_projections over these phases, enough for every
 * launch form: the largest of the per-phase GEMV workspaces (currently 0), the
 * SPAX_STEP_BATCHED descriptor tables (a few hundred bytes per phase) and the
 * SPAX_STEP_DETERMINISTIC partial sums of the widest phase (column chunks x d_out_total
 * floats, about 2 MB for a 7B decoder layer).  0 for invalid input. */
size_t spax_step_workspace_bytes(const spax_phase* phases, int32_t n_phases);

/*
 * One batch-one decode step over all projection groups, in order: for each phase, the
 * tier mask of its activation vector, then the tiered GEMV of its fused matrices.
 * Phase p+1 is enqueued after phase p (stream order), as in a decoder where each
 * group's input depends on the previous group's output.  Launch forms: see spax_step.flags.
 * (eigenradar commentary on SpAx, second and last paragraphs: selection applies per
 * generated token during batch-one decoding.)
 * Errors: the union of spax_build_tiers and spax_tiered_gemv errors, reported before
 * anything is enqueued.
 */
int spax_decode_step_projections(const spax_step* step, hipStream_t stream);

/*
 * spax_decode_step_projections without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same phases, flags, validation and results as spax_decode_step_projections;
 * step->ws and step->ws_bytes are ignored.  SPAX_STEP_BATCHED keeps its descriptor tables
 * in a static device array of the library (256 KiB per GPU, held until the process ends;
 * about 208 bytes per phase, so at most 1257 phases, else SPAX_ERR_WORKSPACE), filled from a
 * static host buffer by one copy on `stream`; SPAX_STEP_DETERMINISTIC, whose partial sums
 * need a workspace, is refused (SPAX_ERR_UNSUPPORTED).  The call makes no hipMalloc,
 * hipHostMalloc or hipFree call and no host heap allocation (its first call on a device looks
 * up the array's address and creates one event).  Every call on one GPU shares
 * that array: calls that overlap on one GPU (different streams, or host threads on one
 * device) race, so callers serialize them, e.g. on one stream.  A call waits on the host
 * until the previous call's table copy has left the host buffer.
 */
int spax_decode_step_projections_noalloc(const spax_step* step, hipStream_t stream);

/* ---------------------------------------------------------------- diagnostics */

/* A plain streaming read, to measure what a launch that only reads gets from the memory
 * system (not a step of the method; the benchmark uses it for a read ceiling and for a
 * read floor at the byte counts of a decode step's launches).  The `bytes` bytes at p
 * (device memory) are read once with 16-byte non-temporal loads by 512-thread workgroups
 * (reads of 1 GiB or more: one contiguous chunk per workgroup, one workgroup per compute
 * unit; smaller reads: grid-stride over four workgroups per unit), and every wave stores
 * the XOR of the 32-bit words it read in its own word of `out` (device memory, out_words
 * uint32, at least 8; fewer words than waves means fewer workgroups).  The XOR of the first
 * *n_written words (host; nullable) is the XOR of all words read.  bytes = 0 launches
 * nothing and sets *n_written = 0.  Asynchronous on `stream`.  Errors: SPAX_ERR_NULL (p or
 * out NULL), SPAX_ERR_ALIGN (p or bytes not a multiple of 16, out not 4-byte aligned),
 * SPAX_ERR_PARAM (out_words < 8), SPAX_ERR_HIP. */
int spax_read_probe(const void* p, size_t bytes, uint32_t* out, int32_t out_words,
                    int32_t* n_written, hipStream_t stream);

/* ---------------------------------------------------------------- host helpers */

/* K(tau): smallest fp16 magnitude key k in [0, 0x7C00] with half(k) >= tau (compared in
 * double), else 0x7C01.  Returns -1 for NaN.  Pages: TopK-Guided section 2.1 (the natural
 * sparsity of a token counts activations below a calibrated threshold); the threshold is
 * compared on fp16 keys so the device compares integers only. */
int32_t spax_key_threshold(double tau);

/* Fixed keep fractions -> counts by cumulative round-half-up:
 * n_full = floor(p_full*d + 0.5), n_keep = floor((p_full + p_approx)*d + 0.5).  Pages:
 * TopK-Guided Abstract and section 1 (a TopK mask keeps a fixed count per token); the pages
 * give no rounding, cumulative round-half-up is this library's choice. */
int spax_counts_from_fractions(int32_t d, double p_full, double p_approx,
                               int32_t* n_full, int32_t* n_approx);

/* TopK-Guided +-delta band on the skip count (section 2.1): n_lo = max(0,
 * ceil(d*(s - delta) - 1e-9)), n_hi = min(d, floor(d*(s + delta) + 1e-9)). */
int spax_guided_bounds(int32_t d, double s, double delta, int32_t* n_lo, int32_t* n_hi);

/* ---------------------------------------------------------------- sparsity budgets (host) */

/*
 * Per-block sparsity targets from measured sensitivities (TopK-Guided, arXiv:2610.01763,
 * section 2.2 "Sensitivity-Aware Block Sparsity": blocks more sensitive than average get less
 * sparsity, the global budget moves to robust blocks, lambda sets how much moves, targets are
 * clamped; the pages clamp to [0.05, 0.95]).  Host only.
 *   sens    : n_blocks finite positive sensitivities (e.g. each block's output change at a
 *             probe sparsity, from a calibration pass).
 *   s_block : n_blocks outputs.  u_b = s + lambda * (mean(sens) - sens_b) / mean(sens);
 *             s_block[b] = min(max(u_b + c, s_min), s_max) with the shift c that makes the
 *             mean of s_block equal s (c = 0 when nothing is clamped).
 * Errors: SPAX_ERR_NULL; SPAX_ERR_PARAM (n_blocks < 1, lambda < 0, s outside [s_min, s_max],
 * a sensitivity not finite and positive).
 */
int spax_block_sparsity(const double* sens, int32_t n_blocks, double s, double lambda,
                        double s_min, double s_max, double* s_block);

/* Block output error of a trial allocation p[0..n_mats) (caller-defined, e.g. measured on
 * calibration tokens). */
typedef double (*spax_block_error_fn)(const double* p, int32_t n_mats, void* user);

/*
 * Greedy split of a block's sparsity over its matrices (TopK-Guided Appendix D "Block-wise
 * Greedy Sparsity Allocation", Table 4).  Host only.  From p = 0, each round tries one
 * increment alpha * mean(params) / params[m] on every matrix m that stays <= 1, keeps the one
 * whose trial allocation has the least block_error (ties: lower m), and records the row
 * (P, p[0..n_mats)), P = sum params[m] p[m] / sum params[m]; every increment moves P by
 * alpha / n_mats.  The first row is (0, zeros); the walk stops once P >= P_max or no matrix
 * can step.  Matrices that share one activation vector share one tier mask, so in a decoder
 * layer the units are the projection groups (q|k|v, o, gate|up, down).
 *   rows   : host, cap rows of (1 + n_mats) doubles; n_rows receives the rows recorded.
 * Errors: SPAX_ERR_NULL, SPAX_ERR_PARAM (n_mats outside 1..64, alpha <= 0, P_max > 1, a
 * parameter count not finite and positive, alpha so small that taking every matrix to 1
 * would need more than 1e7 increments, or a block_error value that is not finite: *n_rows
 * then holds the rows recorded before it), SPAX_ERR_WORKSPACE (more rows than cap; *n_rows
 * then holds the number needed).
 */
int spax_greedy_allocation(const double* params, int32_t n_mats, double alpha, double P_max,
                           spax_block_error_fn block_error, void* user, double* rows,
                           int32_t cap, int32_t* n_rows);

/* The allocation recorded for a block target (Appendix D: allocations are recorded against
 * the block's overall sparsity): p = the first row of `rows` whose P >= target (the last row
 * if none; zeros for target <= 0).  Host only.  Errors: SPAX_ERR_NULL, SPAX_ERR_PARAM. */
int spax_allocation_at(const double* rows, int32_t n_rows, int32_t n_mats, double target,
                       double* p);

const char* spax_status_string(int status);
const char* spax_last_error(void);   /* thread-local; "" if none */
const char* spax_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPAX_H */
