/*
 * qsa.h -- C ABI of libqsa, the MI355X (gfx950) QSA prompt-attention path.
 *
 * QSA attention, as the quantized_sparse_flash audit pages describe it: every
 * prompt token t of a chunk that starts at absolute position pos0 sees the
 * n_kv(t) = pos0 + t + 1 KV cells [0, n_kv(t)) of each KV group.  For each
 * (token, group) row the path
 *   1. selects cells: all of them when n_kv(t) <= budget ("identity ids"),
 *      otherwise the `budget` cells with the largest selection score
 *      (page "round 6 track b - qsa flash", delivered change; ties to the
 *      lower index, ids ascending -- the reading this library takes);
 *   2. gathers the selected cells' int8 K/V codes and their fp16 scales, one
 *      per 64 dims (same page, delivered change: four scales per cell);
 *   3. computes S = 0.0625 * Q K^T for the group's 12 query heads chunk by
 *      chunk over 64 selected cells with an online softmax, forms P in fp16
 *      and accumulates P V (page "opus_r9_qsa", what changed);
 *   4. optionally writes per-chunk partials (o, m, l) that are combined by a
 *      log-sum-exp merge (page "round 27 track b - qsa prep and merge",
 *      decision and correctness: head stride 258, chunk stride 6192).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are device (HBM) pointers owned by the caller;
 *     the library keeps no reference after the call returns and allocates no
 *     memory itself (scratch comes in through a workspace argument).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; results are visible after the caller
 *     synchronises the stream.  Calls are thread-safe.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     non-zero return means nothing was enqueued, except QSA_ERR_LAUNCH,
 *     which reports a failed kernel launch.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Element layouts are dense and row-major with the shapes given below;
 *     all counts are in elements.
 */
#ifndef QSA_H_
#define QSA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define QSA_OK 0
#define QSA_ERR_ARG (-1)         /* NULL or misaligned pointer, bad struct */
#define QSA_ERR_UNSUPPORTED (-2) /* heads_per_group != 12, head_dim != 256, budget too large */
#define QSA_ERR_SHAPE (-3)       /* T < 1, pos0 < 0, n_groups < 1, n_cells < pos0 + T, ... */
#define QSA_ERR_LAUNCH (-4)      /* the HIP runtime rejected a kernel launch */
#define QSA_ERR_TOO_LARGE (-5)   /* qsa_flash_noalloc: the shape needs more scratch than it holds */
#define QSA_ERR_DEVICE (-6)      /* qsa_flash_noalloc: the current HIP device could not be queried */

/* Library limits. */
#define QSA_HEADS_PER_GROUP 12 /* query heads that share one KV group */
#define QSA_HEAD_DIM 256       /* dims per head; scales cover 64 dims each */
#define QSA_SCALE_BLOCK 64     /* dims per fp16 scale */
#define QSA_CHUNK 64           /* selected cells per chunk / partial record */
#define QSA_PART_STRIDE 258    /* floats per partial record: o[256], m, l */
#define QSA_MAX_BUDGET 65536   /* largest supported budget */
#define QSA_MAX_INDEX_DIM 256  /* longest qsa_score vectors */
#define QSA_DEFAULT_BUDGET 2051
#define QSA_NOALLOC_SCRATCH_BYTES (16 << 20) /* device scratch held by qsa_flash_noalloc */

/* An fp16 element: the IEEE 754 binary16 bit pattern, two bytes.  The
 * library only hands these pointers to the GPU, so the host-side element
 * type is a plain 16-bit integer that every C and C++ compiler has; a
 * caller's _Float16 or __half array is passed with a pointer cast. */
typedef uint16_t qsa_f16;

/* Shape of one prompt chunk of one layer. */
typedef struct {
  int32_t T;               /* query tokens in the chunk, >= 1 */
  int32_t pos0;            /* absolute position of token 0, >= 0 */
  int32_t n_groups;        /* KV groups G, >= 1 (the pages use 2) */
  int32_t heads_per_group; /* must be QSA_HEADS_PER_GROUP */
  int32_t head_dim;        /* must be QSA_HEAD_DIM */
  int32_t budget;          /* selection budget B, 1..QSA_MAX_BUDGET */
  int64_t n_cells;         /* KV cells held per group (>= pos0 + T); also the
                              row stride of `scores` */
} qsa_shape;

/*
 * qsa_score -- selection scores, the step before qsa_topk.  The pages name
 * the score kernel and its buffers (page "round 27 track b - qsa prep and
 * merge", decision: its four-value dot products are fully unrolled;
 * correctness: the qidx, pooled and scores buffers; page "round 6 track b -
 * qsa flash", actual runs: a worst relative score difference of 2.76e-6)
 * but not what qidx and pooled hold.  This library's reading: the score of
 * cell c for token t in group g is the dot product of the token's index
 * query with the cell's pooled key,
 *     scores[t][g][c] = sum over d of qidx[t][g][d] * pooled[g][c][d],
 * in fp32, one fused multiply-add per d in ascending order.
 *
 *   index_dim : length of both vectors, a multiple of 4 in
 *               [4, QSA_MAX_INDEX_DIM] (4: one value per 64-dim block).
 *   qidx      : device, const float [T][G][index_dim].
 *   pooled    : device, const float [G][n_cells][index_dim].
 *   scores    : device, float [T][G][n_cells] (the layout qsa_topk reads).
 *               Row (t, g) is written at cells [0, n_kv(t)) when
 *               n_kv(t) > budget, the rows whose selection reads scores;
 *               every other element is left as it was.  When no row is
 *               above budget nothing is read or written and the pointers
 *               may be NULL.
 * Alignment: 16 bytes for qidx, pooled and scores.  Errors:
 * QSA_ERR_UNSUPPORTED (index_dim), QSA_ERR_SHAPE, QSA_ERR_ARG.
 * Numerics: |score - exact| <= index_dim * 2^-24 * sum_d |qidx_d pooled_d|
 * to first order (recursive fp32 summation with fused multiply-adds).
 */
int qsa_score(const qsa_shape *shape, int32_t index_dim, const float *qidx, const float *pooled,
              float *scores, void *stream);

/*
 * qsa_topk -- step 1: selected ids of every (token, group) row.
 *
 *   scores : device, const float [T][G][n_cells]; row (t, g) is read only at
 *            cells [0, n_kv(t)) and only when n_kv(t) > budget.  May be NULL
 *            when pos0 + T <= budget (no row above budget).  Scores must not
 *            be NaN (NaN rows give an unspecified but in-range selection);
 *            -0.0 and +0.0 are equal.
 *   ids    : device, int32 [T][G][budget], written in full:
 *            n_kv(t) <= budget: 0, 1, ..., n_kv(t)-1, then -1 padding;
 *            n_kv(t) >  budget: the budget cells of largest score (equal
 *            scores: lower index first), in ascending order.
 * Alignment: 4 bytes.  Results are bit-exact (integer output).
 */
int qsa_topk(const qsa_shape *shape, const float *scores, int32_t *ids, void *stream);

/*
 * qsa_flash -- steps 2-4: attention over the selected cells.
 *
 *   q        : device, fp16 [T][G*12][256]; head h belongs to group h / 12.
 *   kq, vq   : device, int8 [G][n_cells][256] K and V codes.
 *   ksc, vsc : device, fp16 [G][n_cells][4]; dim d of cell c is scaled by
 *              ksc[g][c][d / 64] (resp. vsc).
 *   ids      : device, int32 [T][G][budget] as written by qsa_topk.  Read
 *              only for rows with n_kv(t) > budget; rows under budget use
 *              the identity cells whatever ids holds.  May be NULL when
 *              pos0 + T <= budget.  Each id read must lie in [0, n_kv(t));
 *              an id outside it is clamped into [0, n_cells) (the output is
 *              then unspecified, the kernel never reads out of bounds).
 *   out      : device, fp16 [T][G*12][256], the softmax-weighted values,
 *              rounded to nearest even.  Written in fused mode (part == NULL);
 *              not touched in split mode.
 *   workspace, workspace_bytes : device scratch of at least
 *              qsa_flash_workspace_bytes(shape) bytes, 256-byte aligned, owned
 *              by the caller; overwritten by the call, so two calls in flight
 *              at once must not share it.  May be NULL (with size 0) when
 *              that size is 0.
 *   part     : NULL for fused mode.  Otherwise split mode: device, float
 *              [T][ceil(budget/64)][G*12][258]; for token t and chunk
 *              k < ceil(n_sel(t)/64), n_sel(t) = min(n_kv(t), budget), the
 *              record at ((t*KC + k)*G*12 + h)*258 holds o[0..255] (the
 *              unnormalised sum of exp(s_c - m) v_c over the chunk's cells),
 *              m (the chunk's max of s_c, natural-log units) and l (the sum of
 *              exp(s_c - m)).  Records of chunks a token does not have are not
 *              written.
 * Alignment: 16 bytes for q, kq, vq, out and part; 8 for ksc, vsc; 4 for ids;
 * 256 for workspace.
 * Numerics: fp16 MFMA products with fp32 accumulation, k = code x scale
 * rounded to fp16 (in fused mode, rows above budget, and every row of a call
 * that runs as row pieces, instead take their scores from exact int8
 * products of the K codes with q split into two int8 pieces, each element
 * of q then within 2^-15 of the head's largest |q|, unless so few rows run
 * that each piece is one chunk); relative L2 error against exact attention
 * about 4e-4 on the pages' value ranges.
 */
int qsa_flash(const qsa_shape *shape, const qsa_f16 *q, const int8_t *kq, const qsa_f16 *ksc,
              const int8_t *vq, const qsa_f16 *vsc, const int32_t *ids, qsa_f16 *out,
              float *part, void *workspace, int64_t workspace_bytes, void *stream);

/*
 * qsa_flash_prepare, qsa_flash_attend -- the two halves of a fused-mode
 * qsa_flash call, for callers that time or schedule them apart.  The fused
 * path first dequantises the cells that every token under budget reads (the
 * shared identity prefix, see qsa_flash_workspace_bytes) into `workspace`,
 * then attends.  qsa_flash_prepare enqueues the first half only (nothing
 * when no token is under budget); qsa_flash_attend enqueues the second
 * half and reads the workspace that a qsa_flash_prepare call with the same
 * shape, K/V arguments and workspace_bytes filled earlier on the same stream
 * (or one ordered before it); qsa_flash_attend may run more than once on
 * one prepared workspace.  The pair computes exactly what one fused
 * qsa_flash call computes, and qsa_flash (fused mode) is these two calls.
 * Arguments, alignment and error behaviour are those of qsa_flash; `out` is
 * written by qsa_flash_attend.  Attending without a prepared workspace
 * gives unspecified output values (never an out-of-bounds access).
 */
int qsa_flash_prepare(const qsa_shape *shape, const int8_t *kq, const qsa_f16 *ksc,
                      const int8_t *vq, const qsa_f16 *vsc, void *workspace,
                      int64_t workspace_bytes, void *stream);
int qsa_flash_attend(const qsa_shape *shape, const qsa_f16 *q, const int8_t *kq,
                     const qsa_f16 *ksc, const int8_t *vq, const qsa_f16 *vsc,
                     const int32_t *ids, qsa_f16 *out, void *workspace,
                     int64_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace qsa_flash needs for this shape in fused mode
 * (0 when it needs none, and split mode needs none); a host-only
 * helper.  The fused path dequantises the cells that tokens under budget
 * share -- cells [0, pos0 + t_id) of every group, t_id being the number of
 * such tokens -- once per call into this workspace: 64 KB per group and
 * 64-cell chunk (fp16 K and V^T).  When the tiled attention of those tokens
 * leaves compute units idle and has blocks of at least 12 chunks (a few
 * tokens after a long prefix), those blocks of 64 queries run as 2 or 3
 * workgroups over consecutive ranges of their chunks that merge their
 * partial results through the workspace; it then also holds, per split
 * block, one partial of 64 x 258 floats per piece and a 4-byte counter
 * (the counters rounded up to 256 bytes).  qsa_flash_prepare clears the
 * counters; every call leaves them at zero.  When at most 512 (token,
 * group) rows are above budget, they run as row pieces plus the merge,
 * which fill the GPU where one wavefront per row would not.  Each row is
 * cut into pieces of cpr consecutive 64-cell chunks of its selection,
 * cpr = ceil(rows x ceil(budget/64) / 1024), and each piece writes one
 * (o, m, l) record of 258 floats per head (part's layout with a record per
 * piece instead of per chunk).  The records follow the part above, rounded
 * up to 256 bytes.  When the whole call has at most 256 rows and some above
 * budget, every token runs that way and the workspace holds the records
 * alone (qsa_flash_prepare then enqueues nothing).  Such calls need a
 * workspace even with no token under budget.
 */
int64_t qsa_flash_workspace_bytes(const qsa_shape *shape);

/*
 * qsa_flash_noalloc -- qsa_flash for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, layouts,
 * results and errors as qsa_flash without the workspace: the fused path's
 * scratch is instead a static device array of QSA_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that each GPU the library runs on holds until the process ends;
 * its address is resolved (hipGetSymbolAddress) on the first call on each
 * device, with that device current.  The call itself allocates nothing.
 * Every call on one GPU shares that GPU's array, so two calls that overlap
 * in time on the same GPU (other streams, other threads) race and give
 * unspecified output; calls ordered on one stream are fine.  Nothing in the
 * array needs to start at zero (each call writes every byte it reads).
 *   returns QSA_ERR_TOO_LARGE when the fused path's chunk images (64 KB
 *   per KV group and 64-cell chunk of identity prefix) exceed
 *   QSA_NOALLOC_SCRATCH_BYTES (more than 256 of them, e.g. 2 groups past
 *   an 8192-cell prefix), checked before anything else touches the device;
 *   QSA_ERR_DEVICE when the device or the array's address cannot be
 *   queried.  The scratch beyond the images holds the split pieces that
 *   qsa_flash_workspace_bytes makes room for, as far as it reaches; blocks
 *   it cannot hold run whole.  Rows above budget run as row pieces plus the
 *   merge, as in qsa_flash, when qsa_flash_workspace_bytes fits the scratch
 *   whole, and on the row kernel otherwise.  Either difference changes the
 *   output only by rounding.
 */
int qsa_flash_noalloc(const qsa_shape *shape, const qsa_f16 *q, const int8_t *kq,
                      const qsa_f16 *ksc, const int8_t *vq, const qsa_f16 *vsc,
                      const int32_t *ids, qsa_f16 *out, float *part, void *stream);

/*
 * qsa_merge -- log-sum-exp merge of split-mode partials (page "round 27
 * track b - qsa prep and merge", decision: the (m, l) merge of chunk
 * partials).  For token t the first ceil(n_sel(t)/64) records of each head
 * are merged:  M = max m_k,  L = sum l_k e^(m_k - M),
 *              out = fp16( sum e^(m_k - M) o_k / L ).
 *   part : device, float [T][ceil(budget/64)][G*12][258] (qsa_flash layout).
 *   out  : device, fp16 [T][G*12][256].
 * Alignment: 16 bytes for both.
 */
int qsa_merge(const qsa_shape *shape, const float *part, qsa_f16 *out, void *stream);

/*
 * qsa_quantize -- the K/V quantiser that fills the int8 cache (the prep step
 * of page "round 27 track b - qsa prep and merge"; the code/scale format of
 * page "round 6 track b - qsa flash", delivered change: int8 codes, one fp16
 * scale per 64 dims).  The pages give no rounding rule; this library's
 * reading, per row and 64-dim block b:
 *   scale[b] = fp16(absmax_b / 127),
 *   code[d]  = clamp(rint(x[d] / scale[b]), -127, 127)   (0 if scale[b] == 0),
 * both divisions correctly rounded IEEE fp32, rint and the fp16 conversion
 * to nearest even: codes and scales are a deterministic function of x.
 *   n_rows : rows to quantise (cells; call once for K and once for V, or
 *            once over [G][n_cells] rows); 0 is a no-op.
 *   dim    : dims per row; only 256 (QSA_HEAD_DIM) is supported.
 *   x      : device, fp16 [n_rows][256], finite values.
 *   codes  : device, int8 [n_rows][256]  (the kq / vq layout of qsa_flash).
 *   scales : device, fp16 [n_rows][4]    (the ksc / vsc layout).
 * Alignment: 16 bytes for x and codes, 2 bytes for scales.  Errors:
 * QSA_ERR_UNSUPPORTED (dim), QSA_ERR_SHAPE (n_rows < 0 or too large),
 * QSA_ERR_ARG (NULL or misaligned pointer).
 */
int qsa_quantize(int64_t n_rows, int32_t dim, const qsa_f16 *x, int8_t *codes,
                 qsa_f16 *scales, void *stream);

/* Human-readable text of a status code (static storage). */
const char *qsa_status_string(int status);

/* Floats needed by a split-mode `part` buffer for this shape (0 on a bad
 * shape); a host-only helper. */
int64_t qsa_part_elems(const qsa_shape *shape);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H_ */
