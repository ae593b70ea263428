/*
 * vl.h -- C ABI of the fused row-wise vocabulary-softmax loss on AMD MI355X
 * (gfx950).  Library: libvl.so.
 *
 * What it computes (the pages):
 *   [CE] aprender-train 0.36.0, entrenar/autograd/wgpu_cross_entropy.rs:
 *        module doc (loss = logsumexp(logits) - logits[label]; gradient
 *        softmax - one_hot(label), written in place), CEForwardParams /
 *        CEBackwardParams (loss range, scale), forward_async (loss and
 *        logsumexp per row), backward (scaled in-place gradient from the
 *        saved logsumexp), read_loss (mean over the loss range).
 *   [KL] cortiq-engine 0.8.21, src/gpu_wgpu/train_head.rs: module doc
 *        (distillation KL against the teacher's renormalised top-k and its
 *        gradient p_S - p_T, written in place and scaled), kl_rows, topk_rows
 *        (teacher top-k with probabilities renormalised over the k), acc_add
 *        (one vocabulary slice's input gradient added into another's),
 *        head_kl (the head's two products around the KL rows).
 *
 * Conventions for every call:
 *   - Pointers are device pointers owned by the caller.  The library keeps
 *     no reference after the call returns and allocates no memory (except
 *     the head calls' hipBLASLt handle, below).
 *   - Calls are asynchronous on `stream` (0 = the null stream of the current
 *     device); the caller observes completion on that stream.
 *   - Matrices are row-major and contiguous: row r of logits starts at
 *     element r * V.  Buffers must not overlap, except that logits are both
 *     input and output.
 *   - Returns VL_OK (0) or a negative status; vl_strerror names it.  Invalid
 *     sizes, dtypes and null pointers are rejected on the host before any
 *     GPU work.  ntok == 0 (or n == 0) is a no-op that returns VL_OK
 *     (except vl_loss_mean, which still writes its result).
 *   - Preconditions NOT checked on the device: label < V; ids < V and,
 *     among the entries with a nonzero probability, distinct within a row;
 *     probs >= 0; logits free of NaN and +inf with at least one finite
 *     value per row.  Entries with probability 0 take no part (a teacher
 *     list padded with a repeated id at probability 0 is fine).  Violating
 *     the preconditions never faults: a label or id >= V makes that row's
 *     loss NaN and is skipped; a repeated id with a nonzero probability
 *     leaves that row's loss and the gradient in the 16-byte vectors
 *     holding the id undefined.
 *   - Rows are 16-byte vectors when the logits pointer is 16-byte aligned
 *     and V * element size is a multiple of 16; otherwise the same result is
 *     computed one element at a time (slower).
 */
#ifndef VL_H
#define VL_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of logits: IEEE float32, or bfloat16 (widened exactly to
 * float32; stores round to nearest even).  VL_F16 (IEEE half) is accepted
 * only as the head's weight type (vl_head_kl). */
typedef enum { VL_F32 = 0, VL_BF16 = 1, VL_F16 = 2 } vl_dtype;

/* Loss range [CE: CEForwardParams / read_loss].  Row r takes part in the
 * loss iff start <= r % seq_len < end; with seq_len == ntok this is one
 * [loss_start, loss_end) range.  Requires 1 <= seq_len and
 * 0 <= start <= end <= seq_len.  A NULL range means every row. */
typedef struct {
    int64_t seq_len;
    int64_t start;
    int64_t end;
} vl_range;

enum {
    VL_OK = 0,
    VL_EINVAL = -1,  /* bad size, range or null pointer */
    VL_EDTYPE = -2,  /* unknown dtype */
    VL_ELAUNCH = -3  /* the HIP runtime rejected the launch */
};

/*
 * Fused cross-entropy forward + backward [CE: module doc, backward].
 *   logits  [ntok][V] dtype, in: logits; out: gradient
 *           scale * (softmax(row) - one_hot(label)), stored in dtype.
 *   labels  [ntok] uint32, read only: the target id of each row (any causal
 *           shift is the caller's).
 *   loss    [ntok] float32, written: logsumexp(row) - row[label], unscaled.
 *   lse     [ntok] float32 or NULL, written: logsumexp(row).
 *   rng     loss range or NULL.  Rows outside it are not read; their loss
 *           and lse are 0 and their gradient row is set to 0.
 *   scale   gradient scale, e.g. 1 / (rows in the range) for the mean loss.
 * Limits: 1 <= V <= 2^31 - 1, ntok >= 0.
 */
int vl_ce_fwd_bwd(void *logits, int dtype, const uint32_t *labels, float *loss, float *lse,
                  int64_t ntok, int64_t V, const vl_range *rng, float scale,
                  hipStream_t stream);

/*
 * Cross-entropy forward only [CE: forward_async, which stores the per-row
 * loss and logsumexp for a later backward and reads nothing back].
 *   logits  [ntok][V] dtype, read only.
 *   labels  [ntok] uint32, read only.
 *   loss    [ntok] float32, written: logsumexp(row) - row[label], unscaled.
 *   lse     [ntok] float32 or NULL, written: logsumexp(row), the input of
 *           vl_ce_bwd.
 *   rng     loss range or NULL.  Rows outside it are not read; their loss
 *           and lse are 0.
 * loss and lse may differ from vl_ce_fwd_bwd's in the last bits: the two
 * reduce the row in different orders.
 * Limits: as vl_ce_fwd_bwd.
 */
int vl_ce_fwd(const void *logits, int dtype, const uint32_t *labels, float *loss, float *lse,
              int64_t ntok, int64_t V, const vl_range *rng, hipStream_t stream);

/*
 * Cross-entropy backward from a saved logsumexp [CE: backward].
 *   logits  [ntok][V] dtype, in: the logits; out: the gradient
 *           scale * (exp(row - lse) - one_hot(label)), stored in dtype.
 *   labels  [ntok] uint32, read only.
 *   lse     [ntok] float32, read only: logsumexp of each row, as vl_ce_fwd
 *           wrote it; used as given.
 *   rng     loss range or NULL.  Rows outside it are not read and their
 *           gradient row is set to 0; their lse is not read either.
 *   scale   gradient scale, e.g. 1 / (rows in the range) for the mean loss.
 * Limits: as vl_ce_fwd_bwd.
 */
int vl_ce_bwd(void *logits, int dtype, const uint32_t *labels, const float *lse, int64_t ntok,
              int64_t V, const vl_range *rng, float scale, hipStream_t stream);

/*
 * Mean loss over the loss range, on the device [CE: read_loss, which sums
 * the loss of every row and divides by the rows in the range].
 *   loss  [ntok] float32, read only (may be NULL when ntok == 0).
 *   mean  one float32 on the device, written: (sum of loss[0..ntok)) / (rows
 *         in rng), or 0 when rng holds no row.  Summed in float64 in a fixed
 *         order, so the result does not vary from run to run, and rounded
 *         once to float32.
 * Unlike the other calls, ntok == 0 still writes *mean (as 0).  The caller
 * copies *mean back whenever it needs the value; nothing here synchronises.
 */
int vl_loss_mean(const float *loss, int64_t ntok, const vl_range *rng, float *mean,
                 hipStream_t stream);

/*
 * Fused distillation KL forward + backward [KL: module doc, kl_rows].
 *   logits  [ntok][V] dtype (student), in: logits; out: gradient
 *           coef * (softmax(row) - t), t_j = probs[q] where ids[q] == j, else 0.
 *   ids     [ntok][k] uint32, read only: the teacher's ids.
 *   probs   [ntok][k] float32, read only: the teacher's probabilities, used
 *           as given (no renormalisation).
 *   loss    [ntok] float32, written: sum over q with probs[q] > 0 of
 *           probs[q] * (ln probs[q] - row[ids[q]] + logsumexp(row)), unscaled.
 *   lse, rng as for vl_ce_fwd_bwd.
 *   coef    gradient scale, e.g. gscale / tokens of the step.
 * Limits: 1 <= k <= V <= 2^19 (two bitmaps of V bits live in LDS).
 */
int vl_kl_fwd_bwd(void *logits, int dtype, const uint32_t *ids, const float *probs, int64_t k,
                  float *loss, float *lse, int64_t ntok, int64_t V, const vl_range *rng,
                  float coef, hipStream_t stream);

/*
 * Workspace bytes the two calls below need at least (256 KiB).
 */
size_t vl_split_workspace_bytes(void);

/*
 * vl_ce_fwd_bwd_ws / vl_kl_fwd_bwd_ws -- vl_ce_fwd_bwd and vl_kl_fwd_bwd
 * with a workspace that lets a row too long for one compute unit's
 * registers be split over 2, 4 or 8 co-resident workgroups [KL: Head, the
 * vocabulary cut into column slices; module doc and kl_rows for the loss
 * and gradient; CE: module doc, backward].  Each workgroup holds one column
 * part of the row in registers; the parts swap their statistics (max, sum
 * of exp, teacher mass and teacher term, 16 bytes) through the workspace,
 * every part forms the row's logsumexp from all of them and writes its part
 * of the gradient from registers, so the row is read once and written once.
 * The split takes rows whose logits pointer is 16-byte aligned with V a
 * multiple of 4 (float32) or 8 (bf16), float32 V in (32768, 524288] and bf16
 * V in (155648, 458752] (the KL's own limit V <= 2^19 still applies); other
 * rows run the kernels of vl_ce_fwd_bwd / vl_kl_fwd_bwd (a bf16 row of up to
 * 155648 values already fits one workgroup's registers) and leave the
 * workspace unused.
 *   workspace        device buffer of at least vl_split_workspace_bytes()
 *                    bytes, owned by the caller; its contents on entry do
 *                    not matter (the call clears what it uses, on `stream`,
 *                    before it starts).  Calls that share a workspace must
 *                    not run at the same time; calls in order on one stream
 *                    may share one.
 *   workspace_bytes  its size.
 * Other arguments, results and limits: as vl_ce_fwd_bwd / vl_kl_fwd_bwd.
 * Losses, lse and gradients agree with theirs within rounding (the row's
 * sums are taken in another order).  The split runs as one cooperative
 * launch, so all its workgroups are resident together; should a part's
 * partners still fail to answer within about a second, that row's loss,
 * lse and gradient come out NaN and the call completes.  On a stream under
 * capture the rows are not split (a cooperative launch is not captured):
 * the call runs vl_ce_fwd_bwd's / vl_kl_fwd_bwd's kernels.
 */
int vl_ce_fwd_bwd_ws(void *logits, int dtype, const uint32_t *labels, float *loss, float *lse,
                     int64_t ntok, int64_t V, const vl_range *rng, float scale, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);
int vl_kl_fwd_bwd_ws(void *logits, int dtype, const uint32_t *ids, const float *probs, int64_t k,
                     float *loss, float *lse, int64_t ntok, int64_t V, const vl_range *rng,
                     float coef, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * vl_kl_fwd_bwd_ws without a workspace argument, for callers that cannot
 * allocate (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the mailbox of the split rows is the library's
 * own device array of vl_split_workspace_bytes() (256 KiB), resident on each
 * device the library runs on until the process ends.  The call allocates
 * nothing (no hipMalloc, no allocating library routine); the first call on
 * a device looks the array's address up once.  The array's size does not
 * depend on ntok, V or k (it holds the mailbox of any launch), so no input
 * size is rejected for it.  Every call on a device shares that device's
 * array and clears what it uses on `stream` before it starts: calls that
 * overlap on one device (on different streams, or from several threads)
 * race and give undefined results; calls in order on one stream are fine.
 * Arguments, results and limits: as vl_kl_fwd_bwd_ws (bit for bit the same
 * results).
 */
int vl_kl_fwd_bwd_noalloc(void *logits, int dtype, const uint32_t *ids, const float *probs,
                          int64_t k, float *loss, float *lse, int64_t ntok, int64_t V,
                          const vl_range *rng, float coef, hipStream_t stream);

/*
 * Teacher top-k with renormalised probabilities [KL: topk_rows].
 *   logits  [ntok][V] dtype, read only.
 *   ids     [ntok][k] uint32, written: the k ids first in the order (value
 *           descending, id ascending); -0 and +0 tie.
 *   probs   [ntok][k] float32, written: exp(v_q - v_0) / sum_{q<k} exp(v_q - v_0)
 *           in the same order (the softmax restricted to the k).
 * Limits: 1 <= k <= min(V, 2048), V <= 2^31 - 1, ntok <= 2^31 - 1.
 */
int vl_topk_renorm(const void *logits, int dtype, int64_t ntok, int64_t V, int64_t k,
                   uint32_t *ids, float *probs, hipStream_t stream);

/*
 * Slice accumulate [KL: acc_add]: dst[i] = dst[i] + src[i] for i < n, the
 * float32 sum rounded to nearest even (bit-exact).
 *   dst [n] float32, read and written;  src [n] float32, read only.
 */
int vl_slice_acc(float *dst, const float *src, int64_t n, hipStream_t stream);

/*
 * The distillation KL over a vocabulary split into slices [KL: module doc
 * (loss and gradient p_S - p_T); Head (the vocabulary cut into column
 * slices, each an offset and a width); head_kl (one product per slice)].
 * Each slice is a block of logits of its own, so no buffer of whole rows is
 * needed; the same three calls serve a vocabulary sharded over devices
 * (exchange the parts, 16 bytes per row and slice, then merge).
 *
 * vl_kl_slice_fwd -- statistics of one slice, one read of it.
 *   logits  slice rows, dtype, read only: row r holds vocabulary ids
 *           [off, off + width) at elements r * ld + [0, width).
 *   ld      row stride in elements, >= width (width for a dense block).
 *   off     vocabulary id of the slice's first column, >= 0.
 *   ids     [ntok][k] uint32, probs [ntok][k] float32, read only: the
 *           teacher's ids and probabilities over the whole vocabulary; each
 *           slice uses the entries whose id falls into it.
 *   part    [ntok][4] float32, written, 16-byte aligned: per row
 *             a = max of the slice's values (0 if none is finite),
 *             z = sum_j exp(s_j - a),
 *             P = sum of probs[q] > 0 whose id is in the slice,
 *             w = sum over those q of probs[q] (ln probs[q] - (s_id - a)).
 *           Rows outside the loss range get (0, 0, 0, 0) and are not read.
 * vl_kl_slice_merge -- the whole rows' loss and logsumexp from the parts of
 * every slice (the slices must partition [0, V) and the parts be written
 * with the same rng).
 *   parts   [nslice][ntok][4] float32, read only, 16-byte aligned: the
 *           nslice slices' part buffers back to back.
 *   loss    [ntok] float32, written: sum over slices with P > 0 of
 *           w + P (lse - a), which is vl_kl_fwd_bwd's loss of the whole row.
 *   lse     [ntok] float32 or NULL, written: ln sum over slices with z > 0
 *           of z exp(a).
 *   Rows outside the loss range get loss 0 and lse 0.
 * vl_kl_slice_bwd -- the gradient of one slice, one read and one write.
 *   logits  as for vl_kl_slice_fwd; in: the logits, out: the gradient
 *           coef (exp(s_j - lse) - t_j), t_j = probs[q] where ids[q] = off + j,
 *           stored in dtype.
 *   lse     [ntok] float32, read only: the merged logsumexp, used as given.
 *   Rows outside the loss range are set to 0 and not read.
 * Cross-entropy over slices is the same calls with k = 1, ids = labels and
 * probs = 1.
 * Limits: 1 <= width, off + width <= 2^31 - 1, ld >= width, k >= 1,
 * nslice >= 1.  Ids outside every slice contribute nothing.  Slice rows are
 * read as 16-byte vectors when the logits pointer is 16-byte aligned and
 * ld and width times the element size are multiples of 16; otherwise one
 * element at a time (same results, slower).
 */
int vl_kl_slice_fwd(const void *logits, int dtype, int64_t ld, int64_t off, int64_t width,
                    const uint32_t *ids, const float *probs, int64_t k, float *part,
                    int64_t ntok, const vl_range *rng, hipStream_t stream);
int vl_kl_slice_merge(const float *parts, int64_t nslice, float *loss, float *lse,
                      int64_t ntok, const vl_range *rng, hipStream_t stream);
int vl_kl_slice_bwd(void *logits, int dtype, int64_t ld, int64_t off, int64_t width,
                    const uint32_t *ids, const float *probs, int64_t k, const float *lse,
                    int64_t ntok, const vl_range *rng, float coef, hipStream_t stream);

/*
 * Scratch bytes vl_head_kl needs for `chunk` rows at a time, each region
 * 256-byte aligned: float32 logits [chunk][V], the half-precision hidden
 * rows [chunk][hs rounded up to 64], the half-precision gradient [chunk][V],
 * the (max, sum exp) records of every 128 columns [chunk][2 ceil(V/256)]
 * (8 bytes each), lse [chunk], the loss sums of every 2048 columns
 * [chunk][ceil(V/2048)] (float32), and a 64 MiB GEMM workspace.  0 for
 * invalid sizes.
 */
size_t vl_head_scratch_bytes(int64_t chunk, int64_t V, int64_t hs);

/*
 * Vocabulary head with the distillation KL [KL: head_kl, Head, HeadScratch]:
 * for chunks of `chunk` rows,
 *   act    = half(x rows)                        (round to nearest even)
 *   logits = act . w^T                           (float32 accumulation)
 *   KL rows as vl_kl_fwd_bwd with coef = gscale / total, giving loss and the
 *           gradient coef (softmax - t) over the logits
 *   dx     = half(gradient) . w / gscale          (float32 accumulation)
 * so dx is the gradient of (sum of the rows' KL) / total with respect to x,
 * the teacher term applied as given.
 *   x       [ntok][hs] float32, read only: the normed hidden rows.
 *   w       [V][hs] head weights in wdtype (VL_F16 or VL_BF16), read only.
 *   ids, probs, k   as for vl_kl_fwd_bwd.
 *   dx      [ntok][hs] float32, written.
 *   loss    [ntok] float32, written: the KL of each row, unscaled.
 *   total   the tokens the step averages over (>= 1); gscale != 0, finite.
 *   scratch device buffer of at least vl_head_scratch_bytes(min(chunk,
 *           ntok), V, hs) bytes, owned by the caller; its contents on entry
 *           do not matter and are undefined after the call.
 * The logits product runs on this library's matrix-core kernel, which also
 * forms each row's softmax statistics, when hs is a multiple of 8 and x and
 * w are 16-byte aligned (otherwise in hipBLASLt, followed by the fused KL
 * row kernel); the dx product runs in hipBLASLt.  The hipBLASLt handle is
 * created on the first call on each device and kept until the process ends
 * (the only allocation the library makes).  Each hipBLASLt product runs the
 * algorithm that vl_head_kl_tune (or vl_head_topk_tune) chose for its shape
 * on this device, or, for a shape not tuned, hipBLASLt's first choice; the
 * call never waits for the stream.
 * Limits: 1 <= k <= V <= 2^19, hs >= 1, chunk >= 1.
 * Returns VL_ELAUNCH if hipBLASLt finds no algorithm or rejects a call.
 */
int vl_head_kl(const float *x, const void *w, int wdtype, const uint32_t *ids,
               const float *probs, int64_t k, float *dx, float *loss, int64_t ntok, int64_t V,
               int64_t hs, int64_t total, float gscale, int64_t chunk, void *scratch,
               size_t scratch_bytes, hipStream_t stream);

/*
 * vl_head_kl_tune -- vl_head_kl (same arguments, same results) that first
 * picks the algorithm of each hipBLASLt product shape not yet tuned on this
 * device, for callers who set up once and then call vl_head_kl: it times
 * up to 16 of hipBLASLt's candidates on `stream` (one untimed and two timed
 * runs each, the three fastest again, four runs each in turns) on the
 * call's own operands, and keeps the fastest for every later head call with
 * that shape.  This call waits for `stream` while it times (the host
 * blocks); shapes already tuned run as in vl_head_kl.  Under stream capture
 * nothing is timed.  Tuned and untuned calls may differ in float32 rounding
 * of the products (another algorithm sums in another order).
 */
int vl_head_kl_tune(const float *x, const void *w, int wdtype, const uint32_t *ids,
                    const float *probs, int64_t k, float *dx, float *loss, int64_t ntok,
                    int64_t V, int64_t hs, int64_t total, float gscale, int64_t chunk,
                    void *scratch, size_t scratch_bytes, hipStream_t stream);

/*
 * Scratch bytes vl_head_topk needs for `chunk` rows at a time, each region
 * 256-byte aligned: float32 logits [chunk][V], the half-precision hidden
 * rows [chunk][hs rounded up to 64] and a 64 MiB GEMM workspace (0 for
 * invalid sizes).
 */
size_t vl_head_topk_scratch_bytes(int64_t chunk, int64_t V, int64_t hs);

/*
 * The teacher side of the vocabulary head [KL: topk (the host function:
 * hidden rows to half precision, the logits product per slice, topk_rows
 * per chunk of rows), Head, HeadScratch]: for chunks of `chunk` rows,
 *   act    = half(x rows)                  (round to nearest even)
 *   logits = act . w^T                     (float32 accumulation)
 *   ids, probs = vl_topk_renorm of the float32 logits rows
 * so each row gets the k ids first in the order (logit descending, id
 * ascending) and their probabilities renormalised over the k.
 *   x       [ntok][hs] float32, read only: the teacher's normed hidden rows.
 *   w       [V][hs] head weights in wdtype (VL_F16 or VL_BF16), read only.
 *   ids     [ntok][k] uint32, written.
 *   probs   [ntok][k] float32, written.
 *   scratch device buffer of at least vl_head_topk_scratch_bytes(min(chunk,
 *           ntok), V, hs) bytes, owned by the caller; contents on entry do
 *           not matter and are undefined after the call.
 * The product runs on this library's matrix-core kernel when hs is a
 * multiple of 8 and x and w are 16-byte aligned, otherwise in hipBLASLt, as
 * in vl_head_kl (same handle, same per-shape algorithm choice; the call
 * never waits for the stream).
 * Limits: 1 <= k <= min(V, 2048), V <= 2^31 - 1, hs >= 1, chunk >= 1,
 * ntok <= 2^31 - 1.
 */
int vl_head_topk(const float *x, const void *w, int wdtype, int64_t ntok, int64_t V, int64_t hs,
                 int64_t k, uint32_t *ids, float *probs, int64_t chunk, void *scratch,
                 size_t scratch_bytes, hipStream_t stream);

/*
 * vl_head_topk_tune -- vl_head_topk (same arguments, same results) that
 * first times hipBLASLt's candidates for its product shape when that
 * product runs in hipBLASLt and the shape is not yet tuned, as
 * vl_head_kl_tune does (this call then waits for `stream`).
 */
int vl_head_topk_tune(const float *x, const void *w, int wdtype, int64_t ntok, int64_t V,
                      int64_t hs, int64_t k, uint32_t *ids, float *probs, int64_t chunk,
                      void *scratch, size_t scratch_bytes, hipStream_t stream);

/* Static text naming a status code. */
const char *vl_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* VL_H */
