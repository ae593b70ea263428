// Internal interface between the C ABI (vl_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vl {

// The order in which a persistent grid visits the rows: the rows in the
// loss range first (index j in [0, n_in)), then the rows outside it
// (j in [0, n_out)).  Row r is in the range iff start <= r mod seq_len < end;
// seq_len <= 0 means every row is.  In-range index j is row
// (j / len_in) * seq_len + start + j % len_in; out-of-range index j is
// position q = j % len_out of sequence j / len_out, where positions
// [0, start) come first and then [end, seq_len).
struct RowWalk {
    int64_t n_in, n_out;
    int64_t seq_len, start, len_in, len_out;
};

// Walks one of the two lists in steps of `stride` without dividing per
// step: (seq, pos) of index j is kept and advanced by the quotient and
// remainder of the stride, computed once.
struct RowCursor {
    int64_t j, seq, pos;      // current index and its (quotient, remainder)
    int64_t len;              // list entries per sequence (len_in or len_out)
    int64_t step_q, step_r;   // stride / len, stride % len

    __host__ __device__ void init(int64_t j0, int64_t stride, int64_t l)
    {
        j = j0;
        len = l > 0 ? l : 1;
        seq = j0 / len;
        pos = j0 % len;
        step_q = stride / len;
        step_r = stride % len;
    }
    __host__ __device__ void advance()
    {
        j += step_q * len + step_r;
        seq += step_q;
        pos += step_r;
        if (pos >= len) {
            pos -= len;
            ++seq;
        }
    }
    __host__ __device__ int64_t in_row(const RowWalk &w) const
    {
        return w.seq_len <= 0 ? j : seq * w.seq_len + w.start + pos;
    }
    __host__ __device__ int64_t out_row(const RowWalk &w) const
    {
        return seq * w.seq_len + (pos < w.start ? pos : pos + w.len_in);
    }
};

// The two lists for `ntok` rows and the range (seq_len, start, end);
// seq_len <= 0: every row is in the loss.
inline RowWalk make_walk(int64_t ntok, int64_t seq_len, int64_t start, int64_t end)
{
    RowWalk w{};
    if (seq_len <= 0) {
        w.n_in = ntok;
        return w;
    }
    w.seq_len = seq_len;
    w.start = start;
    w.len_in = end - start;
    w.len_out = seq_len - w.len_in;
    const int64_t full = ntok / seq_len, rem = ntok % seq_len;
    int64_t last = (rem < end ? rem : end) - start;
    if (last < 0)
        last = 0;
    w.n_in = full * w.len_in + last;
    w.n_out = ntok - w.n_in;
    return w;
}

// One call of the fused CE or KL row kernel.
struct RowArgs {
    void *logits;             // [ntok][V] float32 or bf16, in: logits, out: gradient
    const uint32_t *labels;   // CE: [ntok]
    const uint32_t *ids;      // KL: [ntok][k]
    const float *probs;       // KL: [ntok][k]
    float *loss;              // [ntok]
    float *lse;               // [ntok] or null
    int64_t ntok, V, k;
    RowWalk walk;             // loss range as a row order
    float coef;               // gradient scale
    int64_t lds_vecs;         // online: leading vectors of a row kept in LDS for pass 2
    void *gout;               // out != 0: [ntok][V] half-precision gradient rows
};

// One call of the per-slice KL passes (checked by the caller).
struct SliceArgs {
    void *logits;           // row r of the slice starts at element r * ld
    const uint32_t *ids;    // [ntok][k]
    const float *probs;     // [ntok][k]
    float *part;            // part pass: [ntok][4], 16-byte aligned
    const float *lse;       // gradient pass: [ntok]
    int64_t ntok, ld, off, width, k;
    RowWalk walk;           // loss range as a row order
    float coef;             // gradient scale
};

struct TopkArgs {
    const void *logits;  // [ntok][V]
    int64_t ntok, V, k;
    uint32_t *ids;       // [ntok][k]
    float *probs;        // [ntok][k]
};

// One call of the vocabulary head with the KL (checked by the caller).
struct HeadArgs {
    const float *x;         // [ntok][hs] hidden rows
    const void *w;          // [V][hs] head weights, wdtype
    int wdtype;             // VL_F16 or VL_BF16
    const uint32_t *ids;    // [ntok][k]
    const float *probs;     // [ntok][k]
    float *dx;              // [ntok][hs]
    float *loss;            // [ntok]
    int64_t ntok, V, hs, k, total, chunk;
    float gscale;
    void *scratch;          // head_scratch_bytes(min(chunk, ntok), V, hs) bytes
};

// Scratch bytes of one head call with `chunk` rows at a time.
size_t head_scratch_bytes(int64_t chunk, int64_t V, int64_t hs);
// Returns a VL_ status.
int head_kl(const HeadArgs &a, hipStream_t stream);

// Each returns hipSuccess or the HIP error of the launch.
// out = 0: the gradient is written over the logits; out = 1 / 2: float32 KL
// rows write it rounded to bf16 / f16 into a.gout and leave the logits.
hipError_t launch_rows(int dtype, bool kl, const RowArgs &a, hipStream_t stream, int out = 0);
hipError_t launch_topk(int dtype, const TopkArgs &a, hipStream_t stream);
hipError_t launch_slice_acc(float *dst, const float *src, int64_t n, hipStream_t stream);
// Cross-entropy in two calls, with RowArgs as for launch_rows: the forward
// reads the logits and writes loss and lse (lse may be null); the backward
// reads lse and writes the gradient over the logits (coef is the scale).
hipError_t launch_ce_fwd(int dtype, const RowArgs &a, hipStream_t stream);
hipError_t launch_ce_bwd(int dtype, const RowArgs &a, hipStream_t stream);
// mean[0] = (sum of loss[0..n)) / count, or 0 when count is 0.
hipError_t launch_loss_mean(const float *loss, int64_t n, int64_t count, float *mean,
                            hipStream_t stream);

// The vocabulary-slice KL: per-row statistics of one slice, their merge
// over nslice slices ([nslice][ntok][4]) into loss and lse (lse may be
// null), and one slice's gradient from lse.
hipError_t launch_slice_part(int dtype, const SliceArgs &a, hipStream_t stream);
hipError_t launch_slice_merge(const float *parts, int64_t nslice, int64_t ntok,
                              const RowWalk &walk, float *loss, float *lse, hipStream_t stream);
hipError_t launch_slice_bwd(int dtype, const SliceArgs &a, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cus();

// Resident blocks per CU of kernel `fn` with `block` threads and `lds` bytes
// of dynamic LDS on the current device (at least 1; cached).
int blocks_per_cu(const void *fn, int block, size_t lds);

// Largest KL vocabulary: two row bitmaps of V bits must fit in LDS.
constexpr int64_t kMaxKlVocab = int64_t(1) << 19;
// Largest top-k k.
constexpr int64_t kMaxTopk = 2048;

}  // namespace vl
