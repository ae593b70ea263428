// C ABI of libvl.so (declared in include/vl.h): host-side argument checks,
// then one asynchronous launch on the caller's stream.  No allocation, no
// synchronisation, no retained pointers.
#include "vl.h"

#include <hip/hip_runtime.h>

#include <math.h>

#include <mutex>

#include "vl_launch.hpp"

namespace vl {

int device_cus()
{
    static std::mutex mu;
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    std::lock_guard<std::mutex> lock(mu);
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 1)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

namespace {

struct OccKey {
    const void *fn;
    size_t lds;
    int dev;
};

}  // namespace

int blocks_per_cu(const void *fn, int block, size_t lds)
{
    static thread_local OccKey keys[64];
    static thread_local int vals[64];
    static thread_local int n = 0;
    int dev = 0;
    (void)hipGetDevice(&dev);
    for (int i = 0; i < n; ++i)
        if (keys[i].fn == fn && keys[i].lds == lds && keys[i].dev == dev)
            return vals[i];
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, block, lds) != hipSuccess)
        nb = 1;
    if (nb < 1)
        nb = 1;
    if (n < 64) {
        keys[n] = {fn, lds, dev};
        vals[n] = nb;
        ++n;
    }
    return nb;
}

}  // namespace vl

namespace {

constexpr int64_t kMaxV = (int64_t(1) << 31) - 1;

bool bad_dtype(int dtype) { return dtype != VL_F32 && dtype != VL_BF16; }

// Shared checks of the two loss calls; fills the range fields of `a`.
int check_rows(int dtype, int64_t ntok, int64_t V, const vl_range *rng, vl::RowArgs &a)
{
    if (bad_dtype(dtype))
        return VL_EDTYPE;
    if (ntok < 0 || V < 1 || V > kMaxV)
        return VL_EINVAL;
    if (ntok > INT64_MAX / V)
        return VL_EINVAL;
    if (rng) {
        if (rng->seq_len < 1 || rng->start < 0 || rng->start > rng->end ||
            rng->end > rng->seq_len)
            return VL_EINVAL;
        a.walk = vl::make_walk(ntok, rng->seq_len, rng->start, rng->end);
    } else {
        a.walk = vl::make_walk(ntok, 0, 0, 0);
    }
    a.ntok = ntok;
    a.V = V;
    return VL_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? VL_OK : VL_ELAUNCH; }

// check_rows plus the KL's limits: V <= kMaxKlVocab, 1 <= k <= V.
int check_kl(int dtype, int64_t ntok, int64_t V, int64_t k, const vl_range *rng,
             vl::RowArgs &a)
{
    int st = check_rows(dtype, ntok, V, rng, a);
    if (st != VL_OK)
        return st;
    if (V > vl::kMaxKlVocab || k < 1 || k > V)
        return VL_EINVAL;
    if (ntok > INT64_MAX / k)
        return VL_EINVAL;
    a.k = k;
    return VL_OK;
}

}  // namespace

extern "C" {

int vl_ce_fwd_bwd(void *logits, int dtype, const uint32_t *labels, float *loss, float *lse,
                  int64_t ntok, int64_t V, const vl_range *rng, float scale,
                  hipStream_t stream)
{
    vl::RowArgs a{};
    int st = check_rows(dtype, ntok, V, rng, a);
    if (st != VL_OK)
        return st;
    if (ntok == 0)
        return VL_OK;
    if (!logits || !labels || !loss)
        return VL_EINVAL;
    a.logits = logits;
    a.labels = labels;
    a.loss = loss;
    a.lse = lse;
    a.k = 1;
    a.coef = scale;
    return status_of(vl::launch_rows(dtype, false, a, stream));
}

size_t vl_split_workspace_bytes(void) { return vl::kSplitWorkspaceBytes; }

}  // extern "C"

namespace {

// Rows the single-CU kernels cannot hold on chip go to the split kernels:
// float32 rows past 8192 16-byte vectors (32768 values), bf16 rows past the
// 19456 vectors (155648 values) a 1024-thread block holds in registers.  The
// bf16 rows in between run faster whole in one block's registers (16384 x
// 151936: 1.98 ms, against 2.03-2.10 ms split over 4 to 8 workgroups) and
// need no exchange.
// A split is one cooperative launch, which a stream under capture does not
// take: captured calls run the rows whole (the same results within rounding).
bool use_split(int dtype, const vl::RowArgs &a, int &S, hipStream_t stream)
{
    const int N = dtype == VL_F32 ? 4 : 8;
    if ((uintptr_t)a.logits % 16 != 0 || a.V % N != 0)
        return false;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
        return false;
    const int64_t nvec = a.V / N;
    if (nvec <= (dtype == VL_F32 ? 8192 : 19456))
        return false;
    S = vl::split_parts(dtype, a.V);
    return S > 0;
}

int rows_ws(int dtype, bool kl, const vl::RowArgs &a, void *ws, size_t ws_bytes,
            hipStream_t stream)
{
    int S = 0;
    if (use_split(dtype, a, S, stream))
        return status_of(vl::launch_rows_split(dtype, kl, a, S, ws, ws_bytes, stream));
    return status_of(vl::launch_rows(dtype, kl, a, stream));
}

}  // namespace

extern "C" {

int vl_ce_fwd_bwd_ws(void *logits, int dtype, const uint32_t *labels, float *loss, float *lse,
                     int64_t ntok, int64_t V, const vl_range *rng, float scale, void *workspace,
                     size_t workspace_bytes, hipStream_t stream)
{
    vl::RowArgs a{};
    int st = check_rows(dtype, ntok, V, rng, a);
    if (st != VL_OK)
        return st;
    if (ntok == 0)
        return VL_OK;
    if (!logits || !labels || !loss || !workspace || workspace_bytes < vl::kSplitWorkspaceBytes)
        return VL_EINVAL;
    a.logits = logits;
    a.labels = labels;
    a.loss = loss;
    a.lse = lse;
    a.k = 1;
    a.coef = scale;
    return rows_ws(dtype, false, a, workspace, workspace_bytes, stream);
}

int vl_kl_fwd_bwd_ws(void *logits, int dtype, const uint32_t *ids, const float *probs, int64_t k,
                     float *loss, float *lse, int64_t ntok, int64_t V, const vl_range *rng,
                     float coef, void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    vl::RowArgs a{};
    int st = check_kl(dtype, ntok, V, k, rng, a);
    if (st != VL_OK)
        return st;
    if (ntok == 0)
        return VL_OK;
    if (!logits || !ids || !probs || !loss || !workspace ||
        workspace_bytes < vl::kSplitWorkspaceBytes)
        return VL_EINVAL;
    a.logits = logits;
    a.ids = ids;
    a.probs = probs;
    a.loss = loss;
    a.lse = lse;
    a.coef = coef;
    return rows_ws(dtype, true, a, workspace, workspace_bytes, stream);
}

int vl_kl_fwd_bwd_noalloc(void *logits, int dtype, const uint32_t *ids, const float *probs,
                          int64_t k, float *loss, float *lse, int64_t ntok, int64_t V,
                          const vl_range *rng, float coef, hipStream_t stream)
{
    vl::RowArgs a{};
    int st = check_kl(dtype, ntok, V, k, rng, a);
    if (st != VL_OK)
        return st;
    if (ntok == 0)
        return VL_OK;
    if (!logits || !ids || !probs || !loss)
        return VL_EINVAL;
    a.logits = logits;
    a.ids = ids;
    a.probs = probs;
    a.loss = loss;
    a.lse = lse;
    a.coef = coef;
    int S = 0;
    if (!use_split(dtype, a, S, stream))
        return status_of(vl::launch_rows(dtype, true, a, stream));
    void *ws = nullptr;
    if (vl::split_scratch(&ws) != hipSuccess)
        return VL_ELAUNCH;
    return status_of(vl::launch_rows_split(dtype, true, a, S, ws, vl::kSplitWorkspaceBytes,
                                           stream));
}

int vl_ce_fwd(const void *logits, int dtype, const uint32_t *labels, float *loss, float *lse,
              int64_t ntok, int64_t V, const vl_range *rng, hipStream_t stream)
{
    vl::RowArgs a{};
    int st = check_rows(dtype, ntok, V, rng, a);
    if (st != VL_OK)
        return st;
    if (ntok == 0)
        return VL_OK;
    if (!logits || !labels || !loss)
        return VL_EINVAL;
    // read only: the kernel never stores through it
    a.logits = const_cast<void *>(logits);
    a.labels = labels;
    a.loss = loss;
    a.lse = lse;
    return status_of(vl::launch_ce_fwd(dtype, a, stream));
}

int vl_ce_bwd(void *logits, int dtype, const uint32_t *labels, const float *lse, int64_t ntok,
              int64_t V, const vl_range *rng, float scale, hipStream_t stream)
{
    vl::RowArgs a{};
    int st = check_rows(dtype, ntok, V, rng, a);
    if (st != VL_OK)
        return st;
    if (ntok == 0)
        return VL_OK;
    if (!logits || !labels || !lse)
        return VL_EINVAL;
    a.logits = logits;
    a.labels = labels;
    a.lse = const_cast<float *>(lse);  // read only in the backward
    a.coef = scale;
    return status_of(vl::launch_ce_bwd(dtype, a, stream));
}

int vl_loss_mean(const float *loss, int64_t ntok, const vl_range *rng, float *mean,
                 hipStream_t stream)
{
    vl::RowArgs a{};
    // the range checks of the loss calls (dtype and V play no part here)
    int st = check_rows(VL_F32, ntok, 1, rng, a);
    if (st != VL_OK)
        return st;
    if (!mean || (ntok > 0 && !loss))
        return VL_EINVAL;
    return status_of(vl::launch_loss_mean(loss, ntok, a.walk.n_in, mean, stream));
}

size_t vl_head_scratch_bytes(int64_t chunk, int64_t V, int64_t hs)
{
    if (chunk < 1 || V < 1 || hs < 1 || V > vl::kMaxKlVocab || hs > kMaxV)
        return 0;
    return vl::head_scratch_bytes(chunk, V, hs);
}

}  // extern "C"

namespace {

int head_kl_call(const float *x, const void *w, int wdtype, const uint32_t *ids,
                 const float *probs, int64_t k, float *dx, float *loss, int64_t ntok, int64_t V,
                 int64_t hs, int64_t total, float gscale, int64_t chunk, void *scratch,
                 size_t scratch_bytes, bool tune, hipStream_t stream)
{
    if (wdtype != VL_BF16 && wdtype != VL_F16)
        return VL_EDTYPE;
    if (ntok < 0 || V < 1 || V > vl::kMaxKlVocab || hs < 1 || hs > kMaxV || k < 1 || k > V ||
        total < 1 || chunk < 1 || !(gscale != 0.f) || !isfinite(gscale))
        return VL_EINVAL;
    if (ntok > INT64_MAX / (V > hs ? V : hs) || ntok > INT64_MAX / k)
        return VL_EINVAL;
    if (ntok == 0)
        return VL_OK;
    if (!x || !w || !ids || !probs || !dx || !loss || !scratch)
        return VL_EINVAL;
    const int64_t c = chunk < ntok ? chunk : ntok;
    if (scratch_bytes < vl::head_scratch_bytes(c, V, hs))
        return VL_EINVAL;
    vl::HeadArgs a{x, w, wdtype, ids, probs, dx, loss, ntok, V, hs, k, total, c, gscale,
                   scratch, tune};
    return vl::head_kl(a, stream);
}

}  // namespace

extern "C" {

int vl_head_kl(const float *x, const void *w, int wdtype, const uint32_t *ids,
               const float *probs, int64_t k, float *dx, float *loss, int64_t ntok, int64_t V,
               int64_t hs, int64_t total, float gscale, int64_t chunk, void *scratch,
               size_t scratch_bytes, hipStream_t stream)
{
    return head_kl_call(x, w, wdtype, ids, probs, k, dx, loss, ntok, V, hs, total, gscale, chunk,
                        scratch, scratch_bytes, false, stream);
}

int vl_head_kl_tune(const float *x, const void *w, int wdtype, const uint32_t *ids,
                    const float *probs, int64_t k, float *dx, float *loss, int64_t ntok,
                    int64_t V, int64_t hs, int64_t total, float gscale, int64_t chunk,
                    void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    return head_kl_call(x, w, wdtype, ids, probs, k, dx, loss, ntok, V, hs, total, gscale, chunk,
                        scratch, scratch_bytes, true, stream);
}

size_t vl_head_topk_scratch_bytes(int64_t chunk, int64_t V, int64_t hs)
{
    if (chunk < 1 || V < 1 || hs < 1 || V > kMaxV || hs > kMaxV)
        return 0;
    if (chunk > INT64_MAX / V / 8)
        return 0;
    return vl::head_topk_scratch_bytes(chunk, V, hs);
}

}  // extern "C"

namespace {

int head_topk_call(const float *x, const void *w, int wdtype, int64_t ntok, int64_t V,
                   int64_t hs, int64_t k, uint32_t *ids, float *probs, int64_t chunk,
                   void *scratch, size_t scratch_bytes, bool tune, hipStream_t stream)
{
    if (wdtype != VL_BF16 && wdtype != VL_F16)
        return VL_EDTYPE;
    if (ntok < 0 || V < 1 || V > kMaxV || hs < 1 || hs > kMaxV || k < 1 || k > V ||
        k > vl::kMaxTopk || chunk < 1 || ntok > INT32_MAX)
        return VL_EINVAL;
    if (ntok > INT64_MAX / (V > hs ? V : hs) || chunk > INT64_MAX / V / 8)
        return VL_EINVAL;
    if (ntok == 0)
        return VL_OK;
    if (!x || !w || !ids || !probs || !scratch)
        return VL_EINVAL;
    const int64_t c = chunk < ntok ? chunk : ntok;
    if (scratch_bytes < vl::head_topk_scratch_bytes(c, V, hs))
        return VL_EINVAL;
    vl::HeadTopkArgs a{x, w, wdtype, ntok, V, hs, k, c, ids, probs, scratch, tune};
    return vl::head_topk(a, stream);
}

}  // namespace

extern "C" {

int vl_head_topk(const float *x, const void *w, int wdtype, int64_t ntok, int64_t V, int64_t hs,
                 int64_t k, uint32_t *ids, float *probs, int64_t chunk, void *scratch,
                 size_t scratch_bytes, hipStream_t stream)
{
    return head_topk_call(x, w, wdtype, ntok, V, hs, k, ids, probs, chunk, scratch,
                          scratch_bytes, false, stream);
}

int vl_head_topk_tune(const float *x, const void *w, int wdtype, int64_t ntok, int64_t V,
                      int64_t hs, int64_t k, uint32_t *ids, float *probs, int64_t chunk,
                      void *scratch, size_t scratch_bytes, hipStream_t stream)
{
    return head_topk_call(x, w, wdtype, ntok, V, hs, k, ids, probs, chunk, scratch,
                          scratch_bytes, true, stream);
}

int vl_kl_fwd_bwd(void *logits, int dtype, const uint32_t *ids, const float *probs, int64_t k,
                  float *loss, float *lse, int64_t ntok, int64_t V, const vl_range *rng,
                  float coef, hipStream_t stream)
{
    vl::RowArgs a{};
    int st = check_kl(dtype, ntok, V, k, rng, a);
    if (st != VL_OK)
        return st;
    if (ntok == 0)
        return VL_OK;
    if (!logits || !ids || !probs || !loss)
        return VL_EINVAL;
    a.logits = logits;
    a.ids = ids;
    a.probs = probs;
    a.loss = loss;
    a.lse = lse;
    a.coef = coef;
    return status_of(vl::launch_rows(dtype, true, a, stream));
}

int vl_topk_renorm(const void *logits, int dtype, int64_t ntok, int64_t V, int64_t k,
                   uint32_t *ids, float *probs, hipStream_t stream)
{
    if (bad_dtype(dtype))
        return VL_EDTYPE;
    // one wave per row: the grid holds at most 2^31 - 1 workgroups
    if (ntok < 0 || ntok > kMaxV || V < 1 || V > kMaxV || k < 1 || k > V || k > vl::kMaxTopk)
        return VL_EINVAL;
    if (ntok > INT64_MAX / V)
        return VL_EINVAL;
    if (ntok == 0)
        return VL_OK;
    if (!logits || !ids || !probs)
        return VL_EINVAL;
    vl::TopkArgs a{logits, ntok, V, k, ids, probs};
    return status_of(vl::launch_topk(dtype, a, stream));
}

int vl_slice_acc(float *dst, const float *src, int64_t n, hipStream_t stream)
{
    if (n < 0)
        return VL_EINVAL;
    if (n == 0)
        return VL_OK;
    if (!dst || !src)
        return VL_EINVAL;
    return status_of(vl::launch_slice_acc(dst, src, n, stream));
}

// Shared checks of the two slice passes; fills `a` except the pass's own
// pointers.
static int check_slice(const void *logits, int dtype, int64_t ld, int64_t off, int64_t width,
                       const uint32_t *ids, const float *probs, int64_t k, int64_t ntok,
                       const vl_range *rng, vl::SliceArgs &a)
{
    vl::RowArgs r{};
    int st = check_rows(dtype, ntok, width, rng, r);
    if (st != VL_OK)
        return st;
    if (ld < width || off < 0 || off > kMaxV - width || k < 1)
        return VL_EINVAL;
    if (ntok > INT64_MAX / ld || ntok > INT64_MAX / k)
        return VL_EINVAL;
    if (ntok > 0 && (!logits || !ids || !probs))
        return VL_EINVAL;
    a.logits = const_cast<void *>(logits);
    a.ids = ids;
    a.probs = probs;
    a.ntok = ntok;
    a.ld = ld;
    a.off = off;
    a.width = width;
    a.k = k;
    a.walk = r.walk;
    return VL_OK;
}

int vl_kl_slice_fwd(const void *logits, int dtype, int64_t ld, int64_t off, int64_t width,
                    const uint32_t *ids, const float *probs, int64_t k, float *part,
                    int64_t ntok, const vl_range *rng, hipStream_t stream)
{
    vl::SliceArgs a{};
    int st = check_slice(logits, dtype, ld, off, width, ids, probs, k, ntok, rng, a);
    if (st != VL_OK)
        return st;
    if (ntok == 0)
        return VL_OK;
    if (!part || (uintptr_t)part % 16 != 0)
        return VL_EINVAL;
    a.part = part;
    return status_of(vl::launch_slice_part(dtype, a, stream));
}

int vl_kl_slice_merge(const float *parts, int64_t nslice, float *loss, float *lse,
                      int64_t ntok, const vl_range *rng, hipStream_t stream)
{
    vl::RowArgs r{};
    int st = check_rows(VL_F32, ntok, 1, rng, r);
    if (st != VL_OK)
        return st;
    if (nslice < 1 || ntok > INT64_MAX / 16 / nslice)
        return VL_EINVAL;
    if (ntok == 0)
        return VL_OK;
    if (!parts || (uintptr_t)parts % 16 != 0 || !loss)
        return VL_EINVAL;
    return status_of(vl::launch_slice_merge(parts, nslice, ntok, r.walk, loss, lse, stream));
}

int vl_kl_slice_bwd(void *logits, int dtype, int64_t ld, int64_t off, int64_t width,
                    const uint32_t *ids, const float *probs, int64_t k, const float *lse,
                    int64_t ntok, const vl_range *rng, float coef, hipStream_t stream)
{
    vl::SliceArgs a{};
    int st = check_slice(logits, dtype, ld, off, width, ids, probs, k, ntok, rng, a);
    if (st != VL_OK)
        return st;
    if (ntok == 0)
        return VL_OK;
    if (!lse)
        return VL_EINVAL;
    a.lse = lse;
    a.coef = coef;
    return status_of(vl::launch_slice_bwd(dtype, a, stream));
}

const char *vl_strerror(int status)
{
    switch (status) {
    case VL_OK:
        return "ok";
    case VL_EINVAL:
        return "invalid argument (size, range, k or null pointer)";
    case VL_EDTYPE:
        return "unknown dtype (expected VL_F32 or VL_BF16)";
    case VL_ELAUNCH:
        return "the HIP runtime rejected a kernel launch, or hipBLASLt a product";
    default:
        return "unknown status";
    }
}

}  // extern "C"
