// The C ABI used from native host code alone (include/vl.h + libvl.so, the
// HIP runtime for memory and a stream; no Python): each call on inputs
// whose results have a closed form, plus the host-side error codes.
// Exit status 0 when every check holds; prints the first failure otherwise.
//
//   CE on a constant row:        loss = ln V, g_j = scale (1/V - [j = label])
//   KL, uniform student, uniform teacher over k ids:  loss = ln(V / k)
//   the same KL over two vocabulary slices (fwd, merge, bwd)
//   top-k of a row holding a permutation of 0..V-1: ids = the positions of
//   V-1, V-2, ...; probs = softmax over those k values
//   slice accumulate: the float32 sum
#include <hip/hip_runtime_api.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "vl.h"

static int failures = 0;

#define CHECK(cond, ...)                                                       \
    do {                                                                       \
        if (!(cond)) {                                                         \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);               \
            fprintf(stderr, __VA_ARGS__);                                      \
            fprintf(stderr, "\n");                                             \
            ++failures;                                                        \
        }                                                                      \
    } while (0)

#define HIP_OK(x)                                                              \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
            exit(2);                                                           \
        }                                                                      \
    } while (0)

static void *dev_alloc(size_t bytes)
{
    void *p = NULL;
    HIP_OK(hipMalloc(&p, bytes));
    return p;
}

static int close_rel(double got, double want, double rtol, double atol)
{
    return fabs(got - want) <= rtol * fabs(want) + atol;
}

int main(void)
{
    hipStream_t st;
    HIP_OK(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));

    // ---- host-side argument checks (no GPU work)
    CHECK(vl_ce_fwd_bwd(NULL, 7, NULL, NULL, NULL, 4, 10, NULL, 1.f, st) == VL_EDTYPE,
          "unknown dtype");
    CHECK(vl_kl_fwd_bwd(NULL, VL_F32, NULL, NULL, 0, NULL, NULL, 4, 10, NULL, 1.f, st) ==
              VL_EINVAL,
          "k = 0");
    CHECK(vl_topk_renorm(NULL, VL_F32, 0, 10, 3, NULL, NULL, st) == VL_OK, "ntok = 0 no-op");
    CHECK(vl_strerror(VL_EINVAL) != NULL && strlen(vl_strerror(VL_EINVAL)) > 0, "strerror");

    // ---- CE on constant rows
    {
        const int64_t ntok = 8, V = 4096;
        const float c = 1.25f, scale = 0.125f;
        float *h = (float *)malloc(ntok * V * sizeof(float));
        uint32_t lab[8];
        for (int64_t i = 0; i < ntok * V; ++i)
            h[i] = c;
        for (int r = 0; r < ntok; ++r)
            lab[r] = (uint32_t)(r * 511 % V);
        float *dx = (float *)dev_alloc(ntok * V * sizeof(float));
        uint32_t *dl = (uint32_t *)dev_alloc(sizeof(lab));
        float *dloss = (float *)dev_alloc(ntok * sizeof(float));
        HIP_OK(hipMemcpy(dx, h, ntok * V * sizeof(float), hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(dl, lab, sizeof(lab), hipMemcpyHostToDevice));
        CHECK(vl_ce_fwd_bwd(dx, VL_F32, dl, dloss, NULL, ntok, V, NULL, scale, st) == VL_OK,
              "ce call");
        HIP_OK(hipStreamSynchronize(st));
        float loss[8];
        HIP_OK(hipMemcpy(loss, dloss, sizeof(loss), hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(h, dx, ntok * V * sizeof(float), hipMemcpyDeviceToHost));
        for (int r = 0; r < ntok; ++r) {
            CHECK(close_rel(loss[r], log((double)V), 1e-6, 1e-6), "CE loss row %d: %g", r,
                  loss[r]);
            for (int64_t j = 0; j < V; ++j) {
                const double want = scale * (1.0 / V - (j == lab[r] ? 1.0 : 0.0));
                if (!close_rel(h[r * V + j], want, 0, 1e-7)) {
                    CHECK(0, "CE gradient row %d col %lld: %g want %g", r, (long long)j,
                          h[r * V + j], want);
                    break;
                }
            }
        }
        HIP_OK(hipFree(dx));
        HIP_OK(hipFree(dl));
        HIP_OK(hipFree(dloss));
        free(h);
    }

    // ---- KL, uniform student and teacher: fused and over two slices
    {
        const int64_t ntok = 4, V = 32768, k = 64, half = V / 2;
        float *h = (float *)malloc(ntok * V * sizeof(float));
        uint32_t ids[4 * 64];
        float probs[4 * 64];
        for (int64_t i = 0; i < ntok * V; ++i)
            h[i] = -0.5f;
        for (int r = 0; r < ntok; ++r)
            for (int q = 0; q < k; ++q) {
                ids[r * k + q] = (uint32_t)((q * 509 + r * 17) % V);  // distinct: 509 is odd
                probs[r * k + q] = 1.0f / (float)k;                   // exact: k = 2^6
            }
        float *dx = (float *)dev_alloc(ntok * V * sizeof(float));
        uint32_t *di = (uint32_t *)dev_alloc(sizeof(ids));
        float *dp = (float *)dev_alloc(sizeof(probs));
        float *dloss = (float *)dev_alloc(ntok * sizeof(float));
        float *dlse = (float *)dev_alloc(ntok * sizeof(float));
        float *ds0 = (float *)dev_alloc(ntok * half * sizeof(float));
        float *ds1 = (float *)dev_alloc(ntok * half * sizeof(float));
        float *dparts = (float *)dev_alloc(2 * ntok * 4 * sizeof(float));
        HIP_OK(hipMemcpy(dx, h, ntok * V * sizeof(float), hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(ds0, h, ntok * half * sizeof(float), hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(ds1, h, ntok * half * sizeof(float), hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(di, ids, sizeof(ids), hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(dp, probs, sizeof(probs), hipMemcpyHostToDevice));
        const double want = log((double)V / (double)k);
        float loss[4];

        CHECK(vl_kl_fwd_bwd(dx, VL_F32, di, dp, k, dloss, NULL, ntok, V, NULL, 1.f, st) == VL_OK,
              "kl call");
        HIP_OK(hipStreamSynchronize(st));
        HIP_OK(hipMemcpy(loss, dloss, sizeof(loss), hipMemcpyDeviceToHost));
        for (int r = 0; r < ntok; ++r)
            CHECK(close_rel(loss[r], want, 1e-5, 1e-6), "KL loss row %d: %g want %g", r,
                  loss[r], want);

        CHECK(vl_kl_slice_fwd(ds0, VL_F32, half, 0, half, di, dp, k, dparts, ntok, NULL, st) ==
                  VL_OK,
              "slice fwd 0");
        CHECK(vl_kl_slice_fwd(ds1, VL_F32, half, half, half, di, dp, k, dparts + ntok * 4, ntok,
                              NULL, st) == VL_OK,
              "slice fwd 1");
        CHECK(vl_kl_slice_merge(dparts, 2, dloss, dlse, ntok, NULL, st) == VL_OK, "merge");
        CHECK(vl_kl_slice_bwd(ds0, VL_F32, half, 0, half, di, dp, k, dlse, ntok, NULL, 1.f,
                              st) == VL_OK,
              "slice bwd 0");
        HIP_OK(hipStreamSynchronize(st));
        HIP_OK(hipMemcpy(loss, dloss, sizeof(loss), hipMemcpyDeviceToHost));
        for (int r = 0; r < ntok; ++r)
            CHECK(close_rel(loss[r], want, 1e-5, 1e-6), "sliced KL loss row %d: %g want %g", r,
                  loss[r], want);
        // slice 0's gradient: 1/V everywhere, 1/V - 1/k at the teacher ids in it
        HIP_OK(hipMemcpy(h, ds0, ntok * half * sizeof(float), hipMemcpyDeviceToHost));
        for (int r = 0; r < ntok; ++r)
            for (int64_t j = 0; j < half; ++j) {
                double t = 0.0;
                for (int q = 0; q < k; ++q)
                    if (ids[r * k + q] == (uint32_t)j)
                        t = 1.0 / k;
                if (!close_rel(h[r * half + j], 1.0 / V - t, 0, 1e-6)) {
                    CHECK(0, "sliced KL gradient row %d col %lld: %g", r, (long long)j,
                          h[r * half + j]);
                    r = (int)ntok;
                    break;
                }
            }
        void *bufs[] = {dx, di, dp, dloss, dlse, ds0, ds1, dparts};
        for (unsigned i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i)
            HIP_OK(hipFree(bufs[i]));
        free(h);
    }

    // ---- top-k of a row holding a permutation of 0..V-1
    {
        const int64_t V = 5000, k = 16;
        float *h = (float *)malloc(V * sizeof(float));
        for (int64_t j = 0; j < V; ++j)
            h[j] = (float)((j * 7919) % V);  // 7919 is prime, coprime to 5000
        float *dx = (float *)dev_alloc(V * sizeof(float));
        uint32_t *di = (uint32_t *)dev_alloc(k * sizeof(uint32_t));
        float *dp = (float *)dev_alloc(k * sizeof(float));
        HIP_OK(hipMemcpy(dx, h, V * sizeof(float), hipMemcpyHostToDevice));
        CHECK(vl_topk_renorm(dx, VL_F32, 1, V, k, di, dp, st) == VL_OK, "topk call");
        HIP_OK(hipStreamSynchronize(st));
        uint32_t ids[16];
        float probs[16];
        HIP_OK(hipMemcpy(ids, di, sizeof(ids), hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(probs, dp, sizeof(probs), hipMemcpyDeviceToHost));
        double z = 0.0;
        for (int q = 0; q < k; ++q)
            z += exp(-(double)q);
        for (int q = 0; q < k; ++q) {
            CHECK(h[ids[q]] == (float)(V - 1 - q), "top-k rank %d: id %u holds %g", q, ids[q],
                  ids[q] < V ? h[ids[q]] : -1.f);
            CHECK(close_rel(probs[q], exp(-(double)q) / z, 1e-5, 1e-12), "top-k prob %d: %g", q,
                  probs[q]);
        }
        HIP_OK(hipFree(dx));
        HIP_OK(hipFree(di));
        HIP_OK(hipFree(dp));
        free(h);
    }

    // ---- slice accumulate
    {
        const int64_t n = 1000003;
        float *a = (float *)malloc(n * sizeof(float));
        float *b = (float *)malloc(n * sizeof(float));
        for (int64_t i = 0; i < n; ++i) {
            a[i] = (float)i * 0.001f - 3.f;
            b[i] = 1.0f / (float)(i + 1);
        }
        float *da = (float *)dev_alloc(n * sizeof(float));
        float *db = (float *)dev_alloc(n * sizeof(float));
        HIP_OK(hipMemcpy(da, a, n * sizeof(float), hipMemcpyHostToDevice));
        HIP_OK(hipMemcpy(db, b, n * sizeof(float), hipMemcpyHostToDevice));
        CHECK(vl_slice_acc(da, db, n, st) == VL_OK, "acc call");
        HIP_OK(hipStreamSynchronize(st));
        float *got = (float *)malloc(n * sizeof(float));
        HIP_OK(hipMemcpy(got, da, n * sizeof(float), hipMemcpyDeviceToHost));
        for (int64_t i = 0; i < n; ++i) {
            volatile float want = a[i] + b[i];  // one float32 rounding
            if (memcmp(&got[i], (const void *)&want, sizeof(float)) != 0) {
                CHECK(0, "acc element %lld: %g want %g", (long long)i, got[i], (float)want);
                break;
            }
        }
        HIP_OK(hipFree(da));
        HIP_OK(hipFree(db));
        free(a);
        free(b);
        free(got);
    }

    HIP_OK(hipStreamDestroy(st));
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("vl_c_check: all checks passed\n");
    return 0;
}
