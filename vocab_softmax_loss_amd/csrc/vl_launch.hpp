// Internal interface between the C ABI (vl_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vl {

// One call of the fused CE or KL row kernel.
struct RowArgs {
    void *logits;             // [ntok][V] float32 or bf16, in: logits, out: gradient
    const uint32_t *labels;   // CE: [ntok]
    const uint32_t *ids;      // KL: [ntok][k]
    const float *probs;       // KL: [ntok][k]
    float *loss;              // [ntok]
    float *lse;               // [ntok] or null
    int64_t ntok, V, k;
    int64_t seq_len, start, end;  // loss range; seq_len <= 0: every row
    float coef;               // gradient scale
};

struct TopkArgs {
    const void *logits;  // [ntok][V]
    int64_t ntok, V, k;
    uint32_t *ids;       // [ntok][k]
    float *probs;        // [ntok][k]
};

// Each returns hipSuccess or the HIP error of the launch.
hipError_t launch_rows(int dtype, bool kl, const RowArgs &a, hipStream_t stream);
hipError_t launch_topk(int dtype, const TopkArgs &a, hipStream_t stream);
hipError_t launch_slice_acc(float *dst, const float *src, int64_t n, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cus();

// Largest KL vocabulary: two row bitmaps of V bits must fit in LDS.
constexpr int64_t kMaxKlVocab = int64_t(1) << 19;
// Largest top-k k.
constexpr int64_t kMaxTopk = 2048;

}  // namespace vl
