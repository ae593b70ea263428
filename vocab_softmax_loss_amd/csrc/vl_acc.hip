// Slice accumulate for gfx950 (cortiq-engine train_head.rs, acc_add and the
// slice loop of head_kl): dst[i] += src[i] for i < n, the float32 sum with
// round-to-nearest-even, one add per element.  The input gradient of a later
// vocabulary slice is added into the first slice's.
//
// 2 reads + 1 write per element: 16-byte vectors over the aligned body with
// a grid-stride loop, one element at a time otherwise.
#include "vl_device.hpp"
#include "vl_launch.hpp"

namespace vl {

constexpr int kAccBlock = 256;

__global__ __launch_bounds__(kAccBlock) void slice_acc_vec_kernel(f32x4 *dst, const f32x4 *src,
                                                                  int64_t n4)
{
    const int64_t stride = (int64_t)gridDim.x * kAccBlock;
    for (int64_t i = (int64_t)blockIdx.x * kAccBlock + threadIdx.x; i < n4; i += stride) {
        f32x4 a = dst[i];
        const f32x4 b = src[i];
        a[0] += b[0];
        a[1] += b[1];
        a[2] += b[2];
        a[3] += b[3];
        __builtin_nontemporal_store(a, dst + i);  // written once: keep it out of the caches
    }
}

__global__ __launch_bounds__(kAccBlock) void slice_acc_elem_kernel(float *dst, const float *src,
                                                                   int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * kAccBlock;
    for (int64_t i = (int64_t)blockIdx.x * kAccBlock + threadIdx.x; i < n; i += stride)
        dst[i] += src[i];
}

hipError_t launch_slice_acc(float *dst, const float *src, int64_t n, hipStream_t st)
{
    const int64_t max_grid = (int64_t)device_cus() * 16;
    const bool vec = ((uintptr_t)dst % 16 == 0) && ((uintptr_t)src % 16 == 0);
    int64_t body = 0;
    if (vec) {
        const int64_t n4 = n / 4;
        body = n4 * 4;
        if (n4 > 0) {
            int64_t grid = (n4 + kAccBlock - 1) / kAccBlock;
            if (grid > max_grid)
                grid = max_grid;
            hipLaunchKernelGGL(slice_acc_vec_kernel, dim3((unsigned)grid), dim3(kAccBlock), 0, st,
                               reinterpret_cast<f32x4 *>(dst),
                               reinterpret_cast<const f32x4 *>(src), n4);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
    }
    const int64_t rest = n - body;
    if (rest > 0) {
        int64_t grid = (rest + kAccBlock - 1) / kAccBlock;
        if (grid > max_grid)
            grid = max_grid;
        hipLaunchKernelGGL(slice_acc_elem_kernel, dim3((unsigned)grid), dim3(kAccBlock), 0, st,
                           dst + body, src + body, rest);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace vl
