// Cross-entropy as two separate passes plus the mean loss, for gfx950
// (aprender-train wgpu_cross_entropy.rs: forward_async stores the per-row
// loss and logsumexp, backward rebuilds the softmax from the saved
// logsumexp and writes the scaled gradient over the logits, read_loss takes
// the mean over the loss range):
//   forward   lse_r = max(s) + ln sum_j exp(s_j - max(s)),
//             loss_r = lse_r - s_r[label]                  1 read of the row
//   backward  g_rj = scale (exp(s_rj - lse_r) - [j = label])  1 read + 1 write
//   mean      sum_r loss_r / (rows in the range), 0 for an empty range
// Rows outside the loss range (start <= r mod seq_len < end) are never read:
// the forward writes their loss and lse as 0, the backward zeroes their
// gradient row.
//
// Forward: a persistent grid walks the rows in the range first and the rows
// outside it second, each list strided by the grid, one row per workgroup
// at a time.  Each thread streams 16-byte vectors v = tid + u * BLOCK, U of
// them in flight (non-temporal: the logits exceed every cache), keeps a
// running (max, sum) with one rescale per U vectors, then the block reduces
// with DPP and one LDS barrier per row (slots alternate by row parity, so a
// fast wave never overwrites partials a slow wave still reads).
//
// Backward: element-wise, so it is laid out for the read-then-write stream
// alone: one vector per thread, one chunk of a row per workgroup, and a
// grid of every chunk in row order.  The workgroups in flight then cover a
// narrow window of consecutive addresses, each reads and soon rewrites its
// own vectors, and every wave has one load outstanding.  On MI355X this
// runs an in-place read + write at 6.3 TB/s on 4 GB, where a persistent
// grid of row-owning workgroups with 8 loads per thread in flight reaches
// 5.1 TB/s.  The label and lse of the row are scalar loads; the thread that
// owns the label's vector subtracts the scale there before its store.
//
// Precondition violations never fault: a label >= V gives a NaN loss and a
// gradient without the one-hot term.
#include <math.h>

#include "vl_device.hpp"
#include "vl_launch.hpp"

namespace vl {

namespace {

// Uniform, read-only scalars through the scalar cache.
__device__ __forceinline__ uint32_t scalar_u32(const uint32_t *p, int64_t i)
{
    return ((const __attribute__((address_space(4))) uint32_t *)p)[i];
}
__device__ __forceinline__ float scalar_f32(const float *p, int64_t i)
{
    return ((const __attribute__((address_space(4))) float *)p)[i];
}

template <int DT>
__device__ __forceinline__ char *row_base(void *logits, int64_t row, uint32_t V)
{
    return reinterpret_cast<char *>(logits) + row * (int64_t)V * (int64_t)elt_bytes<DT>();
}

// A gradient store that nothing reads back soon: non-temporal for 16-byte
// vectors of either type.
template <int DT, bool VEC>
__device__ __forceinline__ void store_stream(void *row, uint32_t v,
                                             const float (&g)[RowIO<DT, VEC>::N])
{
    if constexpr (DT == kBF16 && VEC) {
        f32x8 f = {g[0], g[1], g[2], g[3], g[4], g[5], g[6], g[7]};
        const bf16x8 b = __builtin_convertvector(f, bf16x8);
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, b),
                                    reinterpret_cast<u32x4 *>(row) + v);
    } else {
        RowIO<DT, VEC>::store(row, v, g);  // float32 vectors: non-temporal already
    }
}

// Forward: vectors in flight per thread, 8 x 16 bytes or 16 single elements.
template <bool VEC>
constexpr int split_unroll()
{
    return VEC ? 8 : 16;
}

}  // namespace

template <int DT, bool VEC, int BLOCK>
__global__ __launch_bounds__(BLOCK) void ce_fwd_kernel(RowArgs a)
{
    using IO = RowIO<DT, VEC>;
    using Raw = typename IO::Raw;
    constexpr int N = IO::N, NW = BLOCK / kWave, U = split_unroll<VEC>();
    __shared__ float sh_m[2][NW];
    __shared__ float sh_s[2][NW];
    const uint32_t tid = threadIdx.x, wid = tid / kWave;
    const int lane = lane_id();
    const uint32_t V = (uint32_t)a.V, nvec = V / (uint32_t)N;
    const RowWalk &w = a.walk;

    int par = 0;
    RowCursor c;
    c.init(blockIdx.x, gridDim.x, w.len_in);
    for (; c.j < w.n_in; c.advance(), par ^= 1) {
        const int64_t row = c.in_row(w);
        const char *p = row_base<DT>(a.logits, row, V);
        uint32_t label = 0;
        float sl = 0.f;
        if (tid == 0) {
            label = a.labels[row];
            if (label < V)
                sl = IO::load_elem(p, label);
        }
        float m = -INFINITY, s = 0.f;
        for (uint32_t v0 = tid; v0 < nvec; v0 += (uint32_t)BLOCK * U) {
            Raw y[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t v = v0 + (uint32_t)u * BLOCK;
                y[u] = IO::load_stream(p, v < nvec ? v : nvec - 1);
            }
            float x[U][N];
            float cm = -INFINITY;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                IO::unpack(y[u], x[u]);
                const bool in = v0 + (uint32_t)u * BLOCK < nvec;
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    x[u][e] = in ? x[u][e] : -INFINITY;
                    cm = fmaxf(cm, x[u][e]);
                }
            }
            const float mn = fmaxf(m, cm);
            if (mn != -INFINITY) {
                float acc = s * __expf(m - mn);
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int e = 0; e < N; ++e)
                        acc += __expf(x[u][e] - mn);
                s = acc;
                m = mn;
            }
        }

        const float wm = wave_max(m);
        const float ws = wave_sum((m == -INFINITY) ? 0.f : s * __expf(m - wm));
        float M = wm, S = ws;
        if constexpr (NW > 1) {
            if (lane == 0) {
                sh_m[par][wid] = wm;
                sh_s[par][wid] = ws;
            }
            block_sync_lds();
            M = -INFINITY;
#pragma unroll
            for (int i = 0; i < NW; ++i)
                M = fmaxf(M, sh_m[par][i]);
            S = 0.f;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const float mi = sh_m[par][i];
                S += (mi == -INFINITY) ? 0.f : sh_s[par][i] * __expf(mi - M);
            }
        }
        if (tid == 0) {
            const float logS = __logf(S);
            a.loss[row] = (label < V) ? (M - sl) + logS : NAN;
            if (a.lse)
                a.lse[row] = M + logS;
        }
    }

    // Rows outside the range: loss and lse 0, one row per thread.
    const int64_t step = (int64_t)gridDim.x * BLOCK;
    for (int64_t j = (int64_t)blockIdx.x * BLOCK + tid; j < w.n_out; j += step) {
        RowCursor o;
        o.init(j, 0, w.len_out);
        const int64_t row = o.out_row(w);
        a.loss[row] = 0.f;
        if (a.lse)
            a.lse[row] = 0.f;
    }
}

// Backward: one 16-byte vector per thread and one (row, chunk of BLOCK
// vectors) per workgroup, over a grid that covers every chunk once: the
// rows in the range first, then the rows outside it (written as 0).
template <int DT, bool VEC, int BLOCK>
__global__ __launch_bounds__(BLOCK) void ce_bwd_kernel(RowArgs a, int64_t cpr)
{
    using IO = RowIO<DT, VEC>;
    constexpr int N = IO::N;
    const uint32_t V = (uint32_t)a.V, nvec = V / (uint32_t)N;
    const RowWalk &w = a.walk;
    int64_t it = blockIdx.x;
    const int64_t n_in_items = w.n_in * cpr;
    const bool in = it < n_in_items;
    if (!in)
        it -= n_in_items;
    const int64_t j = it / cpr;
    const uint32_t v = (uint32_t)(it - j * cpr) * BLOCK + threadIdx.x;
    RowCursor c;
    c.init(j, 0, in ? w.len_in : w.len_out);
    const int64_t row = in ? c.in_row(w) : c.out_row(w);
    char *p = row_base<DT>(a.logits, row, V);
    float g[N];
    if (!in) {
#pragma unroll
        for (int e = 0; e < N; ++e)
            g[e] = 0.f;
    } else {
        const uint32_t label = scalar_u32(a.labels, row);
        const float L = scalar_f32(a.lse, row);
        const float sc = a.coef;
        float x[N];
        IO::unpack(IO::load_stream(p, v < nvec ? v : nvec - 1), x);
#pragma unroll
        for (int e = 0; e < N; ++e)
            g[e] = sc * __expf(x[e] - L);
        if (label < V && v == label / (uint32_t)N)
            g[label % (uint32_t)N] -= sc;
    }
    if (v < nvec)
        store_stream<DT, VEC>(p, v, g);
}

// Sum of loss[0..n) in float64, in a fixed order (the result does not depend
// on timing), divided by count and rounded once to float32.
constexpr int kMeanBlock = 1024;

__global__ __launch_bounds__(kMeanBlock) void loss_mean_kernel(const float *loss, int64_t n,
                                                               int64_t count, float *mean)
{
    __shared__ double sh[kMeanBlock / kWave];
    const int tid = threadIdx.x;
    double s = 0.0;
    for (int64_t i = tid; i < n; i += kMeanBlock)
        s += (double)loss[i];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        s += __shfl_xor(s, off);
    if (lane_id() == 0)
        sh[tid / kWave] = s;
    __syncthreads();
    if (tid == 0) {
        double t = 0.0;
#pragma unroll
        for (int i = 0; i < kMeanBlock / kWave; ++i)
            t += sh[i];
        mean[0] = count > 0 ? (float)(t / (double)count) : 0.f;
    }
}

namespace {

template <typename K>
hipError_t launch_persistent(K fn, int block, const RowArgs &a, hipStream_t st)
{
    const int per_cu = blocks_per_cu((const void *)fn, block, 0);
    const int64_t rows = a.walk.n_in > a.walk.n_out ? a.walk.n_in : a.walk.n_out;
    int64_t grid = (int64_t)per_cu * device_cus();
    if (grid > rows)
        grid = rows;
    if (grid < 1)
        grid = 1;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(block), 0, st, a);
    return hipGetLastError();
}

// Forward: one wave per row for short rows, four otherwise.  Backward:
// 512-vector chunks for rows of more than 256 vectors, 64 otherwise.
template <int DT, bool VEC>
hipError_t launch_split(bool fwd, const RowArgs &a, hipStream_t st)
{
    const int64_t nvec = a.V / RowIO<DT, VEC>::N;
    if (fwd) {
        if (nvec <= 512)
            return launch_persistent(ce_fwd_kernel<DT, VEC, 64>, 64, a, st);
        return launch_persistent(ce_fwd_kernel<DT, VEC, 256>, 256, a, st);
    }
    const int block = nvec <= 256 ? 64 : 512;
    const int64_t cpr = (nvec + block - 1) / block;
    const int64_t grid = (a.walk.n_in + a.walk.n_out) * cpr;
    if (grid > INT32_MAX)
        return hipErrorInvalidConfiguration;
    if (block == 64)
        hipLaunchKernelGGL((ce_bwd_kernel<DT, VEC, 64>), dim3((unsigned)grid), dim3(64), 0, st, a,
                           cpr);
    else
        hipLaunchKernelGGL((ce_bwd_kernel<DT, VEC, 512>), dim3((unsigned)grid), dim3(512), 0, st,
                           a, cpr);
    return hipGetLastError();
}

hipError_t launch_split_dt(int dtype, bool fwd, const RowArgs &a, hipStream_t st)
{
    const size_t elt = dtype == kF32 ? 4 : 2;
    const bool vec = ((uintptr_t)a.logits % 16 == 0) && (a.V % (int64_t)(16 / elt) == 0);
    if (dtype == kF32)
        return vec ? launch_split<kF32, true>(fwd, a, st) : launch_split<kF32, false>(fwd, a, st);
    return vec ? launch_split<kBF16, true>(fwd, a, st) : launch_split<kBF16, false>(fwd, a, st);
}

}  // namespace

hipError_t launch_ce_fwd(int dtype, const RowArgs &a, hipStream_t st)
{
    return launch_split_dt(dtype, true, a, st);
}

hipError_t launch_ce_bwd(int dtype, const RowArgs &a, hipStream_t st)
{
    return launch_split_dt(dtype, false, a, st);
}

hipError_t launch_loss_mean(const float *loss, int64_t n, int64_t count, float *mean,
                            hipStream_t st)
{
    hipLaunchKernelGGL(loss_mean_kernel, dim3(1), dim3(kMeanBlock), 0, st, loss, n, count, mean);
    return hipGetLastError();
}

}  // namespace vl
