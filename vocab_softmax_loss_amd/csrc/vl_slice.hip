// The distillation KL over a vocabulary split into slices, for gfx950
// (cortiq-engine train_head.rs: the module doc's loss and gradient, and the
// head's vocabulary cuts, each a column offset and a width).  Each slice is
// its own [ntok][width] block of logits (row stride ld), so no buffer of
// whole rows is needed.  Three calls:
//
//   part   per row of one slice, with a = the slice's max (0 if it holds no
//          finite value):  (a, z = sum_j exp(s_j - a),
//                           P = sum of p_q over the teacher ids in the slice,
//                           w = sum of p_q (ln p_q - (s_{id_q} - a)) over them)
//          -- one read of the slice.
//   merge  per row, from every slice's part:
//            lse  = M + ln sum_i z_i exp(a_i - M),  M = max of a_i with z_i > 0
//            loss = sum_i (w_i + P_i (lse - a_i))   over slices with P_i > 0
//          which is the whole row's sum_q p_q (ln p_q - s_{id_q} + lse),
//          because the slices partition the vocabulary.
//   bwd    g_j = coef (exp(s_j - lse) - p_T,j) over one slice, in place --
//          one read and one write of the slice.
//
// A slice's part is 16 bytes per row whatever its width, so the same calls
// serve a vocabulary sharded over devices: exchange the parts, merge, then
// each shard writes its own gradient.  Terms are kept anchored at the
// slice's own max (w holds p (ln p - (s - a)), with s - a <= 0), so no
// sum of large logits cancels in the merge.
//
// Layout choices follow the split cross-entropy kernels: the part pass is a
// persistent grid with one row per workgroup (a row reduction), the
// gradient pass an element-wise grid of (row, chunk) workgroups, which
// streams an in-place read + write best.  In the gradient pass every
// element has one writer: the lane that owns a teacher entry's vector
// subtracts p before its single store.
#include <math.h>

#include "vl_device.hpp"
#include "vl_launch.hpp"

namespace vl {

namespace {

__device__ __forceinline__ float scalar_f32(const float *p, int64_t i)
{
    return ((const __attribute__((address_space(4))) float *)p)[i];
}

template <int DT>
__device__ __forceinline__ char *slice_row(void *logits, int64_t row, int64_t ld)
{
    return reinterpret_cast<char *>(logits) + row * ld * (int64_t)elt_bytes<DT>();
}

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
        RowIO<DT, VEC>::store(row, v, g);
    }
}

}  // namespace

// Part pass: one row of the slice per workgroup, persistent over the rows
// in the loss range, then (a, z, P, w) = 0 for the rows outside it.
template <int DT, bool VEC, int BLOCK>
__global__ __launch_bounds__(BLOCK) void slice_part_kernel(SliceArgs a)
{
    using IO = RowIO<DT, VEC>;
    using Raw = typename IO::Raw;
    constexpr int N = IO::N, NW = BLOCK / kWave, U = VEC ? 8 : 16;
    __shared__ float sh_m[2][NW], sh_s[2][NW], sh_p[2][NW], sh_w[2][NW];
    const uint32_t tid = threadIdx.x, wid = tid / kWave;
    const int lane = lane_id();
    const uint32_t width = (uint32_t)a.width, nvec = width / (uint32_t)N;
    const RowWalk &w = a.walk;

    int par = 0;
    RowCursor c;
    c.init(blockIdx.x, gridDim.x, w.len_in);
    for (; c.j < w.n_in; c.advance(), par ^= 1) {
        const int64_t row = c.in_row(w);
        const char *p = slice_row<DT>(a.logits, row, a.ld);
        // Teacher entries of this row that fall into the slice, gathered
        // before the row is streamed: the lines they touch then sit in the
        // cache when the streaming loads reach them (gathered afterwards,
        // each cost a line fetched a second time, 11% of the slice at
        // k = 256).  The first QR * BLOCK entries wait in registers until
        // the anchor is known; any further ones are gathered afterwards.
        constexpr int QR = 4;
        float gp[QR], gs[QR];
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            const int64_t q = (int64_t)tid + (int64_t)r * BLOCK;
            gp[r] = 0.f;
            gs[r] = 0.f;
            if (q < a.k) {
                const int64_t j = (int64_t)a.ids[row * a.k + q] - a.off;
                const float pq = a.probs[row * a.k + q];
                if (j >= 0 && j < (int64_t)width && pq > 0.f) {
                    gp[r] = pq;
                    gs[r] = IO::load_elem(p, (uint32_t)j);
                }
            }
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
        // a slice with no finite value: anchor 0, z = 0 (the merge skips it)
        const float anchor = (M == -INFINITY) ? 0.f : M;

        float tp = 0.f, tw = 0.f;
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            if (gp[r] > 0.f) {
                tp += gp[r];
                tw += gp[r] * (__logf(gp[r]) - (gs[r] - anchor));
            }
        }
        for (int64_t q = (int64_t)tid + (int64_t)QR * BLOCK; q < a.k; q += BLOCK) {
            const int64_t j = (int64_t)a.ids[row * a.k + q] - a.off;
            const float pq = a.probs[row * a.k + q];
            if (j >= 0 && j < (int64_t)width && pq > 0.f) {
                tp += pq;
                tw += pq * (__logf(pq) - (IO::load_elem(p, (uint32_t)j) - anchor));
            }
        }
        tp = wave_sum(tp);
        tw = wave_sum(tw);
        if constexpr (NW > 1) {
            if (lane == 0) {
                sh_p[par][wid] = tp;
                sh_w[par][wid] = tw;
            }
            block_sync_lds();
            if (tid == 0) {
                tp = 0.f;
                tw = 0.f;
#pragma unroll
                for (int i = 0; i < NW; ++i) {
                    tp += sh_p[par][i];
                    tw += sh_w[par][i];
                }
            }
        }
        if (tid == 0) {
            const f32x4 r = {anchor, M == -INFINITY ? 0.f : S, tp, tw};
            reinterpret_cast<f32x4 *>(a.part)[row] = r;
        }
    }

    const int64_t step = (int64_t)gridDim.x * BLOCK;
    for (int64_t j = (int64_t)blockIdx.x * BLOCK + tid; j < w.n_out; j += step) {
        RowCursor o;
        o.init(j, 0, w.len_out);
        const int64_t row = o.out_row(w);
        reinterpret_cast<f32x4 *>(a.part)[row] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// Merge: one thread per row over the nslice parts ([nslice][ntok][4]).
__global__ __launch_bounds__(256) void slice_merge_kernel(const float *parts, int64_t nslice,
                                                          int64_t ntok, RowWalk walk,
                                                          float *loss, float *lse)
{
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= ntok)
        return;
    bool in = true;
    if (walk.seq_len > 0) {
        const int64_t pos = row % walk.seq_len;
        in = pos >= walk.start && pos < walk.start + walk.len_in;
    }
    if (!in) {
        loss[row] = 0.f;
        if (lse)
            lse[row] = 0.f;
        return;
    }
    const f32x4 *pp = reinterpret_cast<const f32x4 *>(parts);
    // Slices with no finite value (sum 0) are left out; a NaN sum (a NaN
    // logit) is kept, so the row's lse and loss come out NaN.
    float M = -INFINITY;
    for (int64_t i = 0; i < nslice; ++i) {
        const f32x4 r = pp[i * ntok + row];
        if (!(r[1] <= 0.f))
            M = fmaxf(M, r[0]);
    }
    float S = 0.f;
    for (int64_t i = 0; i < nslice; ++i) {
        const f32x4 r = pp[i * ntok + row];
        if (!(r[1] <= 0.f))
            S += r[1] * __expf(r[0] - M);
    }
    const float L = M + __logf(S);
    float l = 0.f;
    for (int64_t i = 0; i < nslice; ++i) {
        const f32x4 r = pp[i * ntok + row];
        if (r[2] > 0.f)
            l += r[3] + r[2] * (L - r[0]);
    }
    loss[row] = l;
    if (lse)
        lse[row] = L;
}

// Gradient pass: one (row, chunk of BLOCK * kBwdVecs vectors) per workgroup,
// over a grid of every chunk (rows in the range first, then the rows
// outside it, written as 0).  Each wave owns kBwdVecs * 64 consecutive
// 16-byte vectors, lane l the vectors 64 u + l, and needs no barrier: it
// reads the row's teacher ids itself (16 bytes per lane, so 256 ids per
// load; the waves of a workgroup share them through the caches), issued
// before its logits so both arrive in one memory latency, and finds the
// ids inside its own span with one ballot per 64 ids.  Hits are rare (about
// k * span / V per wave); each is taken in turn: its id is read across the
// wave, its p with a scalar load, and the lane owning the vector subtracts
// p before the single store.  Four vectors per lane amortise the id reads:
// at 16384 x 75968 bf16 with k = 256 this streams as fast as a gradient
// pass with no teacher at all, where one vector per lane with an LDS list
// and a barrier per workgroup ran 40% slower.
constexpr int kBwdVecs = 4;

template <int DT, bool VEC, int BLOCK>
__global__ __launch_bounds__(BLOCK) void slice_bwd_kernel(SliceArgs a, int64_t cpr)
{
    using IO = RowIO<DT, VEC>;
    constexpr int N = IO::N;
    constexpr int UV = kBwdVecs;
    const uint32_t tid = threadIdx.x;
    const int lane = lane_id();
    const uint32_t width = (uint32_t)a.width, nvec = width / (uint32_t)N;
    const RowWalk &w = a.walk;
    int64_t it = blockIdx.x;
    const int64_t n_in_items = w.n_in * cpr;
    const bool in = it < n_in_items;
    if (!in)
        it -= n_in_items;
    const int64_t jrow = it / cpr;
    const uint32_t chunk = (uint32_t)(it - jrow * cpr);
    // this wave's UV * 64 vectors start at vw; lane owns vw + u * 64 + lane
    const uint32_t vw = chunk * BLOCK * UV + (tid - (uint32_t)lane) * UV;
    RowCursor c;
    c.init(jrow, 0, in ? w.len_in : w.len_out);
    const int64_t row = in ? c.in_row(w) : c.out_row(w);
    char *p = slice_row<DT>(a.logits, row, a.ld);
    float g[UV][N];
    if (!in) {
#pragma unroll
        for (int u = 0; u < UV; ++u)
#pragma unroll
            for (int e = 0; e < N; ++e)
                g[u][e] = 0.f;
    } else {
        const float L = scalar_f32(a.lse, row);
        const uint32_t *idr = a.ids + row * a.k;
        const float *pr = a.probs + row * a.k;
        const int64_t lo = a.off + (int64_t)vw * N;
        const int64_t rest = (int64_t)width - (int64_t)vw * N;
        const int64_t hi = lo + ((int64_t)kWave * UV * N < rest ? (int64_t)kWave * UV * N : rest);
        const bool v4 = (a.k % 4 == 0) && ((uintptr_t)idr % 16 == 0);
        uint32_t id[4];
        // lane l holds teacher entries q0 + 4 l .. q0 + 4 l + 3
        auto load_ids = [&](int64_t q0) {
            if (v4) {
                const int64_t q = q0 + 4 * lane;
                if (q < a.k) {
                    const u32x4 t = *reinterpret_cast<const u32x4 *>(idr + q);
                    id[0] = t[0]; id[1] = t[1]; id[2] = t[2]; id[3] = t[3];
                } else {
                    id[0] = id[1] = id[2] = id[3] = 0xFFFFFFFFu;
                }
            } else {
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int64_t q = q0 + 4 * lane + b;
                    id[b] = q < a.k ? idr[q] : 0xFFFFFFFFu;
                }
            }
        };
        load_ids(0);
        float x[UV][N];
#pragma unroll
        for (int u = 0; u < UV; ++u) {
            const uint32_t v = vw + (uint32_t)u * kWave + (uint32_t)lane;
            IO::unpack(IO::load_stream(p, v < nvec ? v : nvec - 1), x[u]);
        }
#pragma unroll
        for (int u = 0; u < UV; ++u)
#pragma unroll
            for (int e = 0; e < N; ++e)
                g[u][e] = __expf(x[u][e] - L);
        for (int64_t q0 = 0; q0 < a.k; q0 += 4 * kWave) {
            if (q0 > 0)
                load_ids(q0);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                uint64_t mask = ballot((int64_t)id[b] >= lo && (int64_t)id[b] < hi);
                while (mask) {
                    const int src = __builtin_ctzll(mask);
                    mask &= mask - 1;
                    const uint32_t jj =
                        (uint32_t)((int64_t)__builtin_amdgcn_readlane((int)id[b], src) - lo);
                    const float pv = scalar_f32(pr, q0 + 4 * src + b);
                    const uint32_t jv = jj / N;
#pragma unroll
                    for (int u = 0; u < UV; ++u) {
                        if (jv == (uint32_t)(u * kWave + lane)) {
#pragma unroll
                            for (int e = 0; e < N; ++e)
                                g[u][e] -= (jj % N == (uint32_t)e) ? pv : 0.f;
                        }
                    }
                }
            }
        }
        const float sc = a.coef;
#pragma unroll
        for (int u = 0; u < UV; ++u)
#pragma unroll
            for (int e = 0; e < N; ++e)
                g[u][e] *= sc;
    }
#pragma unroll
    for (int u = 0; u < UV; ++u) {
        const uint32_t v = vw + (uint32_t)u * kWave + (uint32_t)lane;
        if (v < nvec)
            store_stream<DT, VEC>(p, v, g[u]);
    }
}

namespace {

template <int DT, bool VEC>
hipError_t launch_slice_t(bool part, const SliceArgs &a, hipStream_t st)
{
    const int64_t nvec = a.width / RowIO<DT, VEC>::N;
    if (part) {
        const int block = nvec <= 512 ? 64 : 256;
        const void *fn = block == 64 ? (const void *)slice_part_kernel<DT, VEC, 64>
                                     : (const void *)slice_part_kernel<DT, VEC, 256>;
        const int per_cu = blocks_per_cu(fn, block, 0);
        const int64_t rows = a.walk.n_in > a.walk.n_out ? a.walk.n_in : a.walk.n_out;
        int64_t grid = (int64_t)per_cu * device_cus();
        if (grid > rows)
            grid = rows;
        if (grid < 1)
            grid = 1;
        if (block == 64)
            hipLaunchKernelGGL((slice_part_kernel<DT, VEC, 64>), dim3((unsigned)grid), dim3(64),
                               0, st, a);
        else
            hipLaunchKernelGGL((slice_part_kernel<DT, VEC, 256>), dim3((unsigned)grid),
                               dim3(256), 0, st, a);
        return hipGetLastError();
    }
    // chunks of 256 vectors up to 1024 vectors per row, 2048 above
    const int block = nvec <= 1024 ? 64 : 512;
    const int64_t cpr = (nvec + (int64_t)block * kBwdVecs - 1) / ((int64_t)block * kBwdVecs);
    const int64_t grid = (a.walk.n_in + a.walk.n_out) * cpr;
    if (grid > INT32_MAX)
        return hipErrorInvalidConfiguration;
    if (block == 64)
        hipLaunchKernelGGL((slice_bwd_kernel<DT, VEC, 64>), dim3((unsigned)grid), dim3(64), 0, st,
                           a, cpr);
    else
        hipLaunchKernelGGL((slice_bwd_kernel<DT, VEC, 512>), dim3((unsigned)grid), dim3(512), 0,
                           st, a, cpr);
    return hipGetLastError();
}

hipError_t launch_slice_dt(int dtype, bool part, const SliceArgs &a, hipStream_t st)
{
    const int64_t elt = dtype == kF32 ? 4 : 2;
    const bool vec = ((uintptr_t)a.logits % 16 == 0) && ((a.ld * elt) % 16 == 0) &&
                     ((a.width * elt) % 16 == 0);
    if (dtype == kF32)
        return vec ? launch_slice_t<kF32, true>(part, a, st)
                   : launch_slice_t<kF32, false>(part, a, st);
    return vec ? launch_slice_t<kBF16, true>(part, a, st)
               : launch_slice_t<kBF16, false>(part, a, st);
}

}  // namespace

hipError_t launch_slice_part(int dtype, const SliceArgs &a, hipStream_t st)
{
    return launch_slice_dt(dtype, true, a, st);
}

hipError_t launch_slice_bwd(int dtype, const SliceArgs &a, hipStream_t st)
{
    return launch_slice_dt(dtype, false, a, st);
}

hipError_t launch_slice_merge(const float *parts, int64_t nslice, int64_t ntok,
                              const RowWalk &walk, float *loss, float *lse, hipStream_t st)
{
    const int64_t grid = (ntok + 255) / 256;
    if (grid > INT32_MAX)
        return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(slice_merge_kernel, dim3((unsigned)grid), dim3(256), 0, st, parts, nslice,
                       ntok, walk, loss, lse);
    return hipGetLastError();
}

}  // namespace vl
