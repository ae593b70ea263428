// Fused row-wise vocabulary-softmax loss for gfx950: cross-entropy against a
// label, or distillation KL against a teacher's top-k distribution, with the
// scaled logits gradient written over the logits.
//
// Per row s[0..V) (cortiq-engine train_head.rs, module doc and kl_rows;
// aprender-train wgpu_cross_entropy.rs, module doc and backward):
//   lse  = max(s) + ln sum_j exp(s_j - max(s))
//   CE:  loss = lse - s_label,                    g_j = coef (p_j - [j = label])
//   KL:  loss = sum_{p_q > 0} p_q (ln p_q - s_{id_q} + lse),
//                                                  g_j = coef (p_j - t_j)
// with p_j = exp(s_j - lse) and t_j the teacher probability of id j (0 off
// the top-k).  Rows outside the loss range (start <= r mod seq_len < end)
// are not read: their loss and lse are 0 and their gradient row is zeroed.
//
// One workgroup owns a row at a time (persistent grid, rows strided by the
// grid size).  Two variants:
//  * staged (NV > 0): the row is held in registers, NV 16-byte vectors per
//    thread, so it is read from HBM once and written once (1R + 1W).  Each
//    thread keeps e = exp(s - m_thread) and rescales by exp(m_thread - lse),
//    one exp per element.
//  * online (NV == 0): the row is streamed twice: pass 1 keeps a running
//    (max, sum) per thread with one rescale per chunk, pass 2 writes the
//    gradient (2R + 1W).
// (max, sum) pairs reduce across the wave with DPP and across waves through
// LDS, one barrier per row.
//
// Targets.  CE: the thread that owns the label's vector subtracts coef from
// that element before its store.  KL: the teacher ids of the row are marked
// in an LDS bitmap of V bits; the main store skips marked elements, and the
// thread that handles id q writes coef (p_id - p_q) there itself, so every
// element has exactly one writer (no read-modify-write of the gradient).
// Bitmaps alternate between two LDS buffers by row parity so that clearing
// one row's marks never races with marking the next row.
//
// Precondition violations are not checked on the device but never fault: a
// label or id >= V gives a NaN loss and no target write; duplicate ids give
// an undefined gradient at that id.
#include <math.h>

#include "vl_device.hpp"
#include "vl_launch.hpp"

namespace vl {

__device__ __forceinline__ bool row_in_loss(int64_t r, const RowArgs &a)
{
    if (a.seq_len <= 0)
        return true;
    int64_t p = r % a.seq_len;
    return a.start <= p && p < a.end;
}

// Vectors per thread per chunk of the online variant: 16 values in flight.
template <int N>
constexpr int online_unroll()
{
    return N >= 16 ? 1 : 16 / N;
}

template <int DT, bool KL, int BLOCK, int NV, bool VEC>
__global__ __launch_bounds__(BLOCK) void row_loss_kernel(RowArgs a)
{
    using IO = RowIO<DT, VEC>;
    constexpr int N = IO::N;
    constexpr int NW = BLOCK / kWave;
    constexpr int U = online_unroll<N>();

    __shared__ float sh_m[2][NW];
    __shared__ float sh_s[2][NW];
    __shared__ float sh_l[2][NW];
    extern __shared__ uint32_t bitmaps[];  // KL: 2 x words

    const int tid = threadIdx.x;
    const int wid = tid / kWave;
    const int lane = lane_id();
    const int64_t V = a.V;
    const int64_t nvec = V / N;
    const int words = (int)((V + 31) >> 5);
    const float coef = a.coef;

    if constexpr (KL) {
        for (int i = tid; i < 2 * words; i += BLOCK)
            bitmaps[i] = 0u;
        __syncthreads();
    }

    int par = 0;
    for (int64_t row = blockIdx.x; row < a.ntok; row += gridDim.x) {
        char *rowp = reinterpret_cast<char *>(a.logits) + row * V * (int64_t)elt_bytes<DT>();

        if (!row_in_loss(row, a)) {
            float z[N];
#pragma unroll
            for (int c = 0; c < N; ++c)
                z[c] = 0.f;
            for (int64_t v = tid; v < nvec; v += BLOCK)
                IO::store(rowp, v, z);
            if (tid == 0) {
                a.loss[row] = 0.f;
                if (a.lse)
                    a.lse[row] = 0.f;
            }
            continue;
        }

        uint32_t *bm = bitmaps + par * words;
        uint32_t *bm_prev = bitmaps + (par ^ 1) * words;

        // ---- targets: label, or this thread's first teacher entry
        uint32_t label = 0;
        float s_tgt = 0.f, p_tgt = 0.f;
        uint32_t id_tgt = 0xFFFFFFFFu;
        if constexpr (!KL) {
            label = a.labels[row];
            if (tid == 0 && label < (uint32_t)V)
                s_tgt = IO::load_elem(rowp, label);
        } else {
            const uint32_t *rid = a.ids + row * a.k;
            for (int64_t q = tid; q < a.k; q += BLOCK) {
                uint32_t id = rid[q];
                if (id < (uint32_t)V)
                    atomicOr(&bm[id >> 5], 1u << (id & 31));
                if (q == tid) {
                    id_tgt = id;
                    p_tgt = a.probs[row * a.k + q];
                    if (id < (uint32_t)V)
                        s_tgt = IO::load_elem(rowp, id);
                }
            }
        }

        // ---- pass 1: thread-local (max, sum of exp)
        float m = -INFINITY, s = 0.f;
        float x[NV > 0 ? NV : 1][N];
        if constexpr (NV > 0) {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                int64_t v = tid + (int64_t)i * BLOCK;
                if (v < nvec) {
                    IO::load(rowp, v, x[i]);
                } else {
#pragma unroll
                    for (int c = 0; c < N; ++c)
                        x[i][c] = -INFINITY;
                }
            }
#pragma unroll
            for (int i = 0; i < NV; ++i)
#pragma unroll
                for (int c = 0; c < N; ++c)
                    m = fmaxf(m, x[i][c]);
            const float ms = (m == -INFINITY) ? 0.f : m;
#pragma unroll
            for (int i = 0; i < NV; ++i)
#pragma unroll
                for (int c = 0; c < N; ++c) {
                    float e = __expf(x[i][c] - ms);
                    x[i][c] = e;
                    s += e;
                }
        } else {
            for (int64_t v0 = tid; v0 < nvec; v0 += (int64_t)BLOCK * U) {
                float y[U][N];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    int64_t v = v0 + (int64_t)u * BLOCK;
                    if (v < nvec) {
                        IO::load(rowp, v, y[u]);
                    } else {
#pragma unroll
                        for (int c = 0; c < N; ++c)
                            y[u][c] = -INFINITY;
                    }
                }
                float cm = -INFINITY;
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int c = 0; c < N; ++c)
                        cm = fmaxf(cm, y[u][c]);
                const float mn = fmaxf(m, cm);
                if (mn != -INFINITY) {
                    float acc = s * __expf(m - mn);
#pragma unroll
                    for (int u = 0; u < U; ++u)
#pragma unroll
                        for (int c = 0; c < N; ++c)
                            acc += __expf(y[u][c] - mn);
                    s = acc;
                    m = mn;
                }
            }
        }

        // ---- block reduction of (max, sum): one barrier
        {
            const float wm = wave_max(m);
            const float sc = (m == -INFINITY) ? 0.f : s * __expf(m - wm);
            const float ws = wave_sum(sc);
            if (lane == 0) {
                sh_m[par][wid] = wm;
                sh_s[par][wid] = ws;
            }
        }
        __syncthreads();
        float M = -INFINITY;
#pragma unroll
        for (int i = 0; i < NW; ++i)
            M = fmaxf(M, sh_m[par][i]);
        float S = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const float mi = sh_m[par][i];
            S += (mi == -INFINITY) ? 0.f : sh_s[par][i] * __expf(mi - M);
        }
        const float logS = __logf(S);
        const float lse = M + logS;

        // ---- loss (and, for KL, the gradient at the teacher ids)
        if constexpr (!KL) {
            if (tid == 0) {
                a.loss[row] = (label < (uint32_t)V) ? (M - s_tgt) + logS : NAN;
                if (a.lse)
                    a.lse[row] = lse;
            }
        } else {
            // The previous row's marks: every thread is past that row's stores.
            for (int i = tid; i < words; i += BLOCK)
                bm_prev[i] = 0u;
            const uint32_t *rid = a.ids + row * a.k;
            const float *rp = a.probs + row * a.k;
            float acc = 0.f;
            for (int64_t q = tid; q < a.k; q += BLOCK) {
                uint32_t id;
                float p, sv = 0.f;
                if (q == tid) {
                    id = id_tgt;
                    p = p_tgt;
                    sv = s_tgt;
                } else {
                    id = rid[q];
                    p = rp[q];
                    if (id < (uint32_t)V)
                        sv = IO::load_elem(rowp, id);
                }
                if (id >= (uint32_t)V) {
                    acc = NAN;
                    continue;
                }
                const float d = (sv - M) - logS;  // log p_S at the id
                if (p > 0.f)
                    acc += p * (__logf(p) - d);
                IO::store_elem(rowp, id, coef * (__expf(d) - p));
            }
            const float wl = wave_sum(acc);
            if (lane == 0)
                sh_l[par][wid] = wl;
            __syncthreads();
            if (tid == 0) {
                float tot = 0.f;
#pragma unroll
                for (int i = 0; i < NW; ++i)
                    tot += sh_l[par][i];
                a.loss[row] = tot;
                if (a.lse)
                    a.lse[row] = lse;
            }
        }

        // ---- gradient store
        auto finish = [&](int64_t v, float (&g)[N]) {
            if constexpr (!KL) {
                if (label < (uint32_t)V && v == (int64_t)(label / N))
                    g[label % N] -= coef;
                IO::store(rowp, v, g);
            } else {
                const int64_t j0 = v * N;
                const uint32_t bits =
                    (bm[j0 >> 5] >> (j0 & 31)) & (uint32_t)((1ull << N) - 1);
                if (bits == 0u) {
                    IO::store(rowp, v, g);
                } else {
#pragma unroll
                    for (int c = 0; c < N; ++c)
                        if (!((bits >> c) & 1u))
                            IO::store_elem(rowp, j0 + c, g[c]);
                }
            }
        };

        if constexpr (NV > 0) {
            const float ms = (m == -INFINITY) ? 0.f : m;
            const float cf = coef * __expf(ms - lse);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                int64_t v = tid + (int64_t)i * BLOCK;
                if (v < nvec) {
                    float g[N];
#pragma unroll
                    for (int c = 0; c < N; ++c)
                        g[c] = x[i][c] * cf;
                    finish(v, g);
                }
            }
        } else {
            for (int64_t v0 = tid; v0 < nvec; v0 += (int64_t)BLOCK * U) {
                float y[U][N];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    int64_t v = v0 + (int64_t)u * BLOCK;
                    if (v < nvec)
                        IO::load(rowp, v, y[u]);
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    int64_t v = v0 + (int64_t)u * BLOCK;
                    if (v < nvec) {
                        float g[N];
#pragma unroll
                        for (int c = 0; c < N; ++c)
                            g[c] = coef * __expf(y[u][c] - lse);
                        finish(v, g);
                    }
                }
            }
        }
        par ^= 1;
    }
}

// ------------------------------------------------------------------ launch

namespace {

struct OccKey {
    const void *fn;
    size_t lds;
    int dev;
};

int cached_blocks_per_cu(const void *fn, int block, size_t lds)
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

template <int DT, bool KL, int BLOCK, int NV, bool VEC>
hipError_t launch_one(const RowArgs &a, hipStream_t st)
{
    auto fn = row_loss_kernel<DT, KL, BLOCK, NV, VEC>;
    size_t lds = 0;
    if (KL) {
        lds = 2 * (size_t)((a.V + 31) >> 5) * sizeof(uint32_t);
        if (lds > 65536) {
            hipError_t e = hipFuncSetAttribute((const void *)fn,
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)lds);
            if (e != hipSuccess)
                return e;
        }
    }
    const int per_cu = cached_blocks_per_cu((const void *)fn, BLOCK, lds);
    int64_t grid = (int64_t)per_cu * device_cus();
    if (grid > a.ntok)
        grid = a.ntok;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(BLOCK), lds, st, a);
    return hipGetLastError();
}

// Staged variants: BLOCK threads x NV vectors cover the row.
template <int DT, bool KL>
hipError_t launch_staged_or_online(const RowArgs &a, hipStream_t st, bool vec)
{
    constexpr int N = RowIO<DT, true>::N;
    if (!vec)
        return launch_one<DT, KL, 256, 0, false>(a, st);
    const int64_t nvec = a.V / N;
    if (nvec <= 64)
        return launch_one<DT, KL, 64, 1, true>(a, st);
    if (nvec <= 128)
        return launch_one<DT, KL, 64, 2, true>(a, st);
    if (nvec <= 256)
        return launch_one<DT, KL, 64, 4, true>(a, st);
    if (nvec <= 512)
        return launch_one<DT, KL, 64, 8, true>(a, st);
    if (nvec <= 1024)
        return launch_one<DT, KL, 256, 4, true>(a, st);
    if (nvec <= 2048)
        return launch_one<DT, KL, 256, 8, true>(a, st);
    if (nvec <= 4096)
        return launch_one<DT, KL, 1024, 4, true>(a, st);
    if (nvec <= 8192)
        return launch_one<DT, KL, 1024, 8, true>(a, st);
    return launch_one<DT, KL, 512, 0, true>(a, st);
}

}  // namespace

hipError_t launch_rows(int dtype, bool kl, const RowArgs &a, hipStream_t st)
{
    const size_t elt = dtype == kF32 ? 4 : 2;
    const int n = 16 / (int)elt;
    const bool vec = ((uintptr_t)a.logits % 16 == 0) && (a.V % n == 0);
    if (dtype == kF32)
        return kl ? launch_staged_or_online<kF32, true>(a, st, vec)
                  : launch_staged_or_online<kF32, false>(a, st, vec);
    return kl ? launch_staged_or_online<kBF16, true>(a, st, vec)
              : launch_staged_or_online<kBF16, false>(a, st, vec);
}

}  // namespace vl
