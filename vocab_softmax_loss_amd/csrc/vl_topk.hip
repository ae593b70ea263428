// Teacher top-k with renormalised probabilities for gfx950
// (cortiq-engine train_head.rs, topk_rows): per row, the k entries that come
// first in the order (value descending, id ascending), and
//   probs_q = exp(v_q - v_0) / sum_{q' < k} exp(v_q' - v_0).
// -0 and +0 tie (the lower id wins).  NaN is a precondition violation.
//
// The page's kernel keeps a best-8 list per thread and sorts 2048
// candidates; that is exact only while no thread sees more than 8 of the
// true top-k.  This kernel is exact for every input:
//
// One wave owns a row and streams it once, in tiles of 64 lanes x U
// 16-byte vectors; a tile's ids are all larger than every earlier tile's.
// Values pass an acceptance test into a per-wave LDS candidate buffer of
// (key, id) pairs, written in id order.  The key is the order-preserving
// unsigned image of the float (sign-flipped, -0 folded onto +0), so key
// order is value order.  Until the buffer first fills every value is
// accepted; when a sub-tile might overflow it, the buffer is compacted to
// its own top-k by an exact radix select on the keys (8-bit digits, LDS
// histogram, 4 passes for float32, 2 for bf16 whose low key half follows
// from the sign), keeping ties at the k-th key in buffer (= id) order.  The
// k-th key becomes the threshold: later elements have larger ids, so only
// values strictly above it can enter the top-k, and a quick per-vector max
// test skips almost every sub-tile.
//
// At the end the buffer is selected once more to exactly k winners, each
// winner's output position is its rank (number of winners with a larger
// key, plus equal keys at lower ids), and probabilities are formed from the
// winners' values.
#include <math.h>

#include "vl_device.hpp"
#include "vl_launch.hpp"

namespace vl {

__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k)
{
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __builtin_bit_cast(float, u);
}

// Exact select among keys[0..cnt): the k-th largest key kstar and how many
// entries equal to kstar belong to the top-k (need >= 1).
template <int DT>
__device__ void radix_select(const uint32_t *keys, int cnt, int k, uint32_t *hist,
                             uint32_t &kstar, int &need)
{
    const int lane = lane_id();
    uint32_t prefix = 0u, pmask = 0u;
    int rem = k;
    constexpr int last = (DT == kBF16) ? 2 : 0;
    for (int d = 3; d >= last; --d) {
        const int shift = 8 * d;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            hist[4 * lane + j] = 0u;
        wave_lds_sync();
        for (int i = lane; i < cnt; i += kWave) {
            const uint32_t key = keys[i];
            if ((key & pmask) == prefix)
                atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        wave_lds_sync();
        uint32_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            h[j] = hist[4 * lane + j];
        const uint32_t c = h[0] + h[1] + h[2] + h[3];
        // inclusive suffix sum over lanes >= this lane
        uint32_t incl = c;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const uint32_t t = __shfl_down(incl, off, kWave);
            if (lane + off < kWave)
                incl += t;
        }
        uint32_t above = incl - c;  // keys in bins of higher lanes
        int found = -1;
        uint32_t found_above = 0u;
#pragma unroll
        for (int j = 3; j >= 0; --j) {
            if (found < 0 && above < (uint32_t)rem && (uint32_t)rem <= above + h[j]) {
                found = j;
                found_above = above;
            }
            above += h[j];
        }
        const uint64_t bl = ballot(found >= 0);
        const int src = __builtin_ctzll(bl);
        const int bin = __builtin_amdgcn_readlane(4 * lane + found, src);
        const int fa = __builtin_amdgcn_readlane((int)found_above, src);
        prefix |= (uint32_t)bin << shift;
        pmask |= 255u << shift;
        rem -= fa;
    }
    if constexpr (DT == kBF16)
        prefix |= (prefix >> 31) ? 0u : 0xFFFFu;
    kstar = prefix;
    need = rem;
}

// Keep, in buffer order, the keys above kstar and the first `need` equal to
// it; returns the new count (= k).
__device__ int compact_topk(uint32_t *keys, uint32_t *ids, int cnt, uint32_t kstar, int need)
{
    const int lane = lane_id();
    int out = 0, eq_seen = 0;
    for (int base = 0; base < cnt; base += kWave) {
        const int i = base + lane;
        const bool valid = i < cnt;
        const uint32_t key = valid ? keys[i] : 0u;
        const uint32_t id = valid ? ids[i] : 0u;
        const bool gt = valid && key > kstar;
        const bool eq = valid && key == kstar;
        const uint64_t eqb = ballot(eq);
        const int eq_rank = eq_seen + lanes_below(eqb);
        const bool keep = gt || (eq && eq_rank < need);
        const uint64_t kb = ballot(keep);
        wave_lds_sync();  // every lane has read its entry before any write
        if (keep) {
            const int pos = out + lanes_below(kb);
            keys[pos] = key;
            ids[pos] = id;
        }
        out += __builtin_popcountll(kb);
        eq_seen += __builtin_popcountll(eqb);
        wave_lds_sync();
    }
    return out;
}

template <int DT, bool VEC, int CAP, int WPB>
__global__ __launch_bounds__(WPB * kWave) void topk_kernel(TopkArgs a)
{
    using IO = RowIO<DT, VEC>;
    using Raw = typename IO::Raw;
    constexpr int N = IO::N;
    constexpr int U = (N == 1) ? 16 : (N == 4 ? 8 : 4);
    constexpr int SUB = kWave * N;  // elements per sub-tile

    __shared__ uint32_t s_key[WPB][CAP];
    __shared__ uint32_t s_id[WPB][CAP];
    __shared__ uint32_t s_hist[WPB][256];

    const int w = threadIdx.x / kWave;
    const int lane = lane_id();
    const int64_t row = (int64_t)blockIdx.x * WPB + w;
    if (row >= a.ntok)
        return;  // whole wave; the kernel has no block barrier

    uint32_t *keys = s_key[w];
    uint32_t *ids = s_id[w];
    uint32_t *hist = s_hist[w];
    const int k = (int)a.k;
    const int64_t V = a.V;
    const int64_t nvec = V / N;
    const char *rowp =
        reinterpret_cast<const char *>(a.logits) + row * V * (int64_t)elt_bytes<DT>();

    int cnt = 0;
    bool thr_set = false;
    float thr = -INFINITY;

    // One tile: U sub-tiles of 64 vectors; sub-tile u of the tile at t0
    // holds vectors t0 + 64u .. t0 + 64u + 63, lane l the vector t0 + 64u + l.
    auto load_tile = [&](int64_t t0, Raw (&buf)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t v = t0 + (int64_t)u * kWave + lane;
            buf[u] = v < nvec ? IO::load_raw(rowp, v) : neg_inf_raw<DT, VEC>();
        }
    };
    auto process_tile = [&](int64_t t0, const Raw (&buf)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t vbase = t0 + (int64_t)u * kWave;
            if (vbase >= nvec)
                break;
            const int64_t v = vbase + lane;
            const bool valid = v < nvec;
            float x[N];
            IO::unpack(buf[u], x);
            if (thr_set) {
                float mx = -INFINITY;
#pragma unroll
                for (int c = 0; c < N; ++c)
                    mx = fmaxf(mx, x[c]);
                if (ballot(valid && mx > thr) == 0ull)
                    continue;
            }
            if (cnt + SUB > CAP) {
                uint32_t kstar;
                int need;
                radix_select<DT>(keys, cnt, k, hist, kstar, need);
                cnt = compact_topk(keys, ids, cnt, kstar, need);
                thr_set = true;
                thr = key_value(kstar);
            }
            uint32_t mask = 0u;
            if (valid) {
#pragma unroll
                for (int c = 0; c < N; ++c)
                    if (!thr_set || x[c] > thr)
                        mask |= 1u << c;
            }
            const uint32_t lc = __builtin_popcount(mask);
            // exclusive prefix of lc over lanes, bit-sliced (lc <= 8)
            int prefix = 0, total = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint64_t bb = ballot((lc >> b) & 1u);
                prefix += lanes_below(bb) << b;
                total += __builtin_popcountll(bb) << b;
            }
            int pos = cnt + prefix;
#pragma unroll
            for (int c = 0; c < N; ++c) {
                if ((mask >> c) & 1u) {
                    keys[pos] = order_key(x[c]);
                    ids[pos] = (uint32_t)(v * N + c);
                    ++pos;
                }
            }
            cnt += total;
            wave_lds_sync();
        }
    };

    // Double-buffered: the next tile's loads are in flight while this one
    // is filtered.
    constexpr int64_t TILE = (int64_t)kWave * U;
    Raw bufA[U], bufB[U];
    int64_t t0 = 0;
    load_tile(0, bufA);
    while (t0 < nvec) {
        if (t0 + TILE < nvec)
            load_tile(t0 + TILE, bufB);
        process_tile(t0, bufA);
        t0 += TILE;
        if (t0 >= nvec)
            break;
        if (t0 + TILE < nvec)
            load_tile(t0 + TILE, bufA);
        process_tile(t0, bufB);
        t0 += TILE;
    }

    // exactly k winners, in id order
    {
        uint32_t kstar;
        int need;
        wave_lds_sync();
        radix_select<DT>(keys, cnt, k, hist, kstar, need);
        cnt = compact_topk(keys, ids, cnt, kstar, need);
    }

    // renormalised probabilities over the k winners
    float vmax = -INFINITY;
    for (int i = lane; i < k; i += kWave)
        vmax = fmaxf(vmax, key_value(keys[i]));
    const float v0 = wave_max(vmax);
    float z = 0.f;
    for (int i = lane; i < k; i += kWave)
        z += __expf(key_value(keys[i]) - v0);
    const float Z = wave_sum(z);

    uint32_t *out_ids = a.ids + row * a.k;
    float *out_p = a.probs + row * a.k;
    for (int i0 = 0; i0 < k; i0 += kWave) {
        const int i = i0 + lane;
        const bool valid = i < k;
        const uint32_t ki = valid ? keys[i] : 0u;
        int rank = 0;
        for (int j = 0; j < k; ++j) {
            const uint32_t kj = keys[j];
            rank += (kj > ki) || (kj == ki && j < i);
        }
        if (valid) {
            out_ids[rank] = ids[i];
            out_p[rank] = __expf(key_value(ki) - v0) / Z;
        }
    }
}

namespace {

template <int DT, bool VEC, int CAP>
hipError_t launch_cap(const TopkArgs &a, hipStream_t st)
{
    constexpr int WPB = CAP <= 1024 ? 4 : (CAP == 2048 ? 2 : 1);
    const int64_t grid = (a.ntok + WPB - 1) / WPB;
    hipLaunchKernelGGL((topk_kernel<DT, VEC, CAP, WPB>), dim3((unsigned)grid),
                       dim3(WPB * kWave), 0, st, a);
    return hipGetLastError();
}

template <int DT, bool VEC>
hipError_t launch_dt(const TopkArgs &a, hipStream_t st)
{
    constexpr int SUB = kWave * RowIO<DT, VEC>::N;
    const int64_t need = a.k + SUB;
    if (need <= 512)
        return launch_cap<DT, VEC, 512>(a, st);
    if (need <= 1024)
        return launch_cap<DT, VEC, 1024>(a, st);
    if (need <= 2048)
        return launch_cap<DT, VEC, 2048>(a, st);
    return launch_cap<DT, VEC, 4096>(a, st);
}

}  // namespace

hipError_t launch_topk(int dtype, const TopkArgs &a, hipStream_t st)
{
    const size_t elt = dtype == kF32 ? 4 : 2;
    const int n = 16 / (int)elt;
    const bool vec = ((uintptr_t)a.logits % 16 == 0) && (a.V % n == 0);
    if (dtype == kF32)
        return vec ? launch_dt<kF32, true>(a, st) : launch_dt<kF32, false>(a, st);
    return vec ? launch_dt<kBF16, true>(a, st) : launch_dt<kBF16, false>(a, st);
}

}  // namespace vl
