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
// One wave owns a row and streams it once, in tiles of 64 lanes x 2
// 16-byte vectors (the next tile's loads in flight while one is filtered);
// a tile's ids are all larger than every earlier tile's.  Values pass an
// acceptance test into a per-wave LDS candidate buffer of (key, id) pairs,
// written in id order.  The key is the order-preserving unsigned image of
// the float (sign-flipped, -0 folded onto +0), so key order is value order.
// Until the buffer first fills every value is accepted; when a sub-tile
// might overflow it, the buffer is compacted.  Mid-row that keeps every key
// at or above a bound that at least k keys reach (the first radix bin edge
// that keeps few enough); at the end it is exact: the keys above the k-th
// key and, of those equal to it, the first ones in buffer (= id) order.
// The bound becomes the threshold: later elements have larger ids, so only
// values strictly above it can enter the top-k.  Each value is compared
// once, straight into a scalar lane mask per value position; the masks'
// OR skips a sub-tile no value of which passes, and when no lane holds two
// candidates (the usual case) the masks also pick each lane's candidate
// value and id with lane-select instructions.
//
// The select holds the candidates in registers and is a radix select on
// key - min(key) over the buffer: 8-bit digits from the highest set bit of
// the range down, counted in an LDS histogram.  Digits relative to the
// buffer's own range spread near-equal keys over the bins (few colliding
// LDS increments) and skip the bits every candidate shares.  Bin counts are
// scanned across the wave with DPP.
//
// At the end the buffer is selected once more to exactly k winners, which
// a bitonic sort on (key, complemented id) puts in output order: in
// registers up to 512 winners (lanes exchange entries with ds_bpermute),
// in the LDS buffer beyond; the probabilities are formed from the winners'
// values.
#include <math.h>

#include <type_traits>

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

// t in the lanes whose bit of the scalar mask m is set, f in the others:
// one v_cndmask_b32 with m as its lane-select operand.
// (m is wave-uniform; readfirstlane makes the compiler keep it in scalar
// registers, which the instruction's mask operand must be.)
__device__ __forceinline__ uint32_t lane_select(uint64_t m, uint32_t t, uint32_t f)
{
    const uint64_t ms =
        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(m >> 32)) << 32) |
        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)m);
    uint32_t r;
    __asm__("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(f), "v"(t), "s"(ms));
    return r;
}

constexpr int pow2_ceil(int x)
{
    int p = 1;
    while (p < x)
        p <<= 1;
    return p;
}

struct Selected {
    int cnt;        // entries kept
    uint32_t key;   // exact: the k-th largest key; else the smallest key kept
};

// Compact the candidate buffer keys/ids[0..cnt) (cnt >= k, at most 64 E
// entries), in buffer order.
//   limit == 0: to its top-k exactly (the k-th largest key, and of the keys
//               equal to it only the first ones).
//   limit > 0:  to every key >= some bound that at least k keys reach; the
//               radix passes stop as soon as that keeps at most `limit`
//               entries.  Whatever it keeps holds the top-k, and a later
//               element (larger id) not above the bound cannot enter it.
template <int E>
__device__ __forceinline__ Selected select_compact(uint32_t *keys, uint32_t *ids, int cnt, int k,
                                                   uint32_t *hist, int limit = 0)
{
    const int lane = lane_id();
    uint32_t kr[E];
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int i = lane + kWave * e;
        kr[e] = i < cnt ? keys[i] : 0u;
        if (i < cnt) {
            lo = min(lo, kr[e]);
            hi = max(hi, kr[e]);
        }
    }
    lo = wave_min_u32(lo);
    hi = wave_max_u32(hi);
    const uint32_t span = hi - lo;
    // Bits below the lowest one on which rel = key - lo varies are zero in
    // every rel (bf16 keys, for one, share their low 16 bits); no pass
    // needs to look at them.
    uint32_t vary = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e)
        if (lane + kWave * e < cnt)
            vary |= kr[e] - lo;
    vary = wave_or_u32(vary);
    const int low = vary ? __builtin_ctz(vary) : 0;

    // Radix select on rel = key - lo: rel of the k-th largest key.
    uint32_t prefix = 0u;  // the bits of that rel decided so far
    int rem = k;           // how many of the keys matching prefix are needed
    bool keep_ge = false;  // stopped early: keep every rel >= prefix
    if (span != 0u) {
        for (int hb = 32 - __builtin_clz(span); hb > low; hb -= 8) {
            const int sh = hb - 8 > low ? hb - 8 : low;
            const uint32_t dmask = (1u << (hb - sh)) - 1u;
            const uint32_t above_mask = hb >= 32 ? 0u : ~((1u << hb) - 1u);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                hist[4 * lane + j] = 0u;
            wave_lds_sync();
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const uint32_t rel = kr[e] - lo;
                if (lane + kWave * e < cnt && (rel & above_mask) == prefix)
                    atomicAdd(&hist[(rel >> sh) & dmask], 1u);
            }
            wave_lds_sync();
            // Lane l holds bins 255-4l .. 252-4l (descending), so the
            // exclusive prefix over lanes counts the keys in higher bins.
            uint32_t h[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                h[j] = hist[255 - 4 * lane - j];
            const uint32_t c = h[0] + h[1] + h[2] + h[3];
            uint32_t above = wave_prefix_sum_u32(c) - c;
            int found = -1;
            uint32_t found_above = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (found < 0 && above < (uint32_t)rem && (uint32_t)rem <= above + h[j]) {
                    found = j;
                    found_above = above;
                }
                above += h[j];
            }
            const uint64_t bl = ballot(found >= 0);
            const int src = bl ? __builtin_ctzll(bl) : 0;
            const int fj = found < 0 ? 0 : found;
            const uint32_t bin = (uint32_t)__builtin_amdgcn_readlane(255 - 4 * lane - fj, src);
            const int fa = __builtin_amdgcn_readlane((int)found_above, src);
            const uint32_t hb_cnt = fj == 0 ? h[0] : fj == 1 ? h[1] : fj == 2 ? h[2] : h[3];
            const int in_bin = __builtin_amdgcn_readlane((int)hb_cnt, src);
            prefix |= (bin & dmask) << sh;
            // keys >= the bin's lower edge: those above the decided digits,
            // those in higher bins of this pass, and the bin itself
            if (limit > 0 && (k - rem) + fa + in_bin <= limit) {
                keep_ge = true;
                break;
            }
            rem -= fa;
        }
    }
    const uint32_t kstar = lo + prefix;

    // Keep the keys above kstar and the first `rem` equal to it, in order.
    // The buffer is rewritten in place: chunk e writes only below
    // 64 (e + 1), and each lane reads its id before any lane writes.
    int out = 0, eq_seen = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const bool valid = lane + kWave * e < cnt;
        const uint32_t id = valid ? ids[lane + kWave * e] : 0u;
        const bool gt = valid && kr[e] > kstar;
        const bool eq = valid && kr[e] == kstar;
        const uint64_t eqb = ballot(eq);
        const bool keep = gt || (eq && (keep_ge || eq_seen + lanes_below(eqb) < rem));
        const uint64_t kb = ballot(keep);
        wave_lds_sync();
        if (keep) {
            const int pos = out + lanes_below(kb);
            keys[pos] = kr[e];
            ids[pos] = id;
        }
        out += __builtin_popcountll(kb);
        eq_seen += __builtin_popcountll(eqb);
    }
    wave_lds_sync();
    return {out, kstar};
}

// Sort entry: the key above the bitwise complement of the id, so that
// descending order of the pair is value descending, id ascending.  Padding
// is 0, below every real entry (ids are below 2^32 - 1).
__device__ __forceinline__ uint64_t sort_pair(uint32_t key, uint32_t id)
{
    return ((uint64_t)key << 32) | (uint32_t)~id;
}

// The value of lane (this lane ^ J): DPP within quads for J = 1, 2,
// ds_bpermute otherwise.
template <int J>
__device__ __forceinline__ uint32_t xor_lanes(uint32_t v, int lane)
{
    if constexpr (J == 1)
        return dpp_u32<0xB1>(v, v);  // quad_perm [1, 0, 3, 2]
    else if constexpr (J == 2)
        return dpp_u32<0x4E>(v, v);  // quad_perm [2, 3, 0, 1]
    else
        return (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ J) << 2, (int)v);
}

template <int J>
__device__ __forceinline__ uint64_t xor_lanes(uint64_t v, int lane)
{
    return ((uint64_t)xor_lanes<J>((uint32_t)(v >> 32), lane) << 32) |
           xor_lanes<J>((uint32_t)v, lane);
}

// One compare-exchange step of a descending bitonic sort over 64 EP entries
// (entry i is register i / 64 of lane i % 64): partner i ^ J; blocks of KK
// entries whose index has bit KK clear end descending, the others
// ascending.  Partners in other lanes are exchanged for all registers
// first, then compared, so one wait covers a step.
template <int KK, int J, int EP, typename T>
__device__ __forceinline__ void bitonic_step(T (&K)[EP], int lane)
{
    if constexpr (J < kWave) {
        T b[EP];
#pragma unroll
        for (int e = 0; e < EP; ++e)
            b[e] = xor_lanes<J>(K[e], lane);
        const bool lower = (lane & J) == 0;
#pragma unroll
        for (int e = 0; e < EP; ++e) {
            const bool desc = ((e * kWave + lane) & KK) == 0;
            const T a = K[e];
            K[e] = (lower == desc) ? (a > b[e] ? a : b[e]) : (a < b[e] ? a : b[e]);
        }
    } else {
        constexpr int JE = J / kWave;
#pragma unroll
        for (int e = 0; e < EP; ++e) {
            if (e & JE)
                continue;
            const bool desc = ((e * kWave) & KK) == 0;
            const T a = K[e], b = K[e | JE];
            const bool sw = desc ? a < b : a > b;
            K[e] = sw ? b : a;
            K[e | JE] = sw ? a : b;
        }
    }
}

template <int KK, int J, int EP, typename T>
__device__ __forceinline__ void bitonic_merge(T (&K)[EP], int lane)
{
    bitonic_step<KK, J, EP>(K, lane);
    if constexpr (J > 1)
        bitonic_merge<KK, J / 2, EP>(K, lane);
}

// Sort the 64 EP entries descending: stages KK = 2, 4, ..., 64 EP, fully
// unrolled.  `lane` is the lane index.
template <int KK, int EP, typename T>
__device__ __forceinline__ void bitonic_sort_desc(T (&K)[EP], int lane)
{
    bitonic_merge<KK, KK / 2, EP>(K, lane);
    if constexpr (KK < kWave * EP)
        bitonic_sort_desc<KK * 2, EP>(K, lane);
}

// The k winners in keys/ids[0..k), in id order: sort them and write the ids
// and renormalised probabilities in rank order; 64 EP >= k entries in EP
// registers a lane.  bf16 keys (BF) carry the value in their upper 16 bits,
// so a 32-bit entry holds the key's upper half above 0xFFFF - (buffer
// index): descending is value descending, index (= id) ascending.
// float32 entries are 64-bit: the key above the complemented id.
template <int EP, bool BF>
__device__ __forceinline__ void write_ranked(const uint32_t *keys, const uint32_t *ids, int k,
                                             uint32_t *out_ids, float *out_p)
{
    const int lane = lane_id();
    typedef typename std::conditional<BF, uint32_t, uint64_t>::type T;
    T K[EP];
#pragma unroll
    for (int e = 0; e < EP; ++e) {
        const int i = lane + kWave * e;
        if constexpr (BF)
            K[e] = i < k ? ((keys[i] & 0xFFFF0000u) | (0xFFFFu - (uint32_t)i)) : 0u;
        else
            K[e] = i < k ? sort_pair(keys[i], ids[i]) : 0ull;
    }
    bitonic_sort_desc<2, EP>(K, lane);
    // the entry's key (bf16: the lower half is 0 for values >= +0 and
    // 0xFFFF below, as order_key makes it)
    auto key_of = [](T x) {
        if constexpr (BF) {
            const uint32_t hi = x & 0xFFFF0000u;
            return hi | ((hi & 0x80000000u) ? 0u : 0xFFFFu);
        } else {
            return (uint32_t)(x >> 32);
        }
    };
    const float v0 = key_value((uint32_t)__builtin_amdgcn_readlane((int)key_of(K[0]), 0));
    float ev[EP];
    float z = 0.f;
#pragma unroll
    for (int e = 0; e < EP; ++e) {
        ev[e] = __expf(key_value(key_of(K[e])) - v0);
        if (lane + kWave * e < k)
            z += ev[e];
    }
    const float Z = wave_sum(z);
#pragma unroll
    for (int e = 0; e < EP; ++e) {
        const int i = lane + kWave * e;
        // Non-temporal: nothing reads the output soon (16384 x 151936
        // bf16, k = 256: 16 us less than ordinary stores).
        if (i < k) {
            if constexpr (BF)
                __builtin_nontemporal_store(ids[0xFFFFu - (K[e] & 0xFFFFu)], out_ids + i);
            else
                __builtin_nontemporal_store(~(uint32_t)K[e], out_ids + i);
            __builtin_nontemporal_store(ev[e] / Z, out_p + i);
        }
    }
}

// Up to CAP 1024 the register budget is held to four waves per SIMD (128
// VGPRs): the 1024-entry bf16 variant would otherwise take 138 and run three
// waves per SIMD, 11% slower at 16384 x 151936 despite a few spilled
// registers in its compaction.
// Above 512 winners the register sort would need 16+ register pairs per
// lane; the k winners are sorted in place in the LDS buffer instead, by the
// same bitonic network over P = the power of two >= k entries (CAP >= P
// because CAP >= k + one sub-tile).  keys/ids[k..P) are padded with the
// pair that sorts last.
__device__ __forceinline__ void write_ranked_lds(uint32_t *keys, uint32_t *ids, int k, uint32_t *out_ids,
                                                 float *out_p)
{
    const int lane = lane_id();
    int P = kWave;
    while (P < k)
        P <<= 1;
    for (int i = k + lane; i < P; i += kWave) {
        keys[i] = 0u;
        ids[i] = 0xFFFFFFFFu;
    }
    wave_lds_sync();
    for (int kk = 2; kk <= P; kk <<= 1) {
        for (int j = kk >> 1; j > 0; j >>= 1) {
            // pair number pp: lower index i, partner i + j
            for (int pp = lane; pp < P / 2; pp += kWave) {
                const int i = 2 * j * (pp / j) + pp % j;
                const int l = i + j;
                const uint64_t a = sort_pair(keys[i], ids[i]);
                const uint64_t b = sort_pair(keys[l], ids[l]);
                const bool desc = (i & kk) == 0;
                if (desc ? a < b : a > b) {
                    keys[i] = (uint32_t)(b >> 32);
                    ids[i] = ~(uint32_t)b;
                    keys[l] = (uint32_t)(a >> 32);
                    ids[l] = ~(uint32_t)a;
                }
            }
            wave_lds_sync();
        }
    }
    const float v0 = key_value(keys[0]);
    float z = 0.f;
    for (int i = lane; i < k; i += kWave)
        z += __expf(key_value(keys[i]) - v0);
    const float Z = wave_sum(z);
    for (int i = lane; i < k; i += kWave) {
        __builtin_nontemporal_store(ids[i], out_ids + i);
        __builtin_nontemporal_store(__expf(key_value(keys[i]) - v0) / Z, out_p + i);
    }
}

template <int DT, bool VEC, int CAP, int WPB>
__global__ __launch_bounds__(WPB * kWave, (CAP <= 1024 ? 4 : 1)) void topk_kernel(TopkArgs a)
{
    using IO = RowIO<DT, VEC>;
    using Raw = typename IO::Raw;
    constexpr int N = IO::N;
    // Tiles of 2 sub-tiles (the next tile in flight while one is filtered):
    // 2-3% faster than 4 at 4096 x 32000 and 16384 x 151936.
    constexpr int U = 2;
    constexpr int SUB = kWave * N;  // elements per sub-tile
    constexpr int E = CAP / kWave;
    // k <= min(CAP - SUB, kMaxTopk); the sort pads k to a power of two.
    constexpr int kMaxK = (CAP - SUB) < kMaxTopk ? (CAP - SUB) : (int)kMaxTopk;
    constexpr int kSortRegs = pow2_ceil(kMaxK) / kWave > 0 ? pow2_ceil(kMaxK) / kWave : 1;
    // Registers a lane may take for the final sort (64 per register a
    // lane): up to 8 in the four-waves-per-SIMD variants (CAP <= 1024); the
    // larger buffers serve k above 256 (bf16) or 512 (float32) and sort in
    // LDS.
    constexpr int kRegSort = CAP <= 1024 ? (kSortRegs < 8 ? kSortRegs : 8) : 0;

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
    const int kSelLimit = topk_sel_limit(k, CAP, SUB);
    const uint32_t nvec = (uint32_t)(a.V / N);
    const char *rowp =
        reinterpret_cast<const char *>(a.logits) + row * a.V * (int64_t)elt_bytes<DT>();

    int cnt = 0;
    bool thr_set = false;
    float thr = -INFINITY;

    // One tile: U sub-tiles of 64 vectors; sub-tile u of the tile at t0
    // holds vectors t0 + 64u .. t0 + 64u + 63, lane l the vector t0 + 64u + l.
    // Loads are unconditional (index clamped into the row) and non-temporal:
    // the row is read once.
    auto load_tile = [&](uint32_t t0, Raw (&buf)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t v = t0 + (uint32_t)u * kWave + lane;
            buf[u] = IO::load_stream(rowp, v < nvec ? v : nvec - 1);
        }
    };
    // Candidate masks of one sub-tile: lane l's bit of cand[c] is set when
    // its value c passes (before the first compaction every valid value
    // does).  One compare per value, each straight into a scalar lane mask.
    // A bf16 value in the high half of a 32-bit word is compared as that
    // word read as float32: the low half only extends the mantissa, so the
    // word lies strictly above thr whenever the value does (thr is itself a
    // bf16 value, so a value above it is at least one bf16 step above), and
    // the only other words above thr hold a value equal to thr -- a later
    // element than the ones already kept at thr, which can never win its
    // tie, so accepting it changes nothing.
    auto candidate_masks = [&](const Raw &r, bool valid, uint64_t (&cand)[N]) {
        if (!thr_set) {
            const uint64_t all = ballot(valid);
#pragma unroll
            for (int c = 0; c < N; ++c)
                cand[c] = all;
            return;
        }
        const uint64_t vm = ballot(valid);
        if constexpr (N == 8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t w = r[j];
                cand[2 * j] = ballot(__builtin_bit_cast(float, w << 16) > thr) & vm;
                cand[2 * j + 1] = ballot(__builtin_bit_cast(float, w) > thr) & vm;
            }
        } else {
            float x[N];
            IO::unpack(r, x);
#pragma unroll
            for (int c = 0; c < N; ++c)
                cand[c] = ballot(x[c] > thr) & vm;
        }
    };
    auto process_tile = [&](uint32_t t0, const Raw (&buf)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t vbase = t0 + (uint32_t)u * kWave;
            if (vbase >= nvec)
                break;
            const uint32_t v = vbase + lane;
            const bool valid = v < nvec;
            uint64_t cand[N];
            candidate_masks(buf[u], valid, cand);
            uint64_t any = 0, multi = 0;
#pragma unroll
            for (int c = 0; c < N; ++c) {
                multi |= any & cand[c];
                any |= cand[c];
            }
            if (any == 0ull)
                continue;  // no value of the sub-tile can enter
            if (cnt + SUB > CAP) {
                const Selected sel = select_compact<E>(keys, ids, cnt, k, hist, kSelLimit);
                cnt = sel.cnt;
                thr = key_value(sel.key);
                thr_set = true;
                candidate_masks(buf[u], valid, cand);
                any = 0;
                multi = 0;
#pragma unroll
                for (int c = 0; c < N; ++c) {
                    multi |= any & cand[c];
                    any |= cand[c];
                }
                if (any == 0ull)
                    continue;
            }
            if (multi == 0ull) {
                // Common case: at most one candidate per lane, picked out
                // of the lane's values by the scalar masks; lane order is
                // id order.
                uint32_t bits, c;
                if constexpr (N == 8) {
                    const uint64_t odd = cand[1] | cand[3] | cand[5] | cand[7];
                    const uint64_t c2 = cand[2] | cand[3] | cand[6] | cand[7];
                    const uint64_t c4 = cand[4] | cand[5] | cand[6] | cand[7];
                    uint32_t w = lane_select(cand[2] | cand[3], buf[u][1], buf[u][0]);
                    w = lane_select(cand[4] | cand[5], buf[u][2], w);
                    w = lane_select(cand[6] | cand[7], buf[u][3], w);
                    bits = lane_select(odd, w & 0xFFFF0000u, w << 16);
                    c = lane_select(odd, 1u, 0u) | lane_select(c2, 2u, 0u) | lane_select(c4, 4u, 0u);
                } else if constexpr (N == 4) {
                    bits = lane_select(cand[1], buf[u][1], buf[u][0]);
                    bits = lane_select(cand[2], buf[u][2], bits);
                    bits = lane_select(cand[3], buf[u][3], bits);
                    c = lane_select(cand[1], 1u, 0u);
                    c = lane_select(cand[2], 2u, c);
                    c = lane_select(cand[3], 3u, c);
                } else {
                    float x[N];
                    IO::unpack(buf[u], x);
                    bits = __builtin_bit_cast(uint32_t, x[0]);
                    c = 0u;
                }
                if ((any >> lane) & 1ull) {
                    const int pos = cnt + lanes_below(any);
                    keys[pos] = order_key(__builtin_bit_cast(float, bits));
                    ids[pos] = v * N + c;
                }
                cnt += __builtin_popcountll(any);
            } else {
                float x[N];
                IO::unpack(buf[u], x);
                uint32_t mask = 0u;
#pragma unroll
                for (int c = 0; c < N; ++c)
                    mask |= lane_select(cand[c], 1u << c, 0u);
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
                        ids[pos] = v * N + c;
                        ++pos;
                    }
                }
                cnt += total;
            }
            wave_lds_sync();
        }
    };

    // The next tile is always loaded (past the row end the clamped index
    // re-reads its last vector), so every iteration issues the same loads
    // and the waits derived for the current tile never cover the next one.
    constexpr uint32_t TILE = (uint32_t)kWave * U;
    Raw bufA[U], bufB[U];
    uint32_t t0 = 0;
    load_tile(0, bufA);
    while (t0 < nvec) {
        load_tile(t0 + TILE, bufB);
        process_tile(t0, bufA);
        t0 += TILE;
        if (t0 >= nvec)
            break;
        load_tile(t0 + TILE, bufA);
        process_tile(t0, bufB);
        t0 += TILE;
    }

    // exactly k winners, in id order, then written at their ranks; the
    // selection runs over as many registers as the buffer's fill needs
    // (it usually holds far fewer than CAP entries by the row's end)
    wave_lds_sync();
    if (E > 2 && cnt <= 2 * kWave)
        select_compact<(E > 2 ? 2 : E)>(keys, ids, cnt, k, hist);
    else if (E > 4 && cnt <= 4 * kWave)
        select_compact<(E > 4 ? 4 : E)>(keys, ids, cnt, k, hist);
    else if (E > 8 && cnt <= 8 * kWave)
        select_compact<(E > 8 ? 8 : E)>(keys, ids, cnt, k, hist);
    else
        select_compact<E>(keys, ids, cnt, k, hist);  // leaves exactly k entries
    uint32_t *oi = a.ids + row * a.k;
    float *op = a.probs + row * a.k;
    constexpr bool BF = DT == kBF16;
    if (k <= kWave && kRegSort >= 1) {
        write_ranked<1, BF>(keys, ids, k, oi, op);
    } else if (k <= 2 * kWave && kRegSort >= 2) {
        write_ranked<2, BF>(keys, ids, k, oi, op);
    } else if (k <= 4 * kWave) {
        if constexpr (kRegSort >= 4)
            write_ranked<4, BF>(keys, ids, k, oi, op);
        else
            write_ranked_lds(keys, ids, k, oi, op);
    } else if (k <= 8 * kWave) {
        if constexpr (kRegSort >= 8)
            write_ranked<8, BF>(keys, ids, k, oi, op);
        else
            write_ranked_lds(keys, ids, k, oi, op);
    } else {
        write_ranked_lds(keys, ids, k, oi, op);
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
    const int cap = topk_cap(a.k, kWave * RowIO<DT, VEC>::N);
    if (cap == 512)
        return launch_cap<DT, VEC, 512>(a, st);
    if (cap == 1024)
        return launch_cap<DT, VEC, 1024>(a, st);
    if (cap == 2048)
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
