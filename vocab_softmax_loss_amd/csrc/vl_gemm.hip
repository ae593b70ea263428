// The vocabulary head's logits product on the gfx950 matrix cores
// (cortiq-engine train_head.rs: head_kl, the per-slice logits product that
// feeds kl_rows; topk, the same product feeding topk_rows):
//
//   C[m][n] = sum_k A[m][k] B[n][k]        A = half(hidden rows)  [M][lda]
//                                          B = head weights W     [N][K]
//                                          C = float32 logits     [M][N]
//
// with an optional row-statistics epilogue: for every row m and every
// 128-column half of a 256-column tile t, the record (a, z) = (max of
// C[m][cols], sum exp(C[m][cols] - a)) goes to rec[m][2t + half].  The
// softmax of a row then needs one merge of its records instead of a pass
// over its logits.
//
// Schedule.  One 256-thread workgroup (4 waves) per 256 x 256 output tile,
// one workgroup per CU (the LDS stages take 128 KB).  K goes in steps of
// 64 through two LDS stages of 64 KB (A and B tiles of 256 rows x 128
// bytes), filled with asynchronous global->LDS loads
// (global_load_lds_dwordx4) one step ahead.  Wave (wm, wn) computes the
// 128 x 128 quarter (wm, wn) as 4 x 4 blocks of v_mfma_f32_32x32x16 (bf16
// or f16 inputs, float32 accumulators: 256 per lane, in AGPRs).  Within a
// step the operand reads of the next K16 slice are issued ahead of the
// current slice's 16 MFMAs, and the next stage's 16 loads go out one per
// 4 MFMAs (sched_barrier groups fix that order).
//
// Tile order.  Workgroup b runs on XCD b % 8; the XCDs take contiguous
// shares of the tile order, which walks groups of 16 tile rows (the rows of
// a group fastest), so the 32 tiles in flight on an XCD share their A and B
// slices in its L2.  Each tile takes its K steps in a rotated order
// (starting at step t mod nk): with 2 KB rows (K = 1024) every row of a
// slice maps to the same few L2 channels, and tiles in flight on different
// slices spread the load (8% faster at 16384 x 151936 x 1024).
//
// LDS layout.  Row r of a tile holds its 64 values as 8 chunks of 16 bytes;
// logical chunk c sits at physical chunk c ^ ((r >> 1) & 7).  An MFMA
// operand read (ds_read_b128, lane l: row l % 32, chunk 2s + l / 32) then
// touches 16 distinct 16-byte bank groups in every 16 lanes, and the
// asynchronous loads, which write 64 lanes x 16 bytes contiguously, load
// each lane's chunk from the matching global address.
//
// MFMA operand layout (v_mfma_f32_32x32x16, checked on the device): lane l
// supplies row l % 32 of A and row l % 32 of B (a column of B^T), 8
// consecutive k values each, the same 8 for A and B; the result has
// C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] in accumulator r of lane l.
#include <type_traits>

#include "vl.h"
#include "vl_device.hpp"
#include "vl_launch.hpp"

namespace vl {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

namespace {

constexpr int kTileM = 256, kTileN = 256, kTileK = 64;
constexpr int kGroupM = 16;                               // tile rows per group
constexpr int kTileBytes = kTileM * kTileK * 2;          // 32 KB: one operand tile
constexpr int kStageBytes = 2 * kTileBytes;              // A and B
static_assert(kTileM == kLogitsTile && kTileN == kLogitsTile && kTileK == kLogitsKStep,
              "tile sizes");

template <bool BF>
__device__ __forceinline__ f32x16 mfma32(const u32x4 &a, const u32x4 &b, const f32x16 &c)
{
    if constexpr (BF)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// (a, z) <- (a, z) merged with (a2, z2): the larger anchor stays and the
// other sum is rescaled by exp(smaller - larger); empty records are
// (-inf, 0).
__device__ __forceinline__ void merge_rec(float &a, float &z, float a2, float z2)
{
    const bool first = a >= a2;
    const float hi = first ? a : a2, lo = first ? a2 : a;
    const float zh = first ? z : z2, zl = first ? z2 : z;
    const float e = hi == -INFINITY ? 0.f : __expf(lo - hi);
    a = hi;
    z = zh + zl * e;
}

}  // namespace

template <bool BF, bool STATS>
__global__ __launch_bounds__(256, 1) void logits_kernel(LogitsArgs g)
{
    __shared__ __attribute__((aligned(1024))) char sm[2 * kStageBytes];
    const uint32_t tid = threadIdx.x, lane = tid & 63u, w = tid >> 6;
    const uint32_t wm = w >> 1, wn = w & 1u;

    // Tile of this workgroup: XCD-contiguous shares (the remainder past a
    // multiple of 8 keeps its own index), then the grouped order.
    const int64_t T = g.tiles_m * g.tiles_n;
    const int64_t b = blockIdx.x;
    const int64_t full = T / 8 * 8;
    const int64_t t = b < full ? (b % 8) * (T / 8) + b / 8 : b;
    const int64_t per_group = (int64_t)kGroupM * g.tiles_n;
    const int64_t grp = t / per_group, in = t - grp * per_group;
    const int64_t gm0 = grp * kGroupM;
    const int64_t gm_n = g.tiles_m - gm0 < kGroupM ? g.tiles_m - gm0 : kGroupM;
    const int64_t tm = gm0 + in % gm_n, tn = in / gm_n;
    const int64_t m0 = tm * kTileM, n0 = tn * kTileN;

    // Asynchronous loads: wave w, load j (0..7) fills tile rows
    // (4 j + w) * 8 .. +8, lane l row + l / 8, physical chunk l % 8, which
    // holds logical chunk c = (l % 8) ^ ((row >> 1) & 7); that swizzle key
    // is 4 (w & 1) + l / 16 (mod 8) for every j.  Rows past M or N load the
    // last row (their results are not stored).
    const uint32_t c = (lane & 7u) ^ ((4u * (w & 1u) + (lane >> 4)) & 7u);
    const char *pa[8];
    const char *pb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t r = (int64_t)((4 * j + (int)w) * 8) + (int64_t)(lane >> 3);
        const int64_t m = m0 + r < g.M ? m0 + r : g.M - 1;
        const int64_t n = n0 + r < g.N ? n0 + r : g.N - 1;
        pa[j] = static_cast<const char *>(g.a) + m * g.lda * 2;
        pb[j] = static_cast<const char *>(g.b) + n * g.K * 2;
    }

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.f;

    // Operand reads: lane l, row l % 32 of each 32-row block, logical
    // chunk 2 s + l / 32 at physical chunk (2 s + l / 32) ^ ((l % 32) >> 1 & 7).
    const uint32_t key = (lane >> 1) & 7u;
    const uint32_t hi = lane >> 5;
    const uint32_t arow = (wm * 128u + (lane & 31u)) * 128u;
    const uint32_t brow = (wn * 128u + (lane & 31u)) * 128u;

    const int nk = (int)((g.K + kTileK - 1) / kTileK);
    // Load q (0..15) of the stage for K offset k0 into LDS stage s: even q
    // the A rows of load j = q / 2, odd q the B rows.  A is zero past K up
    // to lda (a multiple of 64); B's columns past K load from the row start
    // instead (finite values times zero).
    auto load_one = [&](int s, int64_t k0, int q) {
        char *sa = sm + s * kStageBytes;
        const int j = q >> 1;
        const int off = (4 * j + (int)w) * 8 * 128;
        const int64_t ka = (k0 + 8 * (int64_t)c) * 2;
        if ((q & 1) == 0) {
            load_to_lds16(pa[j] + ka, sa + off);
        } else {
            const int64_t kb = k0 + 8 * (int64_t)c < g.K ? ka : 0;
            load_to_lds16(pb[j] + kb, sa + kTileBytes + off);
        }
    };
    u32x4 fa[2][4], fb[2][4];
    auto read_frags = [&](const char *sa, int s, u32x4 (&av)[4], u32x4 (&bv)[4]) {
        const uint32_t co = (((2u * s + hi) ^ key) * 16u);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            av[i] = *reinterpret_cast<const u32x4 *>(sa + arow + i * 32 * 128 + co);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            bv[j] = *reinterpret_cast<const u32x4 *>(sa + kTileBytes + brow + j * 32 * 128 + co);
    };
    const int rot = (int)(t % nk);
    for (int q = 0; q < 16; ++q)
        load_one(0, (int64_t)rot * kTileK, q);
    for (int kt = 0; kt < nk; ++kt) {
        wait_vm_all();
        block_sync_lds();
        const char *sa = sm + (kt & 1) * kStageBytes;
        // The next stage's loads.  On the last step they reload this tile's
        // first K slice into the idle stage (unused), so every step issues
        // the same instruction stream.
        const int ns = (kt + 1) & 1;
        const int64_t nk0 = (int64_t)((kt + 1 + rot) % nk) * kTileK;
        read_frags(sa, 0, fa[0], fb[0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3)
                read_frags(sa, s + 1, fa[(s + 1) & 1], fb[(s + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                load_one(ns, nk0, 4 * s + i);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = mfma32<BF>(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    wait_vm_all();

    // Epilogue: the logits, written once (non-temporal), and the records.
    // Per M block i, each value is stored and folded into its row's record
    // together; then a reduce-scatter over the 32 lanes that share rows
    // halves the 16 records per lane at distance d = 16, 8, 4, 2 (a lane
    // keeps the half chosen by its lane bit d and merges in its partner's
    // copy) and merges the last one with lane d = 1.
    const int64_t rowb = m0 + wm * 128 + 4 * hi;
    const int64_t colb = n0 + wn * 128 + (lane & 31u);
    const int64_t rs = 2 * g.tiles_n;
    float2 *rec = reinterpret_cast<float2 *>(g.rec) + 2 * tn + wn;
    // FULL: every row and column of the tile exists (no checks per value).
    auto epilogue = [&](auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        bool cv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            cv[j] = FULL || colb + 32 * j < g.N;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // Keeps the compiler from reading every accumulator into
            // VGPRs at once before the branch (256 of them would spill).
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __asm__ __volatile__("" : "+a"(acc[i][j]));
            float ra[16], rz[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = rowb + i * 32 + 8 * (r / 4) + (r % 4);
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = acc[i][j][r];
                float *cr = g.c + row * g.ldc + colb;
                if (FULL || row < g.M) {
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (cv[j])
                            __builtin_nontemporal_store(v[j], cr + 32 * j);
                }
                if constexpr (STATS) {
                    float m = -INFINITY;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        m = cv[j] ? fmaxf(m, v[j]) : m;
                    float z = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        z += cv[j] ? __expf(v[j] - m) : 0.f;
                    ra[r] = m;
                    rz[r] = z;
                }
            }
            if constexpr (STATS) {
                // 16 records over 32 lanes: halve them at d = 16, 8, 4, 2,
                // then merge the last one with lane d = 1 (both lanes of a
                // pair end with it).
#pragma unroll
                for (int d = 16, n = 8; d >= 2; d >>= 1, n >>= 1) {
                    const bool up = (lane & (uint32_t)d) != 0u;
#pragma unroll
                    for (int h = 0; h < n; ++h) {
                        const float ka = up ? ra[h + n] : ra[h], kz = up ? rz[h + n] : rz[h];
                        const float oa = __shfl_xor(up ? ra[h] : ra[h + n], d);
                        const float oz = __shfl_xor(up ? rz[h] : rz[h + n], d);
                        float m = ka, z = kz;
                        merge_rec(m, z, oa, oz);
                        ra[h] = m;
                        rz[h] = z;
                    }
                }
                {
                    const float oa = __shfl_xor(ra[0], 1), oz = __shfl_xor(rz[0], 1);
                    merge_rec(ra[0], rz[0], oa, oz);
                }
                // lane L (= l % 32) holds accumulator slot r = L / 2: the
                // step at distance d kept the upper half in the lanes with
                // bit d of L set, so r's bit 3 is L's bit 4, ..., r's bit 0
                // is L's bit 1.
                const uint32_t L = lane & 31u;
                const uint32_t r = L >> 1;
                const int64_t row = rowb + i * 32 + 8 * (r / 4) + (r % 4);
                if ((L & 1u) == 0u && (FULL || row < g.M))
                    rec[row * rs] = make_float2(ra[0], rz[0]);
            }
        }
    };
    if (m0 + kTileM <= g.M && n0 + kTileN <= g.N)
        epilogue(std::true_type{});
    else
        epilogue(std::false_type{});
}

hipError_t launch_logits(bool bf, bool stats, const LogitsArgs &a0, hipStream_t st)
{
    LogitsArgs a = a0;
    a.tiles_m = (a.M + kTileM - 1) / kTileM;
    a.tiles_n = (a.N + kTileN - 1) / kTileN;
    const int64_t grid = a.tiles_m * a.tiles_n;
    if (a.M < 1 || a.N < 1 || a.K < 1 || a.K % 8 != 0 || a.lda % kTileK != 0 || a.lda < a.K ||
        (stats && !a.rec) || grid > INT32_MAX)
        return hipErrorInvalidValue;
    const dim3 gd((unsigned)grid), bd(256);
    if (bf) {
        if (stats)
            hipLaunchKernelGGL((logits_kernel<true, true>), gd, bd, 0, st, a);
        else
            hipLaunchKernelGGL((logits_kernel<true, false>), gd, bd, 0, st, a);
    } else {
        if (stats)
            hipLaunchKernelGGL((logits_kernel<false, true>), gd, bd, 0, st, a);
        else
            hipLaunchKernelGGL((logits_kernel<false, false>), gd, bd, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace vl
