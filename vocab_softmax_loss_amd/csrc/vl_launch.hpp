// Internal interface between the C ABI (vl_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vl {

// The order in which a persistent grid visits the rows: the rows in the
// loss range first (index j in [0, n_in)), then the rows outside it
// (j in [0, n_out)).  Row r is in the range iff start <= r mod seq_len < end;
// seq_len <= 0 means every row is.  In-range index j is row
// (j / len_in) * seq_len + start + j % len_in; out-of-range index j is
// position q = j % len_out of sequence j / len_out, where positions
// [0, start) come first and then [end, seq_len).
struct RowWalk {
    int64_t n_in, n_out;
    int64_t seq_len, start, len_in, len_out;
};

// Walks one of the two lists in steps of `stride` without dividing per
// step: (seq, pos) of index j is kept and advanced by the quotient and
// remainder of the stride, computed once.
struct RowCursor {
    int64_t j, seq, pos;      // current index and its (quotient, remainder)
    int64_t len;              // list entries per sequence (len_in or len_out)
    int64_t step_q, step_r;   // stride / len, stride % len

    __host__ __device__ void init(int64_t j0, int64_t stride, int64_t l)
    {
        j = j0;
        len = l > 0 ? l : 1;
        seq = j0 / len;
        pos = j0 % len;
        step_q = stride / len;
        step_r = stride % len;
    }
    __host__ __device__ void advance()
    {
        j += step_q * len + step_r;
        seq += step_q;
        pos += step_r;
        if (pos >= len) {
            pos -= len;
            ++seq;
        }
    }
    __host__ __device__ int64_t in_row(const RowWalk &w) const
    {
        return w.seq_len <= 0 ? j : seq * w.seq_len + w.start + pos;
    }
    __host__ __device__ int64_t out_row(const RowWalk &w) const
    {
        return seq * w.seq_len + (pos < w.start ? pos : pos + w.len_in);
    }
};

// The two lists for `ntok` rows and the range (seq_len, start, end);
// seq_len <= 0: every row is in the loss.
inline RowWalk make_walk(int64_t ntok, int64_t seq_len, int64_t start, int64_t end)
{
    RowWalk w{};
    if (seq_len <= 0) {
        w.n_in = ntok;
        return w;
    }
    w.seq_len = seq_len;
    w.start = start;
    w.len_in = end - start;
    w.len_out = seq_len - w.len_in;
    const int64_t full = ntok / seq_len, rem = ntok % seq_len;
    int64_t last = (rem < end ? rem : end) - start;
    if (last < 0)
        last = 0;
    w.n_in = full * w.len_in + last;
    w.n_out = ntok - w.n_in;
    return w;
}

// One call of the fused CE or KL row kernel.
struct RowArgs {
    void *logits;             // [ntok][V] float32 or bf16, in: logits, out: gradient
    const uint32_t *labels;   // CE: [ntok]
    const uint32_t *ids;      // KL: [ntok][k]
    const float *probs;       // KL: [ntok][k]
    float *loss;              // [ntok]
    float *lse;               // [ntok] or null
    int64_t ntok, V, k;
    RowWalk walk;             // loss range as a row order
    float coef;               // gradient scale
    int64_t lds_vecs;         // online: leading vectors of a row kept in LDS for pass 2
    void *gout;               // out != 0: [ntok][V] half-precision gradient rows
};

// Launch shape of the fused row kernels for a row of V values (16-byte
// vectors of 4 float32 or 8 bf16 values when vec, single elements
// otherwise): block threads x nv vectors hold the row in registers (nv = 0:
// the online variant, which streams it); pf: the next row streams into LDS
// meanwhile; rl: registers are refilled with the next row as the gradient
// is stored; hk: chunks the online float32 variant holds in registers.
struct RowShape {
    int block, nv;
    bool pf, rl;
    int hk;
};

__host__ __device__ inline RowShape row_shape(bool f32, bool vec, int64_t V)
{
    if (!vec)
        return {256, 0, false, false, 0};
    const int64_t nvec = V / (f32 ? 4 : 8);
    if (nvec <= 64)
        return {64, 1, false, false, 0};
    if (nvec <= 128)
        return {64, 2, false, false, 0};
    if (nvec <= 256)
        return {64, 4, false, false, 0};
    if (f32) {
        if (nvec <= 512)
            return {64, 8, false, false, 0};
        if (nvec <= 1024)
            return {256, 4, false, false, 0};
        if (nvec <= 2048)
            return {256, 8, false, false, 0};
        // One block per CU, the next row streaming into LDS.  At V = 32000
        // 1024 threads x 8 vectors run the KL and CE 1.6-2.2% faster than
        // 512 x 16 (the same 128 KB row, twice the waves to hide the
        // reductions' latency).
        if (nvec <= 4096)
            return {512, 8, true, false, 0};
        if (nvec <= 8192)
            return {1024, 8, true, false, 0};
        // Rows past the registers, online: the row's first four chunks (64
        // registers a thread) in registers, the next part in LDS, the rest
        // streamed twice.
        return {1024, 0, false, false, 4};
    }
    // bf16 widens to twice its register footprint: at most 8 vectors (64
    // values) per thread, except with the refill, where one 1024-thread
    // block per CU holds the whole row and refills its registers with the
    // next row as the gradient is stored.
    if (nvec <= 1024)
        return {256, 4, false, false, 0};
    if (nvec <= 4096)
        return {512, 8, true, false, 0};
    if (nvec <= 1024 * 19)
        return {1024, 19, false, true, 0};
    return {1024, 0, false, false, 0};
}

// Vectors per thread per chunk of the online variant (n values a vector).
__host__ __device__ constexpr int online_unroll_n(int n, int hk)
{
    return n == 1 ? 16 : (hk > 0 ? 4 : 8);
}

// Dynamic LDS of a row kernel launch, in this order: [pf: block x nv
// 16-byte slots][KL: two V-bit row bitmaps, 4-word aligned][online: lds_vecs
// 16-byte slots of the current row, whole units of block vectors, after
// the hk held chunks, as many as fit in max_dyn and the row needs].
struct RowLds {
    size_t bitmap_off, lrow_off, bytes;
    int64_t lds_vecs;
};

__host__ __device__ inline RowLds row_lds(const RowShape &sh, bool kl, int64_t V, int n,
                                          size_t raw_bytes, size_t max_dyn)
{
    RowLds L{};
    size_t at = sh.pf ? (size_t)sh.block * (sh.nv > 0 ? sh.nv : 1) * 16 : 0;
    L.bitmap_off = at;
    if (kl)
        at += ((2 * (size_t)((V + 31) >> 5) + 3) & ~size_t(3)) * sizeof(uint32_t);
    L.lrow_off = at;
    L.lds_vecs = 0;
    if (sh.nv == 0) {
        const size_t unit = (size_t)sh.block * raw_bytes;
        const size_t room = at < max_dyn ? (max_dyn - at) / unit : 0;
        const int64_t nvec = V / n;
        const int64_t held = (int64_t)sh.hk * sh.block * online_unroll_n(n, sh.hk);
        const int64_t rest = nvec > held ? nvec - held : 0;
        const int64_t units = (rest + sh.block - 1) / sh.block;
        const int64_t keep = (int64_t)room < units ? (int64_t)room : units;
        L.lds_vecs = keep * sh.block;
        at += (size_t)keep * unit;
    }
    L.bytes = at;
    return L;
}

// Dynamic LDS a row kernel block may take: 160 KB per CU on gfx950, less a
// margin for the kernel's static arrays (under 1 KB).
constexpr size_t kMaxDynLds = 160 * 1024 - 1024;

// One call of the split-row kernels: rows held by S co-resident
// workgroups that swap per-part statistics through a mailbox.
struct SplitArgs {
    RowArgs r;
    uint64_t *mbox;       // groups x S x S x 2 parities x 2 words, cleared before the launch
    int64_t groups;       // row groups of S workgroups each, a multiple of 8
    uint32_t part_vecs;   // 16-byte vectors per part (the last part may be shorter)
    uint32_t spin_limit;  // polls of one exchange before its row is given up (NaN)
    int parts;            // S, workgroups per row
};

// Split kernels.  A part of a row sits in BLOCK threads x NV 16-byte
// vectors of registers; with PF the next row's part streams into LDS
// meanwhile; PER_CU workgroups share a CU.  float32: 1024 x 8 vectors (a
// 128 KB part, the size of a 32000-value row) with the LDS prefetch, one
// workgroup per CU; bf16: 512 x 7 vectors (56 KB) with the LDS prefetch, two
// per CU (8 vectors spill registers in the KL kernel).
struct SplitShape {
    int block, nv;
    bool pf;
    int per_cu;
};
constexpr SplitShape kSplitF32{1024, 8, true, 1};
constexpr SplitShape kSplitBf16{512, 7, true, 2};
// Most parts a row is split into.
constexpr int kMaxSplit = 16;

// Parts a row of V values (N per 16-byte vector) is split into: the fewest
// whose parts fit one workgroup of `shape`, at least 2; 0 when V is not a
// whole number of vectors or more than kMaxSplit parts would be needed.
inline int split_parts_n(int64_t V, int N, const SplitShape &shape)
{
    const int64_t part = (int64_t)shape.block * shape.nv;
    if (V < 1 || V % N != 0)
        return 0;
    const int64_t nvec = V / N;
    int64_t S = (nvec + part - 1) / part;
    if (S < 2)
        S = 2;
    return S <= kMaxSplit ? (int)S : 0;
}

// Workgroup b of a split launch is member `me` of row group `grp`: the
// hardware deals consecutive workgroups to the 8 XCDs in turn, so b, b + 8,
// b + 16, ... share an XCD, and the S members of a group are S of those.
__host__ __device__ inline void split_member(int64_t b, int S, int &me, int64_t &grp)
{
    const int64_t q = b >> 3;
    me = (int)(q % S);
    grp = (b & 7) + 8 * (q / S);
}

// First of the two 64-bit words of mailbox slot (group g, writer w, reader
// r, row parity par).
__host__ __device__ inline int64_t mbox_index(int64_t g, int S, int w, int r, int par)
{
    return ((((g * S) + w) * S + r) * 2 + par) * 2;
}

// The shape of one split launch: N values per 16-byte vector, S parts, the
// kernel shape (with the workgroups per CU that fit) and the CUs.
struct SplitPlan {
    uint32_t part_vecs;   // 16-byte vectors per part (the last part may be shorter)
    int64_t groups;       // a multiple of 8; 0 when the workspace holds too few
    size_t words;         // KL: 32-bit words of one part bitmap
    size_t lds;           // dynamic LDS bytes (PF slots, KL bitmaps)
    int64_t mbox_words;   // 64-bit mailbox words the launch uses
};

inline SplitPlan split_plan(int64_t V, int N, int S, bool kl, const SplitShape &shape, int cus,
                            size_t ws_bytes)
{
    SplitPlan p{};
    const int64_t nvec = V / N;
    p.part_vecs = (uint32_t)((nvec + S - 1) / S);
    p.words = ((size_t)p.part_vecs * (size_t)N + 31) >> 5;
    p.lds = (shape.pf ? (size_t)shape.block * shape.nv * 16 : 0) +
            (kl ? 2 * p.words * sizeof(uint32_t) : 0);
    int64_t groups = (int64_t)shape.per_cu * cus / S / 8 * 8;
    const int64_t ws_groups = (int64_t)(ws_bytes / ((size_t)S * S * 4 * sizeof(uint64_t))) / 8 * 8;
    if (groups > ws_groups)
        groups = ws_groups;
    p.groups = groups < 8 ? 0 : groups;
    p.mbox_words = p.groups * S * S * 4;
    return p;
}

// Polls of one mailbox exchange before the row is given up: far beyond any
// wait among co-resident workgroups (each poll is two atomic round trips
// plus a short sleep, one to two microseconds, so about half a second).
constexpr uint32_t kSplitSpinLimit = 1u << 18;

// Workspace bytes the split-row calls use at most.
constexpr size_t kSplitWorkspaceBytes = 256 * 1024;

// One call of the per-slice KL passes (checked by the caller).
struct SliceArgs {
    void *logits;           // row r of the slice starts at element r * ld
    const uint32_t *ids;    // [ntok][k]
    const float *probs;     // [ntok][k]
    float *part;            // part pass: [ntok][4], 16-byte aligned
    const float *lse;       // gradient pass: [ntok]
    int64_t ntok, ld, off, width, k;
    RowWalk walk;           // loss range as a row order
    float coef;             // gradient scale
};

struct TopkArgs {
    const void *logits;  // [ntok][V]
    int64_t ntok, V, k;
    uint32_t *ids;       // [ntok][k]
    float *probs;        // [ntok][k]
};

// One call of the vocabulary head with the KL (checked by the caller).
struct HeadArgs {
    const float *x;         // [ntok][hs] hidden rows
    const void *w;          // [V][hs] head weights, wdtype
    int wdtype;             // VL_F16 or VL_BF16
    const uint32_t *ids;    // [ntok][k]
    const float *probs;     // [ntok][k]
    float *dx;              // [ntok][hs]
    float *loss;            // [ntok]
    int64_t ntok, V, hs, k, total, chunk;
    float gscale;
    void *scratch;          // head_scratch_bytes(min(chunk, ntok), V, hs) bytes
    bool tune;              // time hipBLASLt's candidates for an untimed shape
};

// Scratch bytes of one head call with `chunk` rows at a time.
size_t head_scratch_bytes(int64_t chunk, int64_t V, int64_t hs);
// Returns a VL_ status.
int head_kl(const HeadArgs &a, hipStream_t stream);

// One call of the teacher-side head (checked by the caller).
struct HeadTopkArgs {
    const float *x;         // [ntok][hs] hidden rows
    const void *w;          // [V][hs] head weights, wdtype
    int wdtype;             // VL_F16 or VL_BF16
    int64_t ntok, V, hs, k, chunk;
    uint32_t *ids;          // [ntok][k]
    float *probs;           // [ntok][k]
    void *scratch;          // head_topk_scratch_bytes(min(chunk, ntok), V, hs) bytes
    bool tune;              // time hipBLASLt's candidates for an untimed shape
};
size_t head_topk_scratch_bytes(int64_t chunk, int64_t V, int64_t hs);
int head_topk(const HeadTopkArgs &a, hipStream_t stream);

// The head's logits product on the matrix cores, with the per-row
// statistics of each 128-column half tile (vl_gemm.hip).
struct LogitsArgs {
    const void *a;              // [M][lda] half hidden rows; zero in columns [K, lda)
    const void *b;              // [N][K] half head weights, rows 16-byte aligned
    float *c;                   // [M][ldc] float32 logits, written
    float *rec;                 // [M][2 tiles_n] (max, sum exp) pairs, or null
    int64_t M, N, K, lda, ldc;  // lda a multiple of 64
    int64_t tiles_m, tiles_n;   // set by the launcher: 256-row and 256-column tiles
};
constexpr int64_t kLogitsTile = 256;
constexpr int64_t kLogitsKStep = 64;
hipError_t launch_logits(bool bf, bool stats, const LogitsArgs &a, hipStream_t stream);

// Each returns hipSuccess or the HIP error of the launch.
// out = 0: the gradient is written over the logits; out = 1 / 2: float32 KL
// rows write it rounded to bf16 / f16 into a.gout and leave the logits.
hipError_t launch_rows(int dtype, bool kl, const RowArgs &a, hipStream_t stream, int out = 0);
hipError_t launch_topk(int dtype, const TopkArgs &a, hipStream_t stream);
// Parts a row of V values is split into (2 to kMaxSplit), or 0 when the
// split kernels do not take it (V not a whole number of 16-byte vectors, or
// a row longer than kMaxSplit parts hold).
int split_parts(int dtype, int64_t V);
// The fused rows split into S parts (S from split_parts), the mailbox in
// `ws` (ws_bytes bytes, cleared first on `stream`); a.logits 16-byte aligned.
hipError_t launch_rows_split(int dtype, bool kl, const RowArgs &a, int S, void *ws,
                             size_t ws_bytes, hipStream_t stream);
// The device address of the library's own kSplitWorkspaceBytes mailbox on
// the current device (looked up once per device).
hipError_t split_scratch(void **ptr);
hipError_t launch_slice_acc(float *dst, const float *src, int64_t n, hipStream_t stream);
// Cross-entropy in two calls, with RowArgs as for launch_rows: the forward
// reads the logits and writes loss and lse (lse may be null); the backward
// reads lse and writes the gradient over the logits (coef is the scale).
hipError_t launch_ce_fwd(int dtype, const RowArgs &a, hipStream_t stream);
hipError_t launch_ce_bwd(int dtype, const RowArgs &a, hipStream_t stream);
// mean[0] = (sum of loss[0..n)) / count, or 0 when count is 0.
hipError_t launch_loss_mean(const float *loss, int64_t n, int64_t count, float *mean,
                            hipStream_t stream);

// The vocabulary-slice KL: per-row statistics of one slice, their merge
// over nslice slices ([nslice][ntok][4]) into loss and lse (lse may be
// null), and one slice's gradient from lse.
hipError_t launch_slice_part(int dtype, const SliceArgs &a, hipStream_t stream);
hipError_t launch_slice_merge(const float *parts, int64_t nslice, int64_t ntok,
                              const RowWalk &walk, float *loss, float *lse, hipStream_t stream);
hipError_t launch_slice_bwd(int dtype, const SliceArgs &a, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cus();

// Resident blocks per CU of kernel `fn` with `block` threads and `lds` bytes
// of dynamic LDS on the current device (at least 1; cached).
int blocks_per_cu(const void *fn, int block, size_t lds);

// Largest KL vocabulary: two row bitmaps of V bits must fit in LDS.
constexpr int64_t kMaxKlVocab = int64_t(1) << 19;
// Largest top-k k.
constexpr int64_t kMaxTopk = 2048;

// Top-k candidate buffer of one wave: the smallest power of two (512 ...
// 4096 entries) that holds k kept entries, one sub-tile of `sub` values
// (64 lanes x one 16-byte vector) and half of max(k, sub) spare.  Without
// the spare a compaction leaves room for no more than one sub-tile, and the
// buffer compacts on nearly every sub-tile that holds a candidate (float32
// k = 256 at V = 151936 in 512 entries: 5.6 ms instead of 1.7).
__host__ __device__ constexpr int topk_cap(int64_t k, int sub)
{
    const int64_t need = k + sub + (k > sub ? k : sub) / 2;
    return need <= 512 ? 512 : need <= 1024 ? 1024 : need <= 2048 ? 2048 : 4096;
}

// Mid-row compactions may stop at a radix bin edge that keeps up to this
// many entries: a quarter of the way from k to the next compaction's
// trigger (cap - sub).
__host__ __device__ constexpr int topk_sel_limit(int k, int cap, int sub)
{
    return k + (cap - sub - k) / 4;
}

}  // namespace vl
