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
// Schedule.  A persistent grid walks the rows in the loss first, then the
// rows outside it, each list strided by the grid size, so every workgroup
// gets the same share of full and write-only rows whatever the range.  One
// workgroup owns one row at a time.  Two variants:
//  * staged (NV > 0): the row sits in registers, NV 16-byte vectors per
//    thread (V <= 32768 float32, V <= 155648 bf16), so it is read from HBM
//    once and written once (1R + 1W).  How the next row's reads overlap the
//    current row depends on the shape: several blocks per CU (small
//    blocks); an asynchronous copy of the next row into LDS (PF, one
//    512- or 1024-thread block per CU); or, for rows that fill a 1024-thread
//    block's registers, each register refilled with the next row's vector
//    right after its gradient is stored (RL).  float32 keeps
//    e = exp(s - m_thread) in place of s and stores e * coef *
//    exp(m_thread - lse): one exp per element.
//  * online (NV == 0): pass 1 keeps a running (max, sum) per thread with
//    one rescale per chunk, pass 2 writes the gradient.  Pass 1 leaves the
//    row's first HK chunks in registers (float32: half of a 128256-value
//    row) and the next vectors, as many as the block's spare LDS holds, in
//    LDS, so pass 2 reads only the rest again; one 1024-thread block per
//    CU keeps the rows in flight small enough for part of that re-read to
//    come from the Infinity Cache.
// (max, sum) pairs reduce across the wave with DPP and across waves through
// LDS, one barrier per row (an LDS-only barrier: it does not wait for the
// prefetched loads); the LDS slots alternate by row parity so a fast wave
// never overwrites partials a slow wave is still reading.
//
// Targets.  CE: the thread that owns the label's vector subtracts coef from
// that element before its store.  KL: the teacher ids of the row are marked
// in an LDS bitmap of V bits and the bulk store skips every vector holding
// one.  The thread that handles id q writes coef (p_id - p_q) there: if it
// is its vector's only mark, it reads that vector's logits back (nothing
// has overwritten them) and writes the whole vector; otherwise the owner
// writes the vector's unmarked elements one by one and q its own.  Every
// element has exactly one writer (no read-modify-write of the gradient).
// The two bitmaps alternate by row parity and are cleared one row late.
// The label (scalar load), ids and probs of the next row are fetched ahead,
// and the logits at the targets are gathered once the current row is done.
//
// Precondition violations are not checked on the device but never fault: a
// label or id >= V gives a NaN loss and no target write.  Teacher entries
// with probability 0 are not targets and may repeat ids; a repeated id with
// a nonzero probability leaves that row's loss and the 16-byte vectors
// holding the id undefined.
#include <math.h>

#include "vl_device.hpp"
#include "vl_launch.hpp"

namespace vl {

// Vectors per thread per chunk of the online variant.
template <int N>
constexpr int online_unroll(int hk = 0)
{
    return online_unroll_n(N, hk);
}

// PF (staged only): stream the next row into an LDS buffer with asynchronous
// global-to-LDS loads while the current row, held in registers, is reduced
// and stored.  Each lane reads back only the 16-byte slots its own loads
// wrote, so the buffer needs no barrier, only this wave's own waits.
// Without PF the occupancy of several blocks per CU provides the overlap.
// Where the gradient goes: over the logits (OUT = 0), or, rounded to bf16
// (OUT = 1) or f16 (OUT = 2), into a separate row-major [ntok][V] buffer
// that the next step reads as a GEMM operand.
template <int DT, bool KL, int BLOCK, int NV, bool VEC, bool PF, bool RL, int HK, int OUT>
struct RowKernel {
    using IO = RowIO<DT, VEC>;
    using Raw = typename IO::Raw;
    static constexpr int N = IO::N;
    static constexpr int NW = BLOCK / kWave;
    static constexpr int U = online_unroll<N>(NV > 0 ? 0 : HK);
    static constexpr int NB = NV > 0 ? NV : 1;
    // Online: the row's first NH chunks of BLOCK x U vectors stay in
    // registers from pass 1 to pass 2; LDS keeps the nlds vectors after them.
    static constexpr int NH = NV > 0 ? 0 : HK;
    static constexpr uint32_t kChunk = (uint32_t)BLOCK * U;
    static constexpr uint32_t kHeld = (uint32_t)NH * kChunk;
    // float32 vectors hold 4 values in 4 registers, so the staged buffer can
    // take exp(s - m) in place of s; bf16 holds 8 values in 4 registers.
    static constexpr bool kKeepExp = (DT == kF32) && VEC && NV > 0;

    struct Tgt {
        uint32_t label;  // CE
        uint32_t id;     // KL: this thread's first teacher entry
        float p;
        float s;         // logit at the label (thread 0) or at id
    };

    const RowArgs &a;
    float (*sh_m)[NW];
    float (*sh_s)[NW];
    float (*sh_l)[NW];
    uint32_t *bitmaps;
    Raw *pf;  // PF: BLOCK x NB vectors, slot v holds vector v of the next row
    // Online: slot v < nlds holds vector v of the current row from pass 1
    // until pass 2 reads it (each slot is written and read by one thread).
    Raw *lrow;
    uint32_t nlds;
    const int tid, wid, lane, words;
    const uint32_t V, nvec, k;
    const float coef;

    __device__ RowKernel(const RowArgs &args, float (*m)[NW], float (*s)[NW], float (*l)[NW],
                         uint32_t *bm, Raw *pfbuf)
        : a(args), sh_m(m), sh_s(s), sh_l(l), bitmaps(bm), pf(pfbuf), tid(threadIdx.x),
          wid(threadIdx.x / kWave), lane(lane_id()), words((int)((args.V + 31) >> 5)),
          V((uint32_t)args.V), nvec((uint32_t)(args.V / IO::N)), k((uint32_t)args.k),
          coef(args.coef)
    {
        lrow = reinterpret_cast<Raw *>(bm + (KL ? ((2 * words + 3) & ~3) : 0));
        nlds = (uint32_t)args.lds_vecs;
    }

    __device__ char *rowp(int64_t row) const
    {
        return reinterpret_cast<char *>(a.logits) + row * (int64_t)V * (int64_t)elt_bytes<DT>();
    }

    __device__ uint32_t clamp_vec(uint32_t v) const { return v < nvec ? v : nvec - 1; }

    // The gradient row of `row` (the logits row itself unless OUT) and its
    // element size.
    static constexpr uint32_t kOutElt = (OUT == 0 && DT == kF32) ? 4u : 2u;
    __device__ char *grow(int64_t row) const
    {
        if constexpr (OUT == 0)
            return rowp(row);
        else
            return reinterpret_cast<char *>(a.gout) + row * (int64_t)V * 2;
    }
    __device__ static void put(char *q, uint32_t vi, const float (&g)[N])
    {
        if constexpr (OUT == 0)
            IO::store(q, vi, g);
        else
            half_store<OUT == 1, N>(q, vi, g);
    }
    __device__ static void put_elem(char *q, uint32_t j, float g)
    {
        if constexpr (OUT == 0)
            IO::store_elem(q, j, g);
        else if constexpr (OUT == 1)
            reinterpret_cast<__bf16 *>(q)[j] = (__bf16)g;
        else
            reinterpret_cast<_Float16 *>(q)[j] = (_Float16)g;
    }

    // Staged rows (NV > 0, always 16-byte vectors) are far below 4 GiB, so
    // vector v is at a 32-bit byte offset from the row base: one offset
    // register per load, with the base in scalar registers.
    __device__ static Raw load_small(const char *p, uint32_t v)
    {
        return *reinterpret_cast<const Raw *>(p + v * (uint32_t)sizeof(Raw));
    }

    // RL: the thread index as a value the compiler cannot see through, so
    // per-row index arithmetic is redone per row (a few adds) instead of
    // being hoisted out of the row loop and kept live, one register pair
    // per vector, beside a row that fills the registers.  Elsewhere the
    // hoisting is cheaper than the recomputation (2.5 us on the 4096 x
    // 32000 KL).
    __device__ uint32_t fresh_tid() const
    {
        uint32_t t = (uint32_t)tid;
        if constexpr (RL || NH > 0)
            __asm__ __volatile__("" : "+v"(t));
        return t;
    }

    // Hide the buffer's contents from the compiler until `dep` is known, so
    // that a pass widens the raw vectors again after the previous pass's
    // result instead of keeping that pass's widened values alive (8
    // registers per bf16 vector instead of 4).
    __device__ static void opaque(Raw (&buf)[NB], float dep)
    {
#pragma unroll
        for (int i = 0; i < NB; ++i)
            __asm__ __volatile__("" : "+v"(buf[i]) : "v"(dep));
    }

    // With a whole long row per thread (RL), the scheduler may not start the
    // next vector of a pass before this one is consumed: interleaving them
    // widens many vectors at once and spills.
    __device__ static void vector_fence()
    {
        if constexpr (RL)
            __builtin_amdgcn_sched_barrier(0);
    }

    // Widen vector v; past the row end every value reads as -inf.
    __device__ void unpack_masked(const Raw &r, uint32_t v, float (&x)[N]) const
    {
        IO::unpack(r, x);
        if (v >= nvec) {
#pragma unroll
            for (int c = 0; c < N; ++c)
                x[c] = -INFINITY;
        }
    }

    // Loads are unconditional (index clamped into the row) and their values
    // unused here, so the loads of a buffer issue back to back and are
    // waited for only where the values are used.
    __device__ void load_row(const char *p, Raw (&buf)[NB]) const
    {
#pragma unroll
        for (int i = 0; i < NB; ++i)
            buf[i] = load_small(p, clamp_vec(tid + (uint32_t)i * BLOCK));
    }

    // Issued early: the label, or this thread's first id and probability.
    __device__ void fetch_targets(int64_t row, Tgt &t) const
    {
        if constexpr (!KL) {
            // Read-only and wave-uniform: through the scalar cache, so the
            // wait for it does not wait for the vector memory queue.
            const __attribute__((address_space(4))) uint32_t *lab =
                (const __attribute__((address_space(4))) uint32_t *)a.labels;
            t.label = lab[row];
        } else {
            t.id = 0xFFFFFFFFu;
            t.p = 0.f;
            if ((uint32_t)tid < k) {
                t.id = a.ids[row * k + tid];
                t.p = a.probs[row * k + tid];
            }
        }
        t.s = 0.f;
    }

    // The logit at the label (CE) or at this thread's teacher id (KL).
    __device__ void gather_s(int64_t row, Tgt &t) const
    {
        const char *p = rowp(row);
        if constexpr (!KL) {
            if (tid == 0 && t.label < V)
                t.s = IO::load_elem(p, t.label);
        } else {
            if ((uint32_t)tid < k && t.id < V)
                t.s = IO::load_elem(p, t.id);
        }
    }

    // KL: the row's marks in bitmap `bm` (cleared by then).  An entry with
    // probability 0 changes neither the loss nor the gradient, so it is not
    // a target: such entries may repeat an id (a padded teacher list).
    __device__ void mark_targets(int64_t row, const Tgt &t, uint32_t *bm) const
    {
        if constexpr (KL) {
            for (uint32_t q = tid; q < k; q += BLOCK) {
                uint32_t id;
                float pq;
                if (q == (uint32_t)tid) {
                    id = t.id;
                    pq = t.p;
                } else {
                    id = a.ids[row * k + q];
                    pq = a.probs[row * k + q];
                }
                if (id < V && pq != 0.f)
                    atomicOr(&bm[id >> 5], 1u << (id & 31));
            }
        }
    }

    // The gradient of one vector, target handling included, and its store
    // into gradient row `p`.
    __device__ void store_vec(char *p, uint32_t v, float (&g)[N], const Tgt &t,
                              const uint32_t *bm) const
    {
        // Staged rows: vector v at a 32-bit byte offset (see load_small).
        char *q = NV > 0 ? p + v * (uint32_t)(N * kOutElt) : p;
        const uint32_t vi = NV > 0 ? 0u : v;  // vector index from q
        if constexpr (!KL) {
            if (t.label < V && v == t.label / N)
                g[t.label % N] -= coef;
            put(q, vi, g);
        } else {
            const uint32_t j0 = v * N;
            const uint32_t bits = (bm[j0 >> 5] >> (j0 & 31)) & (uint32_t)((1ull << N) - 1);
            if (bits == 0u) {
                put(q, vi, g);
            } else if (__builtin_popcount(bits) > 1) {  // one target: its thread writes it all
#pragma unroll
                for (int c = 0; c < N; ++c)
                    if (!((bits >> c) & 1u))
                        put_elem(q, vi * N + c, g[c]);
            }
        }
    }

    // Online pass 1: fold one chunk of U vectors (v0 + u BLOCK) into the
    // thread's running (max, sum) with a single rescale.
    __device__ void online_chunk(const Raw (&y)[U], uint32_t v0, float &m, float &s) const
    {
        float cm = -INFINITY;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[N];
            unpack_masked(y[u], v0 + (uint32_t)u * BLOCK, x);
#pragma unroll
            for (int c = 0; c < N; ++c)
                cm = fmaxf(cm, x[c]);
        }
        const float mn = fmaxf(m, cm);
        if (mn != -INFINITY) {
            float acc = s * __expf(m - mn);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float x[N];
                unpack_masked(y[u], v0 + (uint32_t)u * BLOCK, x);
#pragma unroll
                for (int c = 0; c < N; ++c)
                    acc += __expf(x[c] - mn);
            }
            s = acc;
            m = mn;
        }
    }

    // Online pass 2: the gradient of one chunk and its stores.
    __device__ void store_chunk(char *p, const Raw (&y)[U], uint32_t v0, float lse, const Tgt &t,
                                const uint32_t *bm) const
    {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t v = v0 + (uint32_t)u * BLOCK;
            if (v < nvec) {
                float x[N], g[N];
                IO::unpack(y[u], x);
#pragma unroll
                for (int c = 0; c < N; ++c)
                    g[c] = coef * __expf(x[c] - lse);
                store_vec(p, v, g, t, bm);
            }
        }
    }

    // One in-range row: reduce, loss, gradient.  `buf` holds the row when
    // staged; with RL each register is refilled with the next row's vector
    // as soon as its own gradient is stored.  Afterwards the next row's
    // targets are gathered into `tn`.
    __device__ void process(int64_t row, Raw (&buf)[NB], Tgt &t, int par, bool has_next,
                            int64_t nrow, Tgt &tn) const
    {
        char *p = rowp(row);
        char *gw = grow(row);
        uint32_t *bm = bitmaps + par * words;
        uint32_t *bm_other = bitmaps + (par ^ 1) * words;
        const uint32_t t0 = fresh_tid();
        Raw hold[NH > 0 ? NH : 1][U];  // online: the row's first NH chunks

        // ---- pass 1: thread-local (max, sum of exp)
        float m = -INFINITY, s = 0.f;
        if constexpr (NV > 0) {
            // Vectors past the row end hold a copy of its last vector (the
            // loads are clamped): harmless to the max, left out of the sum.
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float x[N];
                IO::unpack(buf[i], x);
#pragma unroll
                for (int c = 0; c < N; ++c)
                    m = fmaxf(m, x[c]);
                vector_fence();
            }
            const float ms = (m == -INFINITY) ? 0.f : m;
            if constexpr (!kKeepExp)
                opaque(buf, ms);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                float x[N];
                IO::unpack(buf[i], x);
                float es = 0.f;
#pragma unroll
                for (int c = 0; c < N; ++c) {
                    const float e = __expf(x[c] - ms);
                    es += e;
                    if constexpr (kKeepExp)
                        buf[i][c] = __builtin_bit_cast(uint32_t, e);
                }
                s += (t0 + (uint32_t)i * BLOCK < nvec) ? es : 0.f;
                vector_fence();
            }
        } else {
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                const uint32_t v0 = t0 + (uint32_t)h * kChunk;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    hold[h][u] = IO::load_raw(p, clamp_vec(v0 + (uint32_t)u * BLOCK));
                online_chunk(hold[h], v0, m, s);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    __asm__ __volatile__("" : "+v"(hold[h][u]) : "v"(s));
            }
            for (uint32_t v0 = t0 + kHeld; v0 < nvec; v0 += kChunk) {
                Raw y[U];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    y[u] = IO::load_raw(p, clamp_vec(v0 + (uint32_t)u * BLOCK));
                // nlds is a multiple of BLOCK: each test is uniform
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (v0 - kHeld + (uint32_t)u * BLOCK < nlds)
                        lrow[v0 - kHeld + (uint32_t)u * BLOCK] = y[u];
                online_chunk(y, v0, m, s);
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
        block_sync_lds();
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
                a.loss[row] = (t.label < V) ? (M - t.s) + logS : NAN;
                if (a.lse)
                    a.lse[row] = lse;
            }
        } else {
            // The previous row's marks: every thread is past that row's stores.
            for (int i = tid; i < words; i += BLOCK)
                bm_other[i] = 0u;
            float acc = 0.f;
            for (uint32_t q = tid; q < k; q += BLOCK) {
                uint32_t id;
                float pq, sv = 0.f;
                if (q == (uint32_t)tid) {
                    id = t.id;
                    pq = t.p;
                    sv = t.s;
                } else {
                    id = a.ids[row * k + q];
                    pq = a.probs[row * k + q];
                    if (id < V)
                        sv = IO::load_elem(p, id);
                }
                if (id >= V) {
                    acc = NAN;
                    continue;
                }
                const float d = (sv - M) - logS;  // log p_S at the id
                if (pq > 0.f)
                    acc += pq * (__logf(pq) - d);
                if (pq == 0.f)
                    continue;  // not a target (not marked)
                const float gid = coef * (__expf(d) - pq);
                if constexpr (N > 1) {
                    const uint32_t v = id / N, j0 = v * N;
                    const uint32_t vb = (bm[j0 >> 5] >> (j0 & 31)) & (uint32_t)((1ull << N) - 1);
                    if (__builtin_popcount(vb) == 1) {
                        // The vector's only target: this thread writes the
                        // whole vector (its owner skips it), from the row's
                        // values, which nothing has overwritten.
                        float x[N], g[N];
                        IO::unpack(IO::load_raw(p, v), x);
#pragma unroll
                        for (int c = 0; c < N; ++c)
                            g[c] = (uint32_t)c == id - j0 ? gid : coef * __expf(x[c] - lse);
                        put(gw, v, g);
                        continue;
                    }
                }
                put_elem(gw, id, gid);
            }
            const float wl = wave_sum(acc);
            if (lane == 0)
                sh_l[par][wid] = wl;
            block_sync_lds();
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
        if constexpr (NV > 0) {
            // float32 keeps e = exp(s - m_thread) in the buffer: one exp per
            // element, p = e exp(m_thread - lse).
            const float cf = coef * __expf(((m == -INFINITY) ? 0.f : m) - lse);
            const char *np = rowp(nrow);
            if constexpr (!kKeepExp)
                opaque(buf, lse);
            const uint32_t t1 = fresh_tid();  // indices not kept from pass 1
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const uint32_t v = t1 + (uint32_t)i * BLOCK;
                if (v < nvec) {
                    float x[N], g[N];
                    IO::unpack(buf[i], x);
#pragma unroll
                    for (int c = 0; c < N; ++c)
                        g[c] = kKeepExp ? x[c] * cf : coef * __expf(x[c] - lse);
                    store_vec(gw, v, g, t, bm);
                }
                if constexpr (RL) {
                    // Not before this vector's store: the register is the
                    // one being freed (hoisted loads would need a second
                    // row's worth of registers).
                    __asm__ __volatile__("" ::: "memory");
                    if (has_next)
                        buf[i] = load_small(np, clamp_vec(v));
                }
                vector_fence();
            }
        } else {
#pragma unroll
            for (int h = 0; h < NH; ++h) {
                // widened again here, not kept widened from pass 1
#pragma unroll
                for (int u = 0; u < U; ++u)
                    __asm__ __volatile__("" : "+v"(hold[h][u]) : "v"(lse));
                store_chunk(gw, hold[h], fresh_tid() + (uint32_t)h * kChunk, lse, t, bm);
            }
            for (uint32_t v0 = fresh_tid() + kHeld; v0 < nvec; v0 += kChunk) {
                Raw y[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t v = v0 + (uint32_t)u * BLOCK;
                    y[u] = v - kHeld < nlds ? lrow[v - kHeld] : IO::load_raw(p, clamp_vec(v));
                }
                store_chunk(gw, y, v0, lse, t, bm);
            }
        }

        if (has_next) {
            mark_targets(nrow, tn, bm_other);
            gather_s(nrow, tn);
        }
    }

    __device__ void zero_row(int64_t row) const
    {
        char *p = grow(row);
        float z[N];
#pragma unroll
        for (int c = 0; c < N; ++c)
            z[c] = 0.f;
        for (uint32_t v = tid; v < nvec; v += BLOCK)
            put(p, v, z);
        if (tid == 0) {
            a.loss[row] = 0.f;
            if (a.lse)
                a.lse[row] = 0.f;
        }
    }

    // PF: issue the asynchronous loads of `row` into this lane's LDS slots.
    __device__ void prefetch_row(int64_t row) const
    {
        const char *p = rowp(row);
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const uint32_t v = tid + (uint32_t)i * BLOCK;
            load_to_lds16(p + clamp_vec(v) * (uint32_t)sizeof(Raw),
                          pf + (uint32_t)i * BLOCK + (uint32_t)wid * kWave);
        }
    }

    // Process `row` (its targets in tc).  Staged: with PF the row is taken
    // from this lane's LDS slots (filled during the previous step) and the
    // next row's loads are issued into them; without PF it is loaded here.
    // Returns whether a next row exists.
    // One row; tc holds its targets and receives the next row's, which
    // are fetched into tn.
    __device__ bool step(RowCursor &cur_pos, int64_t &row, Raw (&cur)[NB], Tgt &tc, Tgt &tn,
                         int &par) const
    {
        const RowWalk &w = a.walk;
        RowCursor nc = cur_pos;
        nc.advance();
        const bool has_next = nc.j < w.n_in;
        const int64_t nrow = has_next ? nc.in_row(w) : row;
        if constexpr (NV > 0 && PF) {
            wait_vm_all();  // this row's loads into LDS (and all older)
#pragma unroll
            for (int i = 0; i < NB; ++i)
                cur[i] = pf[tid + (uint32_t)i * BLOCK];
            wait_lds_all();  // read before the slots are refilled
            if (has_next)
                prefetch_row(nrow);
        }
        fetch_targets(nrow, tn);
        if constexpr (NV > 0 && !PF && !RL)
            load_row(rowp(row), cur);
        process(row, cur, tc, par, has_next, nrow, tn);
        par ^= 1;
        cur_pos = nc;
        row = nrow;
        tc = tn;
        return has_next;
    }

    __device__ void run()
    {
        const RowWalk &w = a.walk;
        if constexpr (KL) {
            for (int i = tid; i < 2 * words; i += BLOCK)
                bitmaps[i] = 0u;
            block_sync_lds();
        }
        RowCursor c;
        c.init(blockIdx.x, gridDim.x, w.len_in);
        if (c.j < w.n_in) {
            Raw buf[NB];
            Tgt ta, tb;
            int par = 0;
            int64_t row = c.in_row(w);
            fetch_targets(row, ta);
            if constexpr (NV > 0 && PF)
                prefetch_row(row);
            if constexpr (RL)
                load_row(rowp(row), buf);
            mark_targets(row, ta, bitmaps);
            gather_s(row, ta);
            while (step(c, row, buf, ta, tb, par)) {
            }
        }
        RowCursor o;
        o.init(blockIdx.x, gridDim.x, w.len_out);
        for (; o.j < w.n_out; o.advance())
            zero_row(o.out_row(w));
    }
};

// Waves per SIMD the register allocation must allow.  Staged blocks of 512
// and 256 threads without prefetch rely on two and three resident blocks
// per CU for their overlap; the others run one 1024-thread block per CU.
template <int BLOCK, int NV, bool PF>
constexpr int min_waves_per_simd()
{
    if (NV > 0 && !PF && BLOCK == 512)
        return 4;
    if (NV > 0 && !PF && BLOCK == 256)
        return 3;
    return 1;
}

template <int DT, bool KL, int BLOCK, int NV, bool VEC, bool PF, bool RL, int HK, int OUT>
__global__ __launch_bounds__(BLOCK, (min_waves_per_simd<BLOCK, NV, PF>())) void row_loss_kernel(
    RowArgs a)
{
    constexpr int NW = BLOCK / kWave;
    __shared__ float sh_m[2][NW];
    __shared__ float sh_s[2][NW];
    __shared__ float sh_l[2][NW];
    // Dynamic LDS: [PF: BLOCK x NV 16-byte slots][KL: 2 x ceil(V/32) words]
    extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
    using K = RowKernel<DT, KL, BLOCK, NV, VEC, PF, RL, HK, OUT>;
    constexpr uint32_t pf_words = PF ? (uint32_t)BLOCK * (NV > 0 ? NV : 1) * 4 : 0;
    K k(a, sh_m, sh_s, sh_l, dyn + pf_words, reinterpret_cast<typename K::Raw *>(dyn));
    k.run();
}

// ------------------------------------------------------------------ launch

namespace {

template <int OUT, int DT, bool KL, int BLOCK, int NV, bool VEC, bool PF = false,
          bool RL = false, int HK = 0>
hipError_t launch_one(const RowArgs &a, hipStream_t st)
{
    auto fn = row_loss_kernel<DT, KL, BLOCK, NV, VEC, PF, RL, HK, OUT>;
    RowArgs args = a;
    // Online: after the HK chunks held in registers, the rest of LDS keeps
    // the row's next vectors, in units of BLOCK, for pass 2, which reads
    // them from there instead of HBM.  Those are the first read in pass 1,
    // the least likely to be still cached.
    const RowLds L = row_lds(RowShape{BLOCK, NV, PF, RL, HK}, KL, a.V, RowIO<DT, VEC>::N,
                             sizeof(typename RowIO<DT, VEC>::Raw), kMaxDynLds);
    const size_t lds = L.bytes;
    args.lds_vecs = L.lds_vecs;
    if (lds > kMaxDynLds)
        return hipErrorInvalidValue;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void *)fn,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    int per_cu = blocks_per_cu((const void *)fn, BLOCK, lds);
    if (NV == 0 && per_cu > 1)
        per_cu = 1;  // online: keep the rows in flight inside the Infinity Cache
    const int64_t rows = a.walk.n_in > a.walk.n_out ? a.walk.n_in : a.walk.n_out;
    int64_t grid = (int64_t)per_cu * device_cus();
    if (grid > rows)
        grid = rows;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(BLOCK), lds, st, args);
    return hipGetLastError();
}

// The instantiation of the shape row_shape picks (its table, in
// vl_launch.hpp, is the one place the shapes are chosen).
template <int DT, bool KL, int OUT>
hipError_t launch_dt(const RowArgs &a, hipStream_t st, bool vec)
{
    const RowShape s = row_shape(DT == kF32, vec, a.V);
    auto is = [&](int block, int nv, bool pf, bool rl, int hk) {
        return s.block == block && s.nv == nv && s.pf == pf && s.rl == rl && s.hk == hk;
    };
    if (!vec)
        return is(256, 0, false, false, 0) ? launch_one<OUT, DT, KL, 256, 0, false>(a, st)
                                           : hipErrorInvalidValue;
    if (is(64, 1, false, false, 0))
        return launch_one<OUT, DT, KL, 64, 1, true>(a, st);
    if (is(64, 2, false, false, 0))
        return launch_one<OUT, DT, KL, 64, 2, true>(a, st);
    if (is(64, 4, false, false, 0))
        return launch_one<OUT, DT, KL, 64, 4, true>(a, st);
    if (is(256, 4, false, false, 0))
        return launch_one<OUT, DT, KL, 256, 4, true>(a, st);
    if (is(512, 8, true, false, 0))
        return launch_one<OUT, DT, KL, 512, 8, true, true>(a, st);
    if constexpr (DT == kF32) {
        if (is(64, 8, false, false, 0))
            return launch_one<OUT, DT, KL, 64, 8, true>(a, st);
        if (is(256, 8, false, false, 0))
            return launch_one<OUT, DT, KL, 256, 8, true>(a, st);
        if (is(1024, 8, true, false, 0))
            return launch_one<OUT, DT, KL, 1024, 8, true, true>(a, st);
        if (is(1024, 0, false, false, 4))
            return launch_one<OUT, DT, KL, 1024, 0, true, false, false, 4>(a, st);
    } else {
        if (is(1024, 19, false, true, 0))
            return launch_one<OUT, DT, KL, 1024, 19, true, false, true>(a, st);
        if (is(1024, 0, false, false, 0))
            return launch_one<OUT, DT, KL, 1024, 0, true>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_rows(int dtype, bool kl, const RowArgs &a, hipStream_t st, int out)
{
    const size_t elt = dtype == kF32 ? 4 : 2;
    const int n = 16 / (int)elt;
    bool vec = ((uintptr_t)a.logits % 16 == 0) && (a.V % n == 0);
    if (out != 0) {
        // half-precision gradient rows: float32 KL rows only; vector stores
        // of 4 halves need 8-byte aligned output rows
        if (dtype != kF32 || !kl || !a.gout)
            return hipErrorInvalidValue;
        vec = vec && ((uintptr_t)a.gout % 8 == 0);
        return out == 1 ? launch_dt<kF32, true, 1>(a, st, vec) : launch_dt<kF32, true, 2>(a, st, vec);
    }
    if (dtype == kF32)
        return kl ? launch_dt<kF32, true, 0>(a, st, vec) : launch_dt<kF32, false, 0>(a, st, vec);
    return kl ? launch_dt<kBF16, true, 0>(a, st, vec) : launch_dt<kBF16, false, 0>(a, st, vec);
}

}  // namespace vl
