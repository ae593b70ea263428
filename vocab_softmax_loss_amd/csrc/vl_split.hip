// Rows longer than one compute unit holds, split over S co-resident
// workgroups: the fused cross-entropy or distillation KL of each row with
// the row read once and written once (1R + 1W).
//
// What a row computes is that of vl_rows.hip (cortiq-engine train_head.rs,
// module doc and kl_rows; aprender-train wgpu_cross_entropy.rs, module doc
// and backward): lse = ln sum_j exp(s_j), the loss against a label or the
// teacher's (id, p) entries, and the gradient coef (exp(s - lse) - t) over
// the logits.  The cortiq page cuts a vocabulary into column slices (Head);
// here the S workgroups of a group each hold one contiguous column part of
// the row in registers and combine per-part statistics, the way the
// vocabulary-slice KL merges its slices:
//   part i:   a_i = max over the part, z_i = sum exp(s - a_i),
//             P_i = sum of the teacher p > 0 whose id falls in the part,
//             w_i = sum of those p (ln p - (s_id - a_i))
//   row:      lse = ln sum_i z_i exp(a_i),  loss = sum_i w_i + P_i (lse - a_i)
// (cross-entropy is the case of one entry with p = 1).
//
// Schedule.  One cooperative launch, every workgroup resident (a
// persistent grid of two 512-thread workgroups per CU).  Workgroup b is
// member (b / 8) % S of group 8 (b / (8 S)) + b % 8: the hardware deals
// consecutive workgroups to the 8 XCDs in turn, so the S members of a group
// share one XCD and its L2.  A group walks its share of the rows in the
// loss range (the balanced row order of vl_launch.hpp, strided by the number
// of groups); the rows outside the range are zeroed by every workgroup,
// whole rows strided by the grid, without any exchange.  Each member holds
// its part in registers (NV 16-byte vectors per thread), reduces it, and
// swaps its 16-byte record with the other members through a mailbox in the
// caller's workspace; all members form the same lse from the S records in
// member order, write their part of the gradient from registers, and reload
// each register with the next row's vector right after its store (so the
// next row's reads overlap this row's writes, and the second workgroup on
// the CU streams while this one reduces or waits).
//
// Mailbox.  Slot (group, writer, reader, row parity) holds two 64-bit words,
// each 0 when empty and the bitwise complement of (value bits, value bits)
// when full, so a published word is never 0.  A writer stores its words with
// relaxed device-scope atomic stores; the reader takes them with device-scope
// atomic exchanges against 0, which return the record and leave the slot
// empty.  A slot is reused two rows later, by which time its reader has
// taken it: the writer reaches row r + 2 only after reading the reader's
// record of row r + 1, which the reader publishes only after its exchange
// for row r has returned.  Every wait is bounded (spin_limit polls, and a
// single poll once one wait of the workgroup has timed out): a row whose
// exchange times out gets a NaN loss, lse and gradient, and the kernel still
// ends.  The host clears the mailbox before every launch.
//
// Targets.  As in vl_rows.hip: the label's owner subtracts coef before its
// store; KL ids with a nonzero probability are marked in an LDS bitmap of
// the part's columns (two, alternating by row parity), the bulk store skips
// every vector holding a mark, and the thread of id q writes
// coef (p_S(id) - p_q) -- the whole vector when it is the vector's only mark
// (reading its logits back from the row, which nothing has overwritten),
// else only that element while the owner writes the vector's others.
#include <math.h>

#include <mutex>

#include "vl_device.hpp"
#include "vl_launch.hpp"

namespace vl {

namespace {

__device__ __forceinline__ uint64_t *mbox_slot(uint64_t *mb, int64_t g, int S, int w, int r,
                                               int par)
{
    return mb + mbox_index(g, S, w, r, par);
}

__device__ __forceinline__ uint64_t pack_pair(float lo, float hi)
{
    return ~(((uint64_t)__float_as_uint(hi) << 32) | (uint64_t)__float_as_uint(lo));
}

__device__ __forceinline__ void unpack_pair(uint64_t w, float &lo, float &hi)
{
    const uint64_t v = ~w;
    lo = __uint_as_float((uint32_t)v);
    hi = __uint_as_float((uint32_t)(v >> 32));
}

}  // namespace

template <int DT, bool KL, int BLOCK, int NV, bool PF>
struct SplitKernel {
    using IO = RowIO<DT, true>;
    using Raw = typename IO::Raw;
    static constexpr int N = IO::N;
    static constexpr int NW = BLOCK / kWave;
    // e = exp(s - m_thread) is kept for the store, so each value takes one
    // exponential: float32 in place of s (4 values in 4 registers), bf16 with
    // the LDS prefetch in registers of its own (8 values widen to 8
    // registers; the raw vectors are free once e is formed, since the next
    // row arrives in LDS).  bf16 refilling its registers recomputes e.
    static constexpr bool kKeepExp = DT == kF32 || PF;
    static constexpr bool kOwnExp = kKeepExp && DT != kF32;

    struct Tgt {
        uint32_t label;  // CE
        uint32_t id;     // KL: this thread's first teacher entry
        float p;
        float s;         // logit at the label (thread 0) or at id, if in the part
    };

    const SplitArgs &A;
    const RowArgs &a;
    float (*sh_m)[NW];
    float (*sh_s)[NW];
    float (*sh_w)[NW];
    float (*sh_P)[NW];
    float (*sh_x)[2];  // per parity: lse, loss
    uint32_t *bitmaps;
    Raw *pf;  // PF: BLOCK x NV slots; slot v holds local vector v of the next row's part
    const int tid, wid, lane, words, S;
    int me;
    int64_t grp;
    const uint32_t V, nvec, k;
    uint32_t vbeg, np, c0, c1;  // this part: vectors [vbeg, vbeg + np), columns [c0, c1)
    const float coef;
    // Wave 0, after an exchange timed out: later exchanges poll only once,
    // so a workgroup whose partners never come still ends promptly.
    bool broken = false;

    __device__ SplitKernel(const SplitArgs &sa, float (*m)[NW], float (*s)[NW], float (*w)[NW],
                           float (*P)[NW], float (*x)[2], uint32_t *bm, Raw *pfbuf)
        : A(sa), a(sa.r), sh_m(m), sh_s(s), sh_w(w), sh_P(P), sh_x(x), bitmaps(bm), pf(pfbuf),
          tid(threadIdx.x), wid(threadIdx.x / kWave), lane(lane_id()),
          words((int)((sa.part_vecs * (uint32_t)N + 31) >> 5)), S(sa.parts), V((uint32_t)sa.r.V),
          nvec((uint32_t)(sa.r.V / N)), k((uint32_t)sa.r.k), coef(sa.r.coef)
    {
        split_member(blockIdx.x, S, me, grp);
        vbeg = (uint32_t)me * sa.part_vecs;
        const uint32_t vend = vbeg + sa.part_vecs < nvec ? vbeg + sa.part_vecs : nvec;
        np = vend > vbeg ? vend - vbeg : 0u;
        c0 = vbeg * (uint32_t)N;
        c1 = vend * (uint32_t)N;
    }

    __device__ char *rowp(int64_t row) const
    {
        return reinterpret_cast<char *>(a.logits) + row * (int64_t)V * (int64_t)elt_bytes<DT>();
    }

    __device__ bool in_part(uint32_t id) const { return id >= c0 && id < c1; }

    // exp(x - a) as 2^(x log2(e) - al) with al = a log2(e): one fused
    // multiply-add and one v_exp_f32.  A thread uses the same al for every
    // value it anchors at a, so its values and their sum share the one
    // rounding of al.
    static constexpr float kLog2e = 1.44269504088896341f;
    __device__ static float exp_shifted(float x, float al)
    {
        return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -al));
    }

    // The thread index as a value the compiler cannot see through, so that
    // per-vector addresses are recomputed per row instead of held across the
    // row loop beside a part that fills the registers.
    __device__ uint32_t fresh_tid() const
    {
        uint32_t t = (uint32_t)tid;
        __asm__ __volatile__("" : "+v"(t));
        return t;
    }

    __device__ static void opaque(Raw (&buf)[NV], float dep)
    {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            __asm__ __volatile__("" : "+v"(buf[i]) : "v"(dep));
    }

    // Local vector lv of the part, clamped into it (loads past the part's
    // end re-read its last vector; such slots are left out of the sum).
    __device__ uint32_t clamp_local(uint32_t lv) const { return lv < np ? lv : np - 1; }

    __device__ Raw load_part(const char *p, uint32_t lv) const
    {
        return *reinterpret_cast<const Raw *>(p + (vbeg + clamp_local(lv)) * (uint32_t)sizeof(Raw));
    }

    __device__ void load_row(const char *p, Raw (&buf)[NV]) const
    {
        const uint32_t t = fresh_tid();
#pragma unroll
        for (int i = 0; i < NV; ++i)
            buf[i] = load_part(p, t + (uint32_t)i * BLOCK);
    }

    // PF: the asynchronous loads of `row`'s part into this lane's LDS slots
    // (lane l of a wave lands at the wave's base slot + l, so each lane later
    // reads back exactly the slots its own loads filled).
    __device__ void prefetch_row(int64_t row) const
    {
        const char *p = rowp(row);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const uint32_t lv = (uint32_t)tid + (uint32_t)i * BLOCK;
            load_to_lds16(p + (vbeg + clamp_local(lv)) * (uint32_t)sizeof(Raw),
                          pf + (uint32_t)i * BLOCK + (uint32_t)wid * kWave);
        }
    }

    __device__ void fetch_targets(int64_t row, Tgt &t) const
    {
        if constexpr (!KL) {
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

    // The logit at the label or at this thread's id, when it lies in the part.
    __device__ void gather_s(int64_t row, Tgt &t) const
    {
        const char *p = rowp(row);
        if constexpr (!KL) {
            if (tid == 0 && in_part(t.label))
                t.s = IO::load_elem(p, t.label);
        } else {
            if ((uint32_t)tid < k && in_part(t.id) && t.p != 0.f)
                t.s = IO::load_elem(p, t.id);
        }
    }

    // KL: the part's targets (ids with a nonzero probability) in `bm`.
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
                if (in_part(id) && pq != 0.f) {
                    const uint32_t j = id - c0;
                    atomicOr(&bm[j >> 5], 1u << (j & 31));
                }
            }
        }
    }

    // The gradient of part vector v (global vector index), target handling
    // included, and its store.
    __device__ void store_vec(char *p, uint32_t v, float (&g)[N], const Tgt &t,
                              const uint32_t *bm) const
    {
        char *q = p + v * (uint32_t)sizeof(Raw);
        if constexpr (!KL) {
            if (t.label < V && v == t.label / N)
                g[t.label % N] -= coef;
            IO::store(q, 0, g);
        } else {
            const uint32_t j0 = v * N - c0;
            const uint32_t bits = (bm[j0 >> 5] >> (j0 & 31)) & (uint32_t)((1ull << N) - 1);
            if (bits == 0u) {
                IO::store(q, 0, g);
            } else if (__builtin_popcount(bits) > 1) {  // one target: its thread writes it all
#pragma unroll
                for (int c = 0; c < N; ++c)
                    if (!((bits >> c) & 1u))
                        IO::store_elem(q, c, g[c]);
            }
        }
    }

    // Swap this part's record with the other members' (wave 0): lane i < S
    // takes member i's record (its own at lane me), then the S records merge
    // across the lanes -- the same reduction tree in every member, so every
    // member forms the same lse bits.  Leaves (lse, loss) in sh_x[par].
    __device__ void exchange(int par, float pa, float pz, float pw, float pP)
    {
        float ra = pa, rz = pz, rw = pw, rP = pP;
        bool ok = true;
        if (lane < S && lane != me) {
            uint64_t *out = mbox_slot(A.mbox, grp, S, me, lane, par);
            uint64_t *in = mbox_slot(A.mbox, grp, S, lane, me, par);
            __hip_atomic_store(out, pack_pair(pa, pz), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(out + 1, pack_pair(pw, pP), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            uint64_t u0 = 0, u1 = 0;
            const uint32_t limit = broken ? 0u : A.spin_limit;
            for (uint32_t it = 0;; ++it) {
                if (u0 == 0)
                    u0 = __hip_atomic_exchange(in, (uint64_t)0, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                if (u1 == 0)
                    u1 = __hip_atomic_exchange(in + 1, (uint64_t)0, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                if ((u0 != 0 && u1 != 0) || it >= limit)
                    break;
                __builtin_amdgcn_s_sleep(2);
            }
            ok = u0 != 0 && u1 != 0;
            unpack_pair(u0, ra, rz);
            unpack_pair(u1, rw, rP);
        }
        const bool bad = ballot(!ok) != 0;
        broken = broken || bad;
        // parts with no finite value (sum 0) are left out; a NaN sum is kept
        const bool live = lane < S && !(rz <= 0.f);
        const float M = wave_max(live ? ra : -INFINITY);
        const float Z = wave_sum(live ? rz * __expf(ra - M) : 0.f);
        float lse = M + __logf(Z);
        float term = 0.f;
        if (lane < S)
            term = (rw != rw) ? NAN : (rP > 0.f ? rw + rP * (lse - ra) : 0.f);
        float loss = wave_sum(term);
        if (bad) {
            lse = NAN;
            loss = NAN;
        }
        if (lane == 0) {
            sh_x[par][0] = lse;
            sh_x[par][1] = loss;
        }
    }

    // One in-range row; `buf` holds its part and is refilled with the next
    // row's part as the gradient is stored.
    __device__ void process(int64_t row, Raw (&buf)[NV], Tgt &t, int par, bool has_next,
                            int64_t nrow, Tgt &tn)
    {
        char *p = rowp(row);
        uint32_t *bm = bitmaps + par * words;
        uint32_t *bm_other = bitmaps + (par ^ 1) * words;
        const uint32_t t0 = fresh_tid();

        // ---- thread-local (max, sum of exp) over the held vectors (bf16 with
        // PF: read from this lane's LDS slots; only e is kept in registers)
        float ex[kOwnExp ? NV : 1][N];
        float m = -INFINITY, s = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float x[N];
            IO::unpack(kOwnExp ? pf[t0 + (uint32_t)i * BLOCK] : buf[i], x);
#pragma unroll
            for (int c = 0; c < N; ++c)
                m = fmaxf(m, x[c]);
            __builtin_amdgcn_sched_barrier(0);
        }
        const float ms = (m == -INFINITY) ? 0.f : m;
        const float msl = ms * kLog2e;
        if constexpr (!kKeepExp)
            opaque(buf, ms);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            float x[N];
            IO::unpack(kOwnExp ? pf[t0 + (uint32_t)i * BLOCK] : buf[i], x);
            float es = 0.f;
#pragma unroll
            for (int c = 0; c < N; ++c) {
                const float e = exp_shifted(x[c], msl);
                es += e;
                if constexpr (kOwnExp)
                    ex[i][c] = e;
                else if constexpr (kKeepExp)
                    buf[i][c] = __builtin_bit_cast(uint32_t, e);
            }
            s += (t0 + (uint32_t)i * BLOCK < np) ? es : 0.f;
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kOwnExp) {
            wait_lds_all();  // the slots are read: refill them with the next row
            if (has_next && wid != 0)
                prefetch_row(nrow);
        }

        // ---- the part's (max, sum): one barrier
        {
            const float wm = wave_max(m);
            // s is anchored at msl = m log2(e); rescale it to wm in the same units
            const float sc = (m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f(msl - wm * kLog2e);
            const float ws = wave_sum(sc);
            if (lane == 0) {
                sh_m[par][wid] = wm;
                sh_s[par][wid] = ws;
            }
        }
        block_sync_lds();
        float Mp = -INFINITY;
#pragma unroll
        for (int i = 0; i < NW; ++i)
            Mp = fmaxf(Mp, sh_m[par][i]);
        float Zp = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const float mi = sh_m[par][i];
            Zp += (mi == -INFINITY) ? 0.f
                                    : sh_s[par][i] * __builtin_amdgcn_exp2f(mi * kLog2e - Mp * kLog2e);
        }
        // a part without a finite value: (a, z) = (0, 0), left out of the lse
        const float pa = (Mp == -INFINITY) ? 0.f : Mp;
        const float pz = (Mp == -INFINITY) ? 0.f : Zp;

        // ---- the part's teacher terms, anchored at its max
        float pw = 0.f, pP = 0.f;
        if constexpr (!KL) {
            if (tid == 0) {
                if (t.label >= V) {
                    pw = NAN;
                } else if (in_part(t.label)) {
                    pw = pa - t.s;
                    pP = 1.f;
                }
            }
        } else {
            // the previous row's marks: every thread is past that row's stores
            for (int i = tid; i < words; i += BLOCK)
                bm_other[i] = 0u;
            float accw = 0.f, accP = 0.f;
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
                    if (in_part(id) && pq > 0.f)
                        sv = IO::load_elem(p, id);
                }
                if (id >= V) {
                    accw = NAN;
                    continue;
                }
                if (in_part(id) && pq > 0.f) {
                    accw += pq * (__logf(pq) - (sv - pa));
                    accP += pq;
                }
            }
            const float ww = wave_sum(accw);
            const float wP = wave_sum(accP);
            if (lane == 0) {
                sh_w[par][wid] = ww;
                sh_P[par][wid] = wP;
            }
            block_sync_lds();
            pw = 0.f;
            pP = 0.f;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                pw += sh_w[par][i];
                pP += sh_P[par][i];
            }
        }

        // ---- exchange with the other members, then every thread takes lse
        if (wid == 0) {
            if constexpr (!KL) {
                pw = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                   __builtin_bit_cast(int, pw), 0));
                pP = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                   __builtin_bit_cast(int, pP), 0));
            }
            exchange(par, pa, pz, pw, pP);
            // PF: wave 0 streams its share of the next row only now, so that
            // the exchange's atomics, which wait for every earlier memory
            // operation of the wave, do not wait for the prefetch.
            if constexpr (PF)
                if (has_next)
                    prefetch_row(nrow);
        }
        block_sync_lds();
        const float lse = sh_x[par][0];
        if (me == 0 && tid == 0) {
            a.loss[row] = sh_x[par][1];
            if (a.lse)
                a.lse[row] = lse;
        }

        // ---- KL: the gradient at the teacher ids of the part
        if constexpr (KL) {
            for (uint32_t q = tid; q < k; q += BLOCK) {
                uint32_t id;
                float pq, sv;
                if (q == (uint32_t)tid) {
                    id = t.id;
                    pq = t.p;
                    sv = t.s;
                } else {
                    id = a.ids[row * k + q];
                    pq = a.probs[row * k + q];
                    sv = in_part(id) && pq != 0.f ? IO::load_elem(p, id) : 0.f;
                }
                if (!in_part(id) || pq == 0.f)
                    continue;
                const float gid = coef * (__expf(sv - lse) - pq);
                const uint32_t v = id / N, j0 = v * N, jl = j0 - c0;
                const uint32_t vb = (bm[jl >> 5] >> (jl & 31)) & (uint32_t)((1ull << N) - 1);
                if (__builtin_popcount(vb) == 1) {
                    float x[N], g[N];
                    IO::unpack(IO::load_raw(p, v), x);
#pragma unroll
                    for (int c = 0; c < N; ++c)
                        g[c] = (uint32_t)c == id - j0 ? gid : coef * __expf(x[c] - lse);
                    IO::store(p, v, g);
                } else {
                    IO::store_elem(p, id, gid);
                }
            }
        }

        // ---- gradient store (without PF each register is refilled with the
        // next row's vector right after its store)
        {
            const float lsel = lse * kLog2e;
            const float cf = coef * __builtin_amdgcn_exp2f(msl - lsel);
            const char *np_ = rowp(nrow);
            if constexpr (!kKeepExp)
                opaque(buf, lse);
            const uint32_t t1 = fresh_tid();
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const uint32_t lv = t1 + (uint32_t)i * BLOCK;
                if (lv < np) {
                    float x[N], g[N];
                    if constexpr (kOwnExp) {
#pragma unroll
                        for (int c = 0; c < N; ++c)
                            x[c] = ex[i][c];
                    } else {
                        IO::unpack(buf[i], x);
                    }
#pragma unroll
                    for (int c = 0; c < N; ++c)
                        g[c] = kKeepExp ? x[c] * cf : coef * exp_shifted(x[c], lsel);
                    store_vec(p, vbeg + lv, g, t, bm);
                }
                if constexpr (!PF) {
                    // not before this vector's store: the register is the
                    // one being freed
                    __asm__ __volatile__("" ::: "memory");
                    if (has_next)
                        buf[i] = load_part(np_, lv);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        if (has_next) {
            mark_targets(nrow, tn, bm_other);
            gather_s(nrow, tn);
        }
    }

    __device__ void zero_row(int64_t row) const
    {
        char *p = rowp(row);
        float z[N];
#pragma unroll
        for (int c = 0; c < N; ++c)
            z[c] = 0.f;
        for (uint32_t v = tid; v < nvec; v += BLOCK)
            IO::store(p, v, z);
        if (tid == 0) {
            a.loss[row] = 0.f;
            if (a.lse)
                a.lse[row] = 0.f;
        }
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
        c.init(grp, A.groups, w.len_in);
        if (c.j < w.n_in) {
            Raw buf[NV];
            Tgt ta, tb;
            int par = 0;
            int64_t row = c.in_row(w);
            fetch_targets(row, ta);
            if constexpr (PF)
                prefetch_row(row);
            else
                load_row(rowp(row), buf);
            mark_targets(row, ta, bitmaps);
            gather_s(row, ta);
            for (;;) {
                RowCursor nc = c;
                nc.advance();
                const bool has_next = nc.j < w.n_in;
                const int64_t nrow = has_next ? nc.in_row(w) : row;
                if constexpr (PF) {
                    wait_vm_all();  // this row's loads into LDS (and all older)
                    if constexpr (!kOwnExp) {
#pragma unroll
                        for (int i = 0; i < NV; ++i)
                            buf[i] = pf[tid + i * BLOCK];
                        wait_lds_all();  // read before the slots are refilled
                        if (has_next && wid != 0)
                            prefetch_row(nrow);
                    }
                }
                fetch_targets(nrow, tb);
                process(row, buf, ta, par, has_next, nrow, tb);
                if (!has_next)
                    break;
                par ^= 1;
                c = nc;
                row = nrow;
                ta = tb;
            }
        }
        RowCursor o;
        o.init(blockIdx.x, gridDim.x, w.len_out);
        for (; o.j < w.n_out; o.advance())
            zero_row(o.out_row(w));
    }
};

// WAVES: waves per SIMD the register allocation must allow (the workgroups
// per CU times BLOCK / 256).
template <int DT, bool KL, int BLOCK, int NV, bool PF, int WAVES>
__global__ __launch_bounds__(BLOCK, WAVES) void split_row_kernel(SplitArgs sa)
{
    constexpr int NW = BLOCK / kWave;
    __shared__ float sh_m[2][NW];
    __shared__ float sh_s[2][NW];
    __shared__ float sh_w[2][NW];
    __shared__ float sh_P[2][NW];
    __shared__ float sh_x[2][2];
    // Dynamic LDS: [PF: BLOCK x NV 16-byte slots][KL: two bitmaps of the part's columns]
    extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
    using K = SplitKernel<DT, KL, BLOCK, NV, PF>;
    constexpr uint32_t pf_words = PF ? (uint32_t)BLOCK * NV * 4 : 0;
    K k(sa, sh_m, sh_s, sh_w, sh_P, sh_x, dyn + pf_words, reinterpret_cast<typename K::Raw *>(dyn));
    k.run();
}

__global__ void mbox_clear_kernel(uint64_t *mb, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        mb[i] = 0;
}

namespace {

template <int DT, bool KL, int BLOCK, int NV, bool PF, int PER_CU>
hipError_t launch_split_shape(const RowArgs &a, int S, void *ws, size_t ws_bytes, hipStream_t st)
{
    constexpr int N = RowIO<DT, true>::N;
    constexpr int WAVES = PER_CU * BLOCK / 256;
    auto fn = split_row_kernel<DT, KL, BLOCK, NV, PF, WAVES>;
    SplitArgs sa{};
    sa.r = a;
    sa.parts = S;
    const SplitShape shape{BLOCK, NV, PF, PER_CU};
    // the LDS size does not depend on the grid: plan once for it
    const size_t lds = split_plan(a.V, N, S, KL, shape, 8, ws_bytes).lds;
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute((const void *)fn,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess)
            return e;
    }
    int per_cu = blocks_per_cu((const void *)fn, BLOCK, lds);
    if (per_cu > PER_CU)
        per_cu = PER_CU;
    const SplitShape fit{BLOCK, NV, PF, per_cu};
    // groups in multiples of 8 (one per XCD), as many as the mailbox holds
    const SplitPlan plan = split_plan(a.V, N, S, KL, fit, device_cus(), ws_bytes);
    if (plan.groups < 8 || (int64_t)plan.part_vecs * (S - 1) >= a.V / N ||
        (int64_t)plan.part_vecs > (int64_t)BLOCK * NV)
        return hipErrorInvalidValue;  // too small a workspace, an empty last part, or a
                                      // part longer than the registers hold
    sa.part_vecs = plan.part_vecs;
    sa.groups = plan.groups;
    sa.mbox = static_cast<uint64_t *>(ws);
    sa.spin_limit = kSplitSpinLimit;
    hipLaunchKernelGGL(mbox_clear_kernel, dim3(64), dim3(256), 0, st, sa.mbox, plan.mbox_words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    void *args[] = {&sa};
    return hipLaunchCooperativeKernel((const void *)fn, dim3((unsigned)(plan.groups * S)),
                                      dim3(BLOCK), args, (unsigned)lds, st);
}

template <int DT, bool KL>
hipError_t launch_split_dt(const RowArgs &a, int S, void *ws, size_t ws_bytes, hipStream_t st)
{
    constexpr SplitShape sh = DT == kF32 ? kSplitF32 : kSplitBf16;
    return launch_split_shape<DT, KL, sh.block, sh.nv, sh.pf, sh.per_cu>(a, S, ws, ws_bytes, st);
}

}  // namespace

// The mailbox of the entry point for callers that cannot allocate
// (vl_kl_fwd_bwd_noalloc): one workspace's worth, resident on every device
// the library runs on until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol): split_scratch looks up its device address once per device.
static __device__ __align__(256) uint64_t scratch[kSplitWorkspaceBytes / sizeof(uint64_t)];

hipError_t split_scratch(void **ptr)
{
    static std::mutex mu;
    static void *addr[64] = {nullptr};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= 64)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

int split_parts(int dtype, int64_t V)
{
    return dtype == kF32 ? split_parts_n(V, 4, kSplitF32) : split_parts_n(V, 8, kSplitBf16);
}

hipError_t launch_rows_split(int dtype, bool kl, const RowArgs &a, int S, void *ws,
                             size_t ws_bytes, hipStream_t st)
{
    if (dtype == kF32)
        return kl ? launch_split_dt<kF32, true>(a, S, ws, ws_bytes, st)
                  : launch_split_dt<kF32, false>(a, S, ws, ws_bytes, st);
    return kl ? launch_split_dt<kBF16, true>(a, S, ws, ws_bytes, st)
              : launch_split_dt<kBF16, false>(a, S, ws, ws_bytes, st);
}

}  // namespace vl
