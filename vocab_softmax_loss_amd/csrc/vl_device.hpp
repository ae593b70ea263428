// Device helpers for the gfx950 (CDNA4) kernels of the fused
// vocabulary-softmax loss: wave64 reductions on DPP, 16-byte row vectors of
// float32 or bf16, and round-to-nearest-even bf16 stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vl {

constexpr int kWave = 64;

enum Dtype : int { kF32 = 0, kBF16 = 1 };

// ---------------------------------------------------------------- wave64 reductions
//
// DPP steps: quad_perm [1,0,3,2] and [2,3,0,1] combine lanes inside each
// quad, row_half_mirror and row_mirror inside each row of 16, then
// row_bcast:15 (rows 1 and 3) and row_bcast:31 (rows 2 and 3) carry the row
// totals upward so that lane 63 holds the result for the whole wave, which
// v_readlane turns into a wave-uniform (scalar) value.

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float old, float src)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                           __builtin_bit_cast(int, src), CTRL,
                                           ROW_MASK, 0xF, false));
}

__device__ __forceinline__ float readlane63(float v)
{
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp<0xB1>(v, v));
    v = fmaxf(v, dpp<0x4E>(v, v));
    v = fmaxf(v, dpp<0x141>(v, v));
    v = fmaxf(v, dpp<0x140>(v, v));
    v = fmaxf(v, dpp<0x142, 0xA>(v, v));
    v = fmaxf(v, dpp<0x143, 0xC>(v, v));
    return readlane63(v);
}

__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<0xB1>(0.f, v);
    v += dpp<0x4E>(0.f, v);
    v += dpp<0x141>(0.f, v);
    v += dpp<0x140>(0.f, v);
    v += dpp<0x142, 0xA>(0.f, v);
    v += dpp<0x143, 0xC>(0.f, v);
    return readlane63(v);
}

template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t src)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, CTRL, ROW_MASK, BANK_MASK,
                                                 BOUND_ZERO);
}

// Inclusive prefix sum over the 64 lanes.  row_shr 1..3 of the input, then
// row_shr 4 (banks 1-3) and 8 (banks 2-3) of the running sum complete each
// row of 16; row_bcast 15 / 31 add the totals of the rows below.
__device__ __forceinline__ uint32_t wave_prefix_sum_u32(uint32_t x)
{
    uint32_t acc = x;
    acc += dpp_u32<0x111, 0xF, 0xF, true>(0u, x);
    acc += dpp_u32<0x112, 0xF, 0xF, true>(0u, x);
    acc += dpp_u32<0x113, 0xF, 0xF, true>(0u, x);
    acc += dpp_u32<0x114, 0xF, 0xE>(0u, acc);
    acc += dpp_u32<0x118, 0xF, 0xC>(0u, acc);
    acc += dpp_u32<0x142, 0xA, 0xF>(0u, acc);
    acc += dpp_u32<0x143, 0xC, 0xF>(0u, acc);
    return acc;
}

__device__ __forceinline__ uint32_t readlane63_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, dpp_u32<0xB1>(v, v));
    v = max(v, dpp_u32<0x4E>(v, v));
    v = max(v, dpp_u32<0x141>(v, v));
    v = max(v, dpp_u32<0x140>(v, v));
    v = max(v, dpp_u32<0x142, 0xA>(v, v));
    v = max(v, dpp_u32<0x143, 0xC>(v, v));
    return readlane63_u32(v);
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v)
{
    v = min(v, dpp_u32<0xB1>(v, v));
    v = min(v, dpp_u32<0x4E>(v, v));
    v = min(v, dpp_u32<0x141>(v, v));
    v = min(v, dpp_u32<0x140>(v, v));
    v = min(v, dpp_u32<0x142, 0xA>(v, v));
    v = min(v, dpp_u32<0x143, 0xC>(v, v));
    return readlane63_u32(v);
}

__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v)
{
    v |= dpp_u32<0xB1>(0u, v);
    v |= dpp_u32<0x4E>(0u, v);
    v |= dpp_u32<0x141>(0u, v);
    v |= dpp_u32<0x140>(0u, v);
    v |= dpp_u32<0x142, 0xA>(0u, v);
    v |= dpp_u32<0x143, 0xC>(0u, v);
    return readlane63_u32(v);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// The lanes where p holds: one compare straight into a scalar lane mask.
__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Workgroup barrier for data exchanged through LDS.  It waits only for this
// wave's own LDS operations (lgkmcnt(0)) and then s_barrier; the empty asm
// statements keep the compiler from moving memory accesses across it.
// __syncthreads(), and even an LDS-scoped fence, would also wait for all of
// the wave's outstanding HBM loads and stores -- including asynchronous
// loads into LDS slots that no other wave reads -- and so wait for a
// prefetch at every barrier.
__device__ __forceinline__ void block_sync_lds()
{
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ __volatile__("" ::: "memory");
}

// Asynchronous 16-byte load from global memory into LDS
// (global_load_lds_dwordx4): lane l of the wave writes lds_base + 16 l,
// where lds_base must be the same for the whole wave.  Completion is counted
// by vmcnt only; the compiler does not order later LDS reads after it, so
// callers wait explicitly (wait_vm_all) before reading the destination and
// wait for their own earlier reads of it (wait_lds_all) before issuing.
__device__ __forceinline__ void load_to_lds16(const void *gptr, void *lds_base)
{
    __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void *)lds_base,
                                     16, 0, 0);
}

// s_waitcnt vmcnt(0): every vector memory operation of this wave is done.
// Encoding (gfx9): vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8];
// expcnt and lgkmcnt left at their maxima (no wait on them).
__device__ __forceinline__ void wait_vm_all()
{
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __asm__ __volatile__("" ::: "memory");
}

// s_waitcnt lgkmcnt(0): this wave's LDS (and scalar memory) operations are
// done.
__device__ __forceinline__ void wait_lds_all()
{
    __asm__ __volatile__("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __asm__ __volatile__("" ::: "memory");
}

// Orders the LDS accesses of one wave (no other wave is involved).
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- row vectors
//
// A row is read as 16-byte vectors (4 float32 or 8 bf16) when its start is
// 16-byte aligned and V is a multiple of the vector width, else one element
// at a time.  Vector and element indices inside a row are 32-bit (V is
// below 2^31); addresses are the row base plus the index scaled in 64 bits.
// A vector is held raw (Raw) in registers and widened to float32 where it
// is used; bf16 widens exactly (bits << 16) and narrows with
// round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DT, bool VEC>
struct RowIO;

template <>
struct RowIO<kF32, true> {
    static constexpr int N = 4;
    typedef u32x4 Raw;
    __device__ static Raw load_raw(const void *row, uint32_t v)
    {
        return reinterpret_cast<const Raw *>(row)[v];
    }
    __device__ static void unpack(const Raw &r, float (&x)[N])
    {
        // Copy each element out first: __builtin_bit_cast applied to a
        // vector-element lvalue reads the wrong element with this compiler.
#pragma unroll
        for (int c = 0; c < N; ++c) {
            const uint32_t u = r[c];
            x[c] = __builtin_bit_cast(float, u);
        }
    }
    // A read that nothing re-reads soon (nt): it does not displace what the
    // caches hold, so it does not force out their dirty lines either.
    __device__ static Raw load_stream(const void *row, uint32_t v)
    {
        return __builtin_nontemporal_load(reinterpret_cast<const Raw *>(row) + v);
    }
    // Gradient rows are written once and exceed every cache: nt stores keep
    // them from sitting dirty in the last-level cache, whose write-back
    // would otherwise fall inside the next kernel.
    __device__ static void store(void *row, uint32_t v, const float (&g)[N])
    {
        f32x4 r = {g[0], g[1], g[2], g[3]};
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4 *>(row) + v);
    }
    __device__ static void store_elem(void *row, uint32_t j, float g)
    {
        reinterpret_cast<float *>(row)[j] = g;
    }
    __device__ static float load_elem(const void *row, uint32_t j)
    {
        return reinterpret_cast<const float *>(row)[j];
    }
};

template <>
struct RowIO<kBF16, true> {
    static constexpr int N = 8;
    typedef u32x4 Raw;
    __device__ static Raw load_raw(const void *row, uint32_t v)
    {
        return reinterpret_cast<const Raw *>(row)[v];
    }
    __device__ static Raw load_stream(const void *row, uint32_t v)
    {
        return __builtin_nontemporal_load(reinterpret_cast<const Raw *>(row) + v);
    }
    __device__ static void unpack(const Raw &r, float (&x)[N])
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __builtin_bit_cast(float, r[i] << 16);
            x[2 * i + 1] = __builtin_bit_cast(float, r[i] & 0xFFFF0000u);
        }
    }
    // Non-temporal, as for float32: 16384 x 151936 KL 2.06 -> 1.98 ms, and
    // the next kernel no longer pays the write-back of dirty lines (the
    // slice accumulate after that KL 56 -> 39 us).
    __device__ static void store(void *row, uint32_t v, const float (&g)[N])
    {
        f32x8 f = {g[0], g[1], g[2], g[3], g[4], g[5], g[6], g[7]};
        bf16x8 b = __builtin_convertvector(f, bf16x8);
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, b), reinterpret_cast<u32x4 *>(row) + v);
    }
    __device__ static void store_elem(void *row, uint32_t j, float g)
    {
        reinterpret_cast<__bf16 *>(row)[j] = (__bf16)g;
    }
    __device__ static float load_elem(const void *row, uint32_t j)
    {
        uint32_t u = reinterpret_cast<const uint16_t *>(row)[j];
        return __builtin_bit_cast(float, u << 16);
    }
};

template <>
struct RowIO<kF32, false> {
    static constexpr int N = 1;
    typedef uint32_t Raw;
    __device__ static Raw load_raw(const void *row, uint32_t v)
    {
        return reinterpret_cast<const uint32_t *>(row)[v];
    }
    __device__ static Raw load_stream(const void *row, uint32_t v)
    {
        return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(row) + v);
    }
    __device__ static void unpack(const Raw &r, float (&x)[N]) { x[0] = __builtin_bit_cast(float, r); }
    __device__ static void store(void *row, uint32_t v, const float (&g)[N])
    {
        reinterpret_cast<float *>(row)[v] = g[0];
    }
    __device__ static void store_elem(void *row, uint32_t j, float g)
    {
        reinterpret_cast<float *>(row)[j] = g;
    }
    __device__ static float load_elem(const void *row, uint32_t j)
    {
        return reinterpret_cast<const float *>(row)[j];
    }
};

template <>
struct RowIO<kBF16, false> {
    static constexpr int N = 1;
    typedef uint32_t Raw;
    __device__ static Raw load_raw(const void *row, uint32_t v)
    {
        return reinterpret_cast<const uint16_t *>(row)[v];
    }
    __device__ static Raw load_stream(const void *row, uint32_t v)
    {
        return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(row) + v);
    }
    __device__ static void unpack(const Raw &r, float (&x)[N]) { x[0] = __builtin_bit_cast(float, r << 16); }
    __device__ static void store(void *row, uint32_t v, const float (&g)[N])
    {
        reinterpret_cast<__bf16 *>(row)[v] = (__bf16)g[0];
    }
    __device__ static void store_elem(void *row, uint32_t j, float g)
    {
        reinterpret_cast<__bf16 *>(row)[j] = (__bf16)g;
    }
    __device__ static float load_elem(const void *row, uint32_t j)
    {
        uint32_t u = reinterpret_cast<const uint16_t *>(row)[j];
        return __builtin_bit_cast(float, u << 16);
    }
};

// A raw vector whose elements all read as -inf (padding past the row end).
template <int DT, bool VEC>
__device__ __forceinline__ typename RowIO<DT, VEC>::Raw neg_inf_raw()
{
    typename RowIO<DT, VEC>::Raw r;
    if constexpr (VEC) {
        const uint32_t w = DT == kF32 ? 0xFF800000u : 0xFF80FF80u;
        r = u32x4{w, w, w, w};
    } else {
        r = DT == kF32 ? 0xFF800000u : 0xFF80u;
    }
    return r;
}

// Gradient rows rounded to bf16 (BF) or f16 as they are stored, into a
// separate half-precision row that a GEMM reads next: N values of float32
// vector vi of the row at q (non-temporal: written once, read by the next
// kernel from HBM anyway).
template <bool BF, int N>
__device__ __forceinline__ void half_store(char *q, uint32_t vi, const float (&g)[N])
{
    if constexpr (N == 4) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
        const f32x4 f = {g[0], g[1], g[2], g[3]};
        unsigned long long bits;
        if constexpr (BF)
            bits = __builtin_bit_cast(unsigned long long, __builtin_convertvector(f, bf16x4));
        else
            bits = __builtin_bit_cast(unsigned long long, __builtin_convertvector(f, f16x4));
        __builtin_nontemporal_store(bits, reinterpret_cast<unsigned long long *>(q) + vi);
    } else if constexpr (N == 8) {
        typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
        const f32x8 f = {g[0], g[1], g[2], g[3], g[4], g[5], g[6], g[7]};
        u32x4 bits;
        if constexpr (BF)
            bits = __builtin_bit_cast(u32x4, __builtin_convertvector(f, bf16x8));
        else
            bits = __builtin_bit_cast(u32x4, __builtin_convertvector(f, f16x8));
        __builtin_nontemporal_store(bits, reinterpret_cast<u32x4 *>(q) + vi);
    } else {
        if constexpr (BF)
            reinterpret_cast<__bf16 *>(q)[vi] = (__bf16)g[0];
        else
            reinterpret_cast<_Float16 *>(q)[vi] = (_Float16)g[0];
    }
}


template <int DT>
__device__ __forceinline__ size_t elt_bytes()
{
    return DT == kF32 ? 4 : 2;
}

}  // namespace vl
