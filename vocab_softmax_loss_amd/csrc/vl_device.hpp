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

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
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
// at a time.  Values are widened to float32 in registers; bf16 widens exactly
// (bits << 16) and narrows with round-to-nearest-even.

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int DT, bool VEC>
struct RowIO;

template <>
struct RowIO<kF32, true> {
    static constexpr int N = 4;
    __device__ static void load(const void *row, int64_t v, float (&x)[N])
    {
        f32x4 r = reinterpret_cast<const f32x4 *>(row)[v];
        x[0] = r[0]; x[1] = r[1]; x[2] = r[2]; x[3] = r[3];
    }
    __device__ static void store(void *row, int64_t v, const float (&g)[N])
    {
        f32x4 r = {g[0], g[1], g[2], g[3]};
        reinterpret_cast<f32x4 *>(row)[v] = r;
    }
    __device__ static void store_elem(void *row, int64_t j, float g)
    {
        reinterpret_cast<float *>(row)[j] = g;
    }
    __device__ static float load_elem(const void *row, int64_t j)
    {
        return reinterpret_cast<const float *>(row)[j];
    }
};

template <>
struct RowIO<kBF16, true> {
    static constexpr int N = 8;
    __device__ static void load(const void *row, int64_t v, float (&x)[N])
    {
        uint4 r = reinterpret_cast<const uint4 *>(row)[v];
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
        }
    }
    __device__ static void store(void *row, int64_t v, const float (&g)[N])
    {
        f32x8 f = {g[0], g[1], g[2], g[3], g[4], g[5], g[6], g[7]};
        bf16x8 b = __builtin_convertvector(f, bf16x8);
        reinterpret_cast<bf16x8 *>(row)[v] = b;
    }
    __device__ static void store_elem(void *row, int64_t j, float g)
    {
        reinterpret_cast<__bf16 *>(row)[j] = (__bf16)g;
    }
    __device__ static float load_elem(const void *row, int64_t j)
    {
        uint32_t u = reinterpret_cast<const uint16_t *>(row)[j];
        return __builtin_bit_cast(float, u << 16);
    }
};

template <>
struct RowIO<kF32, false> {
    static constexpr int N = 1;
    __device__ static void load(const void *row, int64_t v, float (&x)[N])
    {
        x[0] = reinterpret_cast<const float *>(row)[v];
    }
    __device__ static void store(void *row, int64_t v, const float (&g)[N])
    {
        reinterpret_cast<float *>(row)[v] = g[0];
    }
    __device__ static void store_elem(void *row, int64_t j, float g)
    {
        reinterpret_cast<float *>(row)[j] = g;
    }
    __device__ static float load_elem(const void *row, int64_t j)
    {
        return reinterpret_cast<const float *>(row)[j];
    }
};

template <>
struct RowIO<kBF16, false> {
    static constexpr int N = 1;
    __device__ static void load(const void *row, int64_t v, float (&x)[N])
    {
        uint32_t u = reinterpret_cast<const uint16_t *>(row)[v];
        x[0] = __builtin_bit_cast(float, u << 16);
    }
    __device__ static void store(void *row, int64_t v, const float (&g)[N])
    {
        reinterpret_cast<__bf16 *>(row)[v] = (__bf16)g[0];
    }
    __device__ static void store_elem(void *row, int64_t j, float g)
    {
        reinterpret_cast<__bf16 *>(row)[j] = (__bf16)g;
    }
    __device__ static float load_elem(const void *row, int64_t j)
    {
        uint32_t u = reinterpret_cast<const uint16_t *>(row)[j];
        return __builtin_bit_cast(float, u << 16);
    }
};

template <int DT>
__device__ __forceinline__ size_t elt_bytes()
{
    return DT == kF32 ? 4 : 2;
}

}  // namespace vl
