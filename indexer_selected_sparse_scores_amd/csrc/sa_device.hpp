// Device-side helpers shared by the gfx950 kernels of libsparse_attn.
//
// Wave64 CDNA4 building blocks: bf16 <-> fp32 bit conversions, 128-bit fragment loads,
// the MFMA operand types, and an order-preserving map from fp32 scores to uint32 keys
// used by the radix top-k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __uint_as_float((uint32_t)b << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Element loads for the generic (VALU) kernels.
__device__ __forceinline__ float load_elem(const float *p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t *p) { return bf16_bits_to_f32(*p); }

// 16-byte load that the compiler can issue as one global_load_dwordx4.
__device__ __forceinline__ uint4 load16(const void *p)
{
    return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v)
{
    return __builtin_bit_cast(bf16x8, v);
}

// Map an fp32 score to a uint32 whose unsigned order is the numeric order of the
// scores; -0.0 and +0.0 map to the same key (they compare equal).
__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// max(x, 0) as one signed-integer max on the bits: a float with the sign bit set is a
// negative int and becomes +0; fmaxf would first canonicalise x (one more instruction).
__device__ __forceinline__ float relu(float x)
{
    return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ void flag_error(uint32_t *err, uint32_t bit)
{
    if (err) atomicOr(err, bit);
}

// Cross-lane reductions over each 32-lane half of the wave on the VALU: DPP quad
// permutations and row mirrors combine 16 lanes, v_permlane16_swap the two 16-lane rows.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

__device__ __forceinline__ float half_wave_max(float x)
{
    x = fmaxf(x, dpp_mov<kDppXor1>(x));
    x = fmaxf(x, dpp_mov<kDppXor2>(x));
    x = fmaxf(x, dpp_mov<kDppRowHalfMirror>(x));
    x = fmaxf(x, dpp_mov<kDppRowMirror>(x));
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

__device__ __forceinline__ float half_wave_sum(float x)
{
    x += dpp_mov<kDppXor1>(x);
    x += dpp_mov<kDppXor2>(x);
    x += dpp_mov<kDppRowHalfMirror>(x);
    x += dpp_mov<kDppRowMirror>(x);
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace sa
