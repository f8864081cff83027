// common.hpp -- types and small device helpers shared by the WeDLM decode
// step kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "../../include/wedlm.h"

namespace wedlm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 storage is the raw 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

constexpr int kPage = 16;   // tokens per KV page
constexpr int kWave = 64;   // CDNA wavefront width
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<uint16_t>((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct DT;
template <> struct DT<float> {
    static constexpr int kBytes = 4;
    __device__ static float load(const float* p, size_t i) { return p[i]; }
    __device__ static void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct DT<bf16_t> {
    static constexpr int kBytes = 2;
    __device__ static float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i].bits); }
    __device__ static void store(bf16_t* p, size_t i, float x) { p[i].bits = f32_to_bf16(x); }
};

__device__ __forceinline__ float4 add4(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}

// four floats -> four bf16 (round to nearest even) as one 8-byte store
__device__ __forceinline__ uint2 pack_bf16x4(float4 v) {
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16);
    o.y = (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16);
    return o;
}
__device__ __forceinline__ float4 unpack_bf16x4(uint2 u) {
    return make_float4(bf16_to_f32(u.x & 0xffff), bf16_to_f32(u.x >> 16), bf16_to_f32(u.y & 0xffff),
                       bf16_to_f32(u.y >> 16));
}

__device__ __forceinline__ void set_status(int32_t* st, uint32_t bit) {
    if (st) atomicOr(st, static_cast<int32_t>(bit));
}

}  // namespace wedlm

// Host-side helpers (defined in api.hip).
namespace wedlm {
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
}  // namespace wedlm
