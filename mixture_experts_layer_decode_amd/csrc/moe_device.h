// moe_device.h -- device helpers for the gfx950 (CDNA4) kernels: storage
// types, 16-byte weight vectors, bf16/fp8 unpacking and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_internal.h"

namespace moe {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------ XCD-aware work placement
//
// The MI355X has 8 XCDs, each with its own L2, and the command processor
// hands consecutive workgroups of a launch to the XCDs in turn.  In the plain
// grid-stride order XCD x therefore takes units x, x + 8, x + 16, ...: one
// unit in every eight.  xcd_walk deals the units to the XCDs in chunks of C
// consecutive units instead (chunk c to XCD c % 8), so each XCD streams runs
// of C consecutive units.  The walk covers every unit exactly once whatever
// the dispatch order, so only speed depends on it.
constexpr int kXcds = 8;

// Position pos of this workgroup's walk -> unit (increasing in pos).
// x < 0: the plain order (grids of fewer than kXcds workgroups, and the
// workgroups past the last whole group of kXcds, which start past every unit).
struct XcdWalk {
    int x, first, step, chunk;
    __device__ __forceinline__ int unit(int pos) const {
        return x < 0 ? pos : (x + kXcds * (pos / chunk)) * chunk + pos % chunk;
    }
};
__device__ __forceinline__ XcdWalk xcd_walk(int chunk) {
    const int G = gridDim.x, b = blockIdx.x;
    const int per = G / kXcds;
    if (per == 0) return {-1, b, G, 1};
    if (b >= per * kXcds) return {-1, 0x3fffffff, 1, 1};
    return {b % kXcds, b / kXcds, per, chunk};
}

// ------------------------------------------------------------ storage types

template <int DT> struct Storage;
template <> struct Storage<DT_F32> { typedef float type; };
template <> struct Storage<DT_BF16> { typedef uint16_t type; };
template <> struct Storage<DT_FP8> { typedef uint8_t type; };

// Elements in one 16-byte vector of a weight row.
template <int DT> constexpr int vec_elems() { return 16 / (int)sizeof(typename Storage<DT>::type); }

// --------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two bf16 products accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// Four OCP e4m3 codes (one dword) -> two packed bf16 pairs, exactly: every
// e4m3 value is representable in bf16, so the upper half of the fp32 result
// of the hardware conversion is the bf16 value.
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
    f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    lo = (__float_as_uint(a.x) >> 16) | (__float_as_uint(a.y) & 0xffff0000u);
    hi = (__float_as_uint(b.x) >> 16) | (__float_as_uint(b.y) & 0xffff0000u);
}

// --------------------------------------------------------------- loads

// Weight streams are read once per forward: non-temporal loads keep them from
// displacing activations, routing data and partial sums in the caches.  Only
// weights and router matrices (never data written during the forward) are
// read this way.
__device__ __forceinline__ u32x4 load_weights16(const void* p) {
    return __builtin_nontemporal_load((const u32x4*)p);
}

__device__ __forceinline__ u32x4 load16(const void* p) { return *(const u32x4*)p; }

// --------------------------------------------------------- wave reductions

// Butterfly sum over the 64 lanes: a fixed tree, so results are reproducible.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// -------------------------------------------------- weight vector x activation
//
// A 16-byte weight vector is first unpacked into "operands" (shared by every
// activation row it multiplies), then dotted with VEC activation values read
// from LDS.  fp32 accumulation throughout.

template <int WDT> struct WOps;

template <> struct WOps<DT_BF16> {
    static constexpr int kOps = 4;  // 4 dwords = 8 bf16
    __device__ __forceinline__ static void unpack(u32x4 v, uint32_t (&o)[kOps]) {
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    // a: 8 bf16 activations (16 bytes in LDS)
    __device__ __forceinline__ static float dot(const uint32_t (&o)[kOps], const uint16_t* a,
                                                float acc) {
        u32x4 av = *(const u32x4*)a;
        acc = dot2_bf16(o[0], av.x, acc);
        acc = dot2_bf16(o[1], av.y, acc);
        acc = dot2_bf16(o[2], av.z, acc);
        acc = dot2_bf16(o[3], av.w, acc);
        return acc;
    }
    // the 8 activations in registers (one 16-byte vector)
    __device__ __forceinline__ static float dotr(const uint32_t (&o)[kOps], const u32x4* a,
                                                 float acc) {
        acc = dot2_bf16(o[0], a[0].x, acc);
        acc = dot2_bf16(o[1], a[0].y, acc);
        acc = dot2_bf16(o[2], a[0].z, acc);
        acc = dot2_bf16(o[3], a[0].w, acc);
        return acc;
    }
};

template <> struct WOps<DT_FP8> {
    static constexpr int kOps = 8;  // 16 e4m3 -> 8 bf16 pairs
    __device__ __forceinline__ static void unpack(u32x4 v, uint32_t (&o)[kOps]) {
        fp8x4_to_bf16x4(v.x, o[0], o[1]);
        fp8x4_to_bf16x4(v.y, o[2], o[3]);
        fp8x4_to_bf16x4(v.z, o[4], o[5]);
        fp8x4_to_bf16x4(v.w, o[6], o[7]);
    }
    // a: 16 bf16 activations (32 bytes in LDS)
    __device__ __forceinline__ static float dot(const uint32_t (&o)[kOps], const uint16_t* a,
                                                float acc) {
        u32x4 a0 = *(const u32x4*)a;
        u32x4 a1 = *(const u32x4*)(a + 8);
        acc = dot2_bf16(o[0], a0.x, acc);
        acc = dot2_bf16(o[1], a0.y, acc);
        acc = dot2_bf16(o[2], a0.z, acc);
        acc = dot2_bf16(o[3], a0.w, acc);
        acc = dot2_bf16(o[4], a1.x, acc);
        acc = dot2_bf16(o[5], a1.y, acc);
        acc = dot2_bf16(o[6], a1.z, acc);
        acc = dot2_bf16(o[7], a1.w, acc);
        return acc;
    }
    // the 16 activations in registers (two 16-byte vectors)
    __device__ __forceinline__ static float dotr(const uint32_t (&o)[kOps], const u32x4* a,
                                                 float acc) {
        acc = dot2_bf16(o[0], a[0].x, acc);
        acc = dot2_bf16(o[1], a[0].y, acc);
        acc = dot2_bf16(o[2], a[0].z, acc);
        acc = dot2_bf16(o[3], a[0].w, acc);
        acc = dot2_bf16(o[4], a[1].x, acc);
        acc = dot2_bf16(o[5], a[1].y, acc);
        acc = dot2_bf16(o[6], a[1].z, acc);
        acc = dot2_bf16(o[7], a[1].w, acc);
        return acc;
    }
};

template <> struct WOps<DT_F32> {
    static constexpr int kOps = 4;
    __device__ __forceinline__ static void unpack(u32x4 v, uint32_t (&o)[kOps]) {
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
    // a: 4 fp32 activations (16 bytes in LDS)
    __device__ __forceinline__ static float dot(const uint32_t (&o)[kOps], const float* a,
                                                float acc) {
        f32x4 av = *(const f32x4*)a;
        acc = fmaf(__uint_as_float(o[0]), av.x, acc);
        acc = fmaf(__uint_as_float(o[1]), av.y, acc);
        acc = fmaf(__uint_as_float(o[2]), av.z, acc);
        acc = fmaf(__uint_as_float(o[3]), av.w, acc);
        return acc;
    }
    // the 4 activations in registers (one 16-byte vector)
    __device__ __forceinline__ static float dotr(const uint32_t (&o)[kOps], const u32x4* a,
                                                 float acc) {
        acc = fmaf(__uint_as_float(o[0]), __uint_as_float(a[0].x), acc);
        acc = fmaf(__uint_as_float(o[1]), __uint_as_float(a[0].y), acc);
        acc = fmaf(__uint_as_float(o[2]), __uint_as_float(a[0].z), acc);
        acc = fmaf(__uint_as_float(o[3]), __uint_as_float(a[0].w), acc);
        return acc;
    }
};

// Store one activation-typed value (h or out), rounding fp32 to nearest even.
template <int ACT> __device__ __forceinline__ void store_act(void* base, int64_t i, float v);
template <> __device__ __forceinline__ void store_act<DT_F32>(void* base, int64_t i, float v) {
    ((float*)base)[i] = v;
}
template <> __device__ __forceinline__ void store_act<DT_BF16>(void* base, int64_t i, float v) {
    ((uint16_t*)base)[i] = (uint16_t)f32_to_bf16_bits(v);
}

template <int ACT> __device__ __forceinline__ float load_act(const void* base, int64_t i);
template <> __device__ __forceinline__ float load_act<DT_F32>(const void* base, int64_t i) {
    return ((const float*)base)[i];
}
template <> __device__ __forceinline__ float load_act<DT_BF16>(const void* base, int64_t i) {
    return __uint_as_float((uint32_t)((const uint16_t*)base)[i] << 16);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

}  // namespace moe
