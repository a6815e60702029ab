// Internal helpers shared by the libmoe translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "moe.h"

namespace moe {

constexpr int kWave = 64;  // CDNA wavefront width

// Device status flag bits (first int32 of the dispatch workspace).
constexpr int kFlagBadIndex = 1;
constexpr int kFlagCapacity = 2;

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int64_t elt_size(moe_dtype_t dt) { return dt == MOE_BF16 ? 2 : 4; }
inline bool valid_dtype(moe_dtype_t dt) { return dt == MOE_BF16 || dt == MOE_F32; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// One-time set-up per GPU (kernel attributes, device queries). The library's only
// process-wide state: every device the process calls the library on runs `f` once,
// with that device current, and its result is kept for that device. Thread-safe.
constexpr int kMaxDevices = 64;
template <class T = int> struct PerDevice {
    std::once_flag once[kMaxDevices];
    T value[kMaxDevices] = {};
};
template <class T, class F> T per_device(PerDevice<T> &pd, F f) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return f();
    std::call_once(pd.once[dev], [&] { pd.value[dev] = f(); });
    return pd.value[dev];
}

// Raises a kernel's dynamic LDS limit on the current device (once per device).
template <auto Kernel> bool lds_limit_once(int bytes) {
    static PerDevice<int> pd;
    return per_device(pd, [bytes] {
               return int(hipFuncSetAttribute(reinterpret_cast<const void *>(Kernel),
                                              hipFuncAttributeMaxDynamicSharedMemorySize,
                                              bytes) == hipSuccess);
           }) != 0;
}

// Division by a divisor fixed at launch, as a multiply and a shift (there is no integer
// divide instruction; a runtime division costs dozens of instructions). For d >= 1 and
// dividends n < 2^31: with p = ceil(log2 d) and m = ceil(2^(31+p) / d) (< 2^32),
// n / d = (n * m) >> (31 + p) exactly, since n * m / 2^(31+p) exceeds n / d by less than
// n / 2^(31+p) < 1 / d.
struct FastDiv {
    uint32_t d, m, k;
    FastDiv() = default;
    explicit FastDiv(uint32_t dv) : d(dv) {
        uint32_t p = 0;
        while ((uint64_t(1) << p) < dv) ++p;
        k = 31 + p;
        m = uint32_t(((uint64_t(1) << k) + dv - 1) / dv);
    }
    __device__ __forceinline__ int div(int n) const {   // 0 <= n < 2^31
        return int((uint64_t(uint32_t(n)) * m) >> k);
    }
    __device__ __forceinline__ int64_t div64(int64_t n) const { return div(int(n)); }
};

inline moe_status_t launch_status() {
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// bf16 <-> f32. Widening is exact; narrowing is round-to-nearest-even
// (gfx950 lowers the cast to v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 b = static_cast<__bf16>(f);
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return uint32_t(f32_to_bf16_bits(lo)) | (uint32_t(f32_to_bf16_bits(hi)) << 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// 16 bytes of a row as 8 floats (bf16) or 4 floats (f32).
template <int DT> struct Vec;
template <> struct Vec<MOE_BF16> {
    static constexpr int N = 8;
    __device__ __forceinline__ static void unpack(const uint4 &v, float *f) {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
    __device__ __forceinline__ static uint4 pack(const float *f) {
        return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                          pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    }
};
template <> struct Vec<MOE_F32> {
    static constexpr int N = 4;
    __device__ __forceinline__ static void unpack(const uint4 &v, float *f) {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
    __device__ __forceinline__ static uint4 pack(const float *f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                          __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
};

}  // namespace moe
