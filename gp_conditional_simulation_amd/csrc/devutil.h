// Device helpers shared by the gfx950 kernels of libgpex.
#pragma once
#include <hip/hip_runtime.h>

namespace gpex {

// Correct round-to-nearest-even FP64 -> FP16: round to odd at FP32 (24 significant bits, at
// least two more than FP16's 11), then let the hardware round FP32 -> FP16 to nearest even.
__device__ __forceinline__ _Float16 f64_to_f16(double d) {
    float f = (float)d;
    double back = (double)f;
    if (back != d && d == d) {
        unsigned u = __float_as_uint(f);
        if (fabs(back) > fabs(d)) u -= 1u;
        u |= 1u;
        f = __uint_as_float(u);
    }
    return (_Float16)f;
}

__device__ __forceinline__ double load_as_double(const void* p, int dt, int64_t i) {
    if (dt == 0) return static_cast<const double*>(p)[i];
    if (dt == 1) return (double)static_cast<const float*>(p)[i];
    return (double)static_cast<const _Float16*>(p)[i];
}

// Stores v in type dt (RNE); returns true when an FP16/FP32 store overflowed to +-inf.
__device__ __forceinline__ bool store_from_double(void* p, int dt, int64_t i, double v) {
    if (dt == 0) {
        static_cast<double*>(p)[i] = v;
        return false;
    }
    if (dt == 1) {
        float f = (float)v;
        static_cast<float*>(p)[i] = f;
        return __builtin_isinf(f) && !__builtin_isinf(v);
    }
    _Float16 h = f64_to_f16(v);
    static_cast<_Float16*>(p)[i] = h;
    return __builtin_isinf((float)h) && !__builtin_isinf(v);
}

}  // namespace gpex
