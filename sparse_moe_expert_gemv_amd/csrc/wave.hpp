// Wavefront (64-lane) reductions built from DPP row operations and readlane.
#pragma once
#include <hip/hip_runtime.h>

namespace moe {

// DPP controls (gfx9 encoding)
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRor4 = 0x124;  // row_ror:4
constexpr int kDppRor8 = 0x128;  // row_ror:8

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ bool better(double v, int i, double ov, int oi) {
    return ov > v || (ov == v && oi < i);
}

template <int CTRL>
__device__ __forceinline__ void argmax_step(double& v, int& i) {
    const int lo = __double2loint(v), hi = __double2hiint(v);
    const double ov = __hiloint2double(dpp_i<CTRL>(hi), dpp_i<CTRL>(lo));
    const int oi = dpp_i<CTRL>(i);
    if (better(v, i, ov, oi)) { v = ov; i = oi; }
}

// Wave-uniform (value, index) with the largest value, lowest index on ties.
// Must be called by all 64 lanes.
__device__ __forceinline__ void wave_argmax(double& v, int& i) {
    argmax_step<kDppXor1>(v, i);
    argmax_step<kDppXor2>(v, i);
    argmax_step<kDppRor4>(v, i);
    argmax_step<kDppRor8>(v, i);  // every lane now holds its row's best
    double bv = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 0),
                                 __builtin_amdgcn_readlane(__double2loint(v), 0));
    int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const double ov = __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 16 * r),
                                           __builtin_amdgcn_readlane(__double2loint(v), 16 * r));
        const int oi = __builtin_amdgcn_readlane(i, 16 * r);
        if (better(bv, bi, ov, oi)) { bv = ov; bi = oi; }
    }
    v = bv;
    i = bi;
}

__device__ __forceinline__ double wave_sum_d(double v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

}  // namespace moe
