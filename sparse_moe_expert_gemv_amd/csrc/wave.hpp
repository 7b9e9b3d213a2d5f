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

// Value held by lane (lane ^ J), J in {1, 2, 4, 8, 16, 32}, with VALU lane
// exchanges only: DPP within rows of 16 lanes (xor 4 from two row rotations),
// v_permlane16_swap / v_permlane32_swap across rows.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
    const int lane = threadIdx.x & 63;
    if constexpr (J == 1) return __builtin_amdgcn_update_dpp(v, v, kDppXor1, 0xF, 0xF, false);
    else if constexpr (J == 2) return __builtin_amdgcn_update_dpp(v, v, kDppXor2, 0xF, 0xF, false);
    else if constexpr (J == 4) {
        const uint32_t a = __builtin_amdgcn_update_dpp(v, v, kDppRor4, 0xF, 0xF, false);   // lane - 4 (mod 16)
        const uint32_t b = __builtin_amdgcn_update_dpp(v, v, 0x12C, 0xF, 0xF, false);      // lane + 4 (mod 16)
        return (lane & 4) ? a : b;
    } else if constexpr (J == 8) return __builtin_amdgcn_update_dpp(v, v, kDppRor8, 0xF, 0xF, false);
    else if constexpr (J == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}

template <int J>
__device__ __forceinline__ double lane_xor_d(double v) {
    return __hiloint2double((int)lane_xor<J>((uint32_t)__double2hiint(v)), (int)lane_xor<J>((uint32_t)__double2loint(v)));
}

// Sum over the 64 lanes, every lane gets the total (butterfly order).
__device__ __forceinline__ double wave_sum_xor_d(double v) {
    v += lane_xor_d<1>(v);
    v += lane_xor_d<2>(v);
    v += lane_xor_d<4>(v);
    v += lane_xor_d<8>(v);
    v += lane_xor_d<16>(v);
    v += lane_xor_d<32>(v);
    return v;
}

__device__ __forceinline__ double wave_sum_d(double v) {
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

}  // namespace moe
