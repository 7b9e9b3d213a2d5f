// Calibration kernels: issue rates of the matrix-core and vector instructions
// the expert FFN kernels are built from, and a plain HBM read stream.  They
// give the measured ceilings against which the layer's kernels are judged
// (datasheet peaks aside).  Built into its own library, libmoe_probe.so; the
// layer library does not contain or call them.
//
// Every kernel runs a fixed number of iterations on register operands, then
// writes one value per thread so that nothing is optimised away.  The host
// times launches with events on the stream it passes in.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));
typedef unsigned uint4v __attribute__((ext_vector_type(4)));

enum {
    PROBE_MFMA_I8_32X32X32 = 0,
    PROBE_MFMA_I8_16X16X64 = 1,
    PROBE_MFMA_F16_32X32X16 = 2,
    PROBE_MFMA_F16_16X16X32 = 3,
    PROBE_VALU_FMA_F32 = 4,
    PROBE_I8_MFMA_TWO_OP_EPILOGUE = 5,   // one 32x32x32 int8 MFMA + 2 fp32 FMAs per output
    PROBE_STREAM_READ = 6,
    PROBE_I8_MFMA_ONE_OP_EPILOGUE = 7,   // one 32x32x32 int8 MFMA + 1 fp32 FMA per output
    PROBE_STREAM_READ_BURST = 8,         // the read with eight loads in flight per thread
};

__global__ __launch_bounds__(256) void k_mfma_i8_32(int iters, int seed, float* out) {
    int4v a = {seed + (int)threadIdx.x, seed * 3, 5, 7};
    const int4v b = {seed ^ 0x01020304, 11, 13, (int)threadIdx.x};
    int16v c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    int s = 0;
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = (float)s;
}

__global__ __launch_bounds__(256) void k_mfma_i8_16(int iters, int seed, float* out) {
    const int4v a = {seed + (int)threadIdx.x, seed * 3, 5, 7};
    const int4v b = {seed ^ 0x01020304, 11, 13, (int)threadIdx.x};
    int4v c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(b, b, c3, 0, 0, 0);
    }
    int s = 0;
    for (int r = 0; r < 4; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = (float)s;
}

__global__ __launch_bounds__(256) void k_mfma_f16_32(int iters, int seed, float* out) {
    half8 a, b;
    for (int j = 0; j < 8; ++j) {
        a[j] = (_Float16)(0.001f * (float)(seed + j + (int)threadIdx.x % 7));
        b[j] = (_Float16)(0.002f * (float)(j - 3));
    }
    float16v c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, c3, 0, 0, 0);
    }
    float s = 0.f;
    for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void k_mfma_f16_16(int iters, int seed, float* out) {
    half8 a, b;
    for (int j = 0; j < 8; ++j) {
        a[j] = (_Float16)(0.001f * (float)(seed + j + (int)threadIdx.x % 7));
        b[j] = (_Float16)(0.002f * (float)(j - 3));
    }
    float4v c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, b, c3, 0, 0, 0);
    }
    float s = 0.f;
    for (int r = 0; r < 4; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// 16 independent fp32 FMA chains per lane (plain v_fma_f32: packed fp32 code
// generation is switched off for every HIP file of this project).
__global__ __launch_bounds__(256) void k_valu_fma(int iters, int seed, float* out) {
    float v[16];
    const float m = 1.0f - 1e-7f * (float)(seed & 7), c = 1e-6f;
    for (int j = 0; j < 16; ++j) v[j] = (float)(threadIdx.x + j);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = fmaf(v[j], m, c);
    }
    float s = 0.f;
    for (int j = 0; j < 16; ++j) s += v[j];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// The exact block-scaled int8 pattern of the prefill gate/up kernel: per
// 32-wide block, one 32x32x32 int8 MFMA seeded with the bits of 1.5 * 2^23,
// then per output t = fma(D, sw, -1.5 * 2^23 * sw) and acc = fma(t, sa, acc)
// (TWO_OP), or the accumulation alone (ONE_OP).  Two n-tiles per iteration, as
// in the kernel; the A operand changes every iteration so that the MFMAs stay
// inside the loop.
template <bool TWO_OP>
__global__ __launch_bounds__(256) void k_i8_epilogue(int iters, int seed, float* out) {
    int4v a = {seed + (int)threadIdx.x, seed * 3, 5, 7};
    const int4v b0 = {seed ^ 0x01020304, 11, 13, (int)threadIdx.x};
    const int4v b1 = {seed ^ 0x05060708, 17, 19, (int)threadIdx.x * 3};
    int16v cm;
    for (int r = 0; r < 16; ++r) cm[r] = 0x4B400000;
    asm volatile("" : "+v"(cm));
    const float sw0 = 0.01f + 1e-5f * (float)(threadIdx.x & 31), sw1 = 0.02f - 1e-5f * (float)(threadIdx.x & 31);
    const float nc0 = -12582912.0f * sw0, nc1 = -12582912.0f * sw1;
    float sa[16];
    for (int r = 0; r < 16; ++r) sa[r] = 0.003f * (float)(r + 1 + (seed & 3) + (int)(threadIdx.x >> 5));
    float16v acc0 = {}, acc1 = {};
    for (int i = 0; i < iters; ++i) {
        a[0] += 1;
        const int16v d0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b0, cm, 0, 0, 0);
        const int16v d1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b1, cm, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if constexpr (TWO_OP) {
                const float t0 = fmaf(__int_as_float(d0[r]), sw0, nc0);
                const float t1 = fmaf(__int_as_float(d1[r]), sw1, nc1);
                acc0[r] = fmaf(t0, sa[r], acc0[r]);
                acc1[r] = fmaf(t1, sa[r], acc1[r]);
            } else {
                acc0[r] = fmaf(__int_as_float(d0[r]), sa[r], acc0[r]);
                acc1[r] = fmaf(__int_as_float(d1[r]), sa[r], acc1[r]);
            }
        }
    }
    float s = 0.f;
    for (int r = 0; r < 16; ++r) s += acc0[r] + acc1[r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Read n16 16-byte words, grid-strided, coalesced; one partial sum per thread.
__global__ __launch_bounds__(256) void k_stream_read(const uint4v* __restrict__ in, size_t n16, float* out) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint32_t s = 0;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const uint4v v = __builtin_nontemporal_load(in + i);
        s += v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = (float)s;
}

// The same read with eight loads in flight per thread and iteration, the
// shape of a short read (a few MB in one launch) at its best: no load waits
// on the previous one.
__global__ __launch_bounds__(256) void k_stream_read_burst(const uint4v* __restrict__ in, size_t n16, float* out) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    uint32_t s = 0;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        uint4v v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(in + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += stride) {
        const uint4v v = __builtin_nontemporal_load(in + i);
        s += v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    out[blockIdx.x * blockDim.x + threadIdx.x] = (float)s;
}

extern "C" {

// Launches one calibration kernel on `stream` (a hipStream_t, or null for the
// default stream).  grid workgroups of 256 threads; out must hold grid * 256
// floats.  For PROBE_STREAM_READ and PROBE_STREAM_READ_BURST, in points to
// in_bytes (a multiple of 16) of device memory; the other kinds ignore it.  Returns 0, -1 for a bad argument
// (checked before any launch), or the hipError_t of the launch.
int moe_probe_run(int kind, int grid, int iters, int seed, float* out, const void* in, size_t in_bytes,
                  void* stream) {
    if (grid <= 0 || iters < 0 || !out) return -1;
    if ((kind == PROBE_STREAM_READ || kind == PROBE_STREAM_READ_BURST) && (!in || in_bytes % 16)) return -1;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    switch (kind) {
        case PROBE_MFMA_I8_32X32X32: k_mfma_i8_32<<<grid, 256, 0, s>>>(iters, seed, out); break;
        case PROBE_MFMA_I8_16X16X64: k_mfma_i8_16<<<grid, 256, 0, s>>>(iters, seed, out); break;
        case PROBE_MFMA_F16_32X32X16: k_mfma_f16_32<<<grid, 256, 0, s>>>(iters, seed, out); break;
        case PROBE_MFMA_F16_16X16X32: k_mfma_f16_16<<<grid, 256, 0, s>>>(iters, seed, out); break;
        case PROBE_VALU_FMA_F32: k_valu_fma<<<grid, 256, 0, s>>>(iters, seed, out); break;
        case PROBE_I8_MFMA_TWO_OP_EPILOGUE: k_i8_epilogue<true><<<grid, 256, 0, s>>>(iters, seed, out); break;
        case PROBE_I8_MFMA_ONE_OP_EPILOGUE: k_i8_epilogue<false><<<grid, 256, 0, s>>>(iters, seed, out); break;
        case PROBE_STREAM_READ:
            k_stream_read<<<grid, 256, 0, s>>>(reinterpret_cast<const uint4v*>(in), in_bytes / 16, out);
            break;
        case PROBE_STREAM_READ_BURST:
            k_stream_read_burst<<<grid, 256, 0, s>>>(reinterpret_cast<const uint4v*>(in), in_bytes / 16, out);
            break;
        default: return -1;
    }
    return (int)hipGetLastError();
}

}  // extern "C"
