// Measured ceilings for the roofline report (not part of the gdn_* boundary).
//
// The spec peaks (2.5 PFLOP/s dense fp16, 8 TB/s HBM) are the roofline
// denominators.  These two kernels measure what plain code reaches on the same
// part, as second denominators:
//   * a matrix-core loop: each wave repeats a 16 x 128 x 128 fp16 product with
//     its operands in registers (one 64 x 128 x 128 product per 4-wave
//     workgroup), fp32 accumulation, no memory traffic in the loop;
//   * an in-place read-modify-write stream over an fp32 array: per step a lane
//     loads four 16-byte pieces, one workgroup-width apart, then stores them.
//     The decode step's state update has this pattern, and four loads in
//     flight per lane move more than one (~5.5 against ~4.8 TB/s from HBM
//     on MI355X).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int MFMA_THREADS = 256;

// Operands from a counter hash (random-looking, small), so the matrix cores
// see data like the real kernels' rather than constants.
__device__ __forceinline__ h8_t hashed_operand(uint32_t seed) {
    h8_t v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t x = seed * 0x9E3779B1u + (uint32_t)e * 0x85EBCA77u;
        x ^= x >> 15;
        x *= 0x2C1B3C6Du;
        x ^= x >> 12;
        v[e] = (_Float16)((float)((int)(x & 0x3FF) - 512) * (1.0f / 65536.0f));
    }
    return v;
}

__global__ __launch_bounds__(MFMA_THREADS) void mfma_loop_kernel(int iters, float* __restrict__ sink) {
    const uint32_t base = (blockIdx.x * MFMA_THREADS + threadIdx.x) * 64u;
    h8_t a[4], b[4][8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        a[k] = hashed_operand(base + k);
#pragma unroll
        for (int n = 0; n < 8; ++n) b[k][n] = hashed_operand(base + 4 + 8 * k + n);
    }
    f4_t acc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = f4_t{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int n = 0; n < 8; ++n) acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[k], b[k][n], acc[n], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) s += acc[n][0] + acc[n][1] + acc[n][2] + acc[n][3];
    sink[blockIdx.x * MFMA_THREADS + threadIdx.x] = s;  // every lane's result is live
}

constexpr int RMW_THREADS = 256;
constexpr int RMW_UNROLL = 4;  // float4 loads in flight per lane

// x <- x * a + b over n4 float4 elements, grid-stride: each step a workgroup
// covers RMW_UNROLL * RMW_THREADS consecutive float4.
__global__ __launch_bounds__(RMW_THREADS) void rmw_stream_kernel(float4* __restrict__ x, size_t n4, float a,
                                                                  float b) {
    const size_t stride = (size_t)gridDim.x * RMW_THREADS * RMW_UNROLL;
    for (size_t i = (size_t)blockIdx.x * RMW_THREADS * RMW_UNROLL + threadIdx.x; i < n4; i += stride) {
        float4 v[RMW_UNROLL];
#pragma unroll
        for (int u = 0; u < RMW_UNROLL; ++u)
            if (i + (size_t)u * RMW_THREADS < n4) v[u] = x[i + (size_t)u * RMW_THREADS];
#pragma unroll
        for (int u = 0; u < RMW_UNROLL; ++u) {
            if (i + (size_t)u * RMW_THREADS >= n4) continue;
            float4 w = v[u];
            w.x = w.x * a + b;
            w.y = w.y * a + b;
            w.z = w.z * a + b;
            w.w = w.w * a + b;
            x[i + (size_t)u * RMW_THREADS] = w;
        }
    }
}

}  // namespace

extern "C" {

// Flops of one gdn_calib_mfma_f16 launch: 2 * 16 * 128 * 128 per wave and
// iteration.
double gdn_calib_mfma_f16_flops(int iters, int workgroups) {
    return 2.0 * 16 * 128 * 128 * (double)iters * workgroups * (MFMA_THREADS / 64);
}

// Launches the matrix-core loop: `workgroups` workgroups of 4 waves, `iters`
// iterations each; `sink` (device, >= 256 * workgroups floats) receives one
// value per thread.  Returns a hipError_t code (0 on success).
int gdn_calib_mfma_f16(int iters, int workgroups, float* sink, hipStream_t stream) {
    if (iters < 1 || workgroups < 1 || !sink) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(MFMA_THREADS), 0, stream, iters, sink);
    return (int)hipGetLastError();
}

// One in-place read-modify-write pass over `n` floats at `x` (device, 16-byte
// aligned, n a multiple of 4), with `workgroups` workgroups of 256 threads.
int gdn_calib_rmw_f32(float* x, size_t n, int workgroups, hipStream_t stream) {
    if (!x || n == 0 || n % 4 != 0 || ((uintptr_t)x & 15) != 0 || workgroups < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(rmw_stream_kernel, dim3(workgroups), dim3(RMW_THREADS), 0, stream,
                       reinterpret_cast<float4*>(x), n / 4, 0.999f, 1e-7f);
    return (int)hipGetLastError();
}

}  // extern "C"
