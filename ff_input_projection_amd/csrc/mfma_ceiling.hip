// The sustained matrix-core rate of the GPU, measured with a kernel that issues only MFMAs
// (a measurement aid for the benchmark, not part of the projection).
//
// One workgroup of 4 waves per CU, one wave per SIMD: a single wave keeps its SIMD's
// matrix core busy when its MFMAs are independent (8 accumulators, each updated every 8th
// instruction, far apart compared with the MFMA's latency). The operands are four sets
// of pseudo-random bf16 values per lane, rotated between instructions, so the data in
// the datapath keeps changing as it does in a real product: with constant or zero
// operands the chip draws less power and holds a higher clock than any real GEMM sees.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "fused_proj_calibrate.h"
#include "fused_proj_kernels.h"

namespace fp {
namespace {

using namespace dev;

constexpr int kThreads = 256;

// A value in [-1, 1) from a 32-bit hash (splitmix32-style finaliser).
__device__ __forceinline__ float hash_unit(unsigned x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    return (float)(x >> 8) * (2.0f / 16777216.0f) - 1.0f;
}

__global__ __launch_bounds__(kThreads) void mfma_ceiling_kernel(int iterations, unsigned seed, float* sink) {
    const unsigned gid = blockIdx.x * kThreads + threadIdx.x;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[s][i] = (__bf16)hash_unit(seed ^ (gid * 64u + (unsigned)(s * 16 + i)));
            b[s][i] = (__bf16)hash_unit(~seed ^ (gid * 64u + (unsigned)(s * 16 + 8 + i)));
        }
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    for (int it = 0; it < iterations; ++it) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + r) & 3], b[(j + 2 * r) & 3], acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    sink[gid] = s;
}

}  // namespace

extern "C" int fused_proj_mfma_ceiling(int iterations, unsigned seed, float* sink, size_t sink_bytes, void* stream,
                                       double* flops_per_launch) {
    if (iterations < 1 || flops_per_launch == nullptr || sink == nullptr) return FUSED_PROJ_EINVAL;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || cus < 1) {
        set_last_hip_error(e);
        return FUSED_PROJ_EHIP;
    }
    if (sink_bytes < (size_t)cus * kThreads * sizeof(float)) return FUSED_PROJ_EINVAL;
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(cus), dim3(kThreads), 0, static_cast<hipStream_t>(stream), iterations,
                       seed, sink);
    e = hipGetLastError();
    if (e != hipSuccess) {
        set_last_hip_error(e);
        return FUSED_PROJ_EHIP;
    }
    *flops_per_launch = (double)cus * 4.0 * iterations * 16.0 * 32768.0;
    return FUSED_PROJ_OK;
}

}  // namespace fp
