// peak.hip -- measurement aid, not part of the quantization path: a register-only MFMA loop
// that gives the matrix-core rate this GPU sustains under load (the denominator beside the
// published peak for the GEMM roofline).  Each wave issues iters x 8 independent MFMAs of one
// kind on constant operands; the accumulators are summed into sink so nothing is dead.
// Built into its own library (libbsq_peak.so); bench.py times it with events.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop(float* __restrict__ sink, int64_t iters) {
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
    half8 a, b;
    i32x8 ia, ib;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (_Float16)(threadIdx.x * 0.001f + j);
        b[j] = (_Float16)(blockIdx.x * 0.0001f + j);
        ia[j] = (int)(threadIdx.x * 0x01010101u + j) & 0x37373737;
        ib[j] = (int)(blockIdx.x + j * 0x03030303u) & 0x37373737;
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (KIND == 0) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[i], 0, 0, 0);
            else acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ia, ib, acc[i], 0, 0, 0, 127, 0, 127);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[i][r];
    sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// kind 0: v_mfma_f32_32x32x16_f16 (32768 flops each); kind 1: v_mfma_scale_f32_32x32x64_f8f6f4
// with FP8 E4M3 operands (131072 flops each).  workgroups of 256 threads; sink holds one float
// per thread (workgroups * 256, device).  Returns 0 or a hipError_t.
extern "C" int bsq_peak_mfma_loop(int kind, int64_t workgroups, int64_t iters, float* sink, void* hip_stream) {
    if (workgroups <= 0 || workgroups > 65536 || iters <= 0 || !sink || (kind != 0 && kind != 1)) return (int)hipErrorInvalidValue;
    hipStream_t s = (hipStream_t)hip_stream;
    if (kind == 0) hipLaunchKernelGGL(mfma_loop<0>, dim3((unsigned)workgroups), dim3(256), 0, s, sink, iters);
    else hipLaunchKernelGGL(mfma_loop<1>, dim3((unsigned)workgroups), dim3(256), 0, s, sink, iters);
    return (int)hipGetLastError();
}
