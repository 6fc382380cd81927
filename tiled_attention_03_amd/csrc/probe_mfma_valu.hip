// Issue-rate probe of the f32 matrix instructions against vector-ALU work:
// measurement only, not part of the library's entry points (built into
// libta03_probe.so, which only the benchmark loads).
//
// Each wave runs `iters` iterations of a fixed instruction mix and the
// benchmark times the launch: mode 1 issues 32 v_mfma_f32_16x16x4_f32 per
// iteration (four independent accumulator chains), mode 2 issues 128
// independent vector FMAs (eight chains), mode 3 issues both in the same
// loop body. With one block of `threads` threads per compute unit, threads /
// 256 waves share each SIMD. If the SIMD overlapped the two kinds of work,
// mode 3 would take about as long as the longer of modes 1 and 2; it takes
// about their sum (see the profiles), which is why every vector instruction
// in the attention kernels' inner loops adds to their time. Every lane stores
// one float of its results (in bounds: out holds blocks * threads floats),
// so no work is dropped.
//
// C entry point:
//   int ta03_probe_mfma_valu(float* out, int blocks, int threads, int iters,
//                            int mode, hipStream_t stream)
// threads: 64..512, a multiple of 64; mode 1, 2 or 3. Returns 0, -2 for
// invalid arguments, -5 for a failed launch.

#include <hip/hip_runtime.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ void __launch_bounds__(512) mfma_valu_kernel(float* __restrict__ out, int iters,
                                                        float x) {
    f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = x * (float)(threadIdx.x + i);
    const float a = x * (float)threadIdx.x, b = x + (float)threadIdx.x;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if constexpr (MODE == 1 || MODE == 3) {
                c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c1, 0, 0, 0);
                c2 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c2, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c3, 0, 0, 0);
            }
            if constexpr (MODE == 2 || MODE == 3) {
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(v[i], a, b);
            }
        }
    }
    float s = c0[0] + c1[1] + c2[2] + c3[3];
#pragma unroll
    for (int i = 0; i < 8; ++i) s += v[i];
    out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" int ta03_probe_mfma_valu(float* out, int blocks, int threads, int iters, int mode,
                                    hipStream_t stream) {
    if (out == nullptr || blocks < 1 || threads < 64 || threads > 512 || threads % 64 != 0 ||
        iters < 1)
        return -2;
    const dim3 grid((unsigned)blocks), block((unsigned)threads);
    switch (mode) {
        case 1:
            hipLaunchKernelGGL(mfma_valu_kernel<1>, grid, block, 0, stream, out, iters, 1e-7f);
            break;
        case 2:
            hipLaunchKernelGGL(mfma_valu_kernel<2>, grid, block, 0, stream, out, iters, 1e-7f);
            break;
        case 3:
            hipLaunchKernelGGL(mfma_valu_kernel<3>, grid, block, 0, stream, out, iters, 1e-7f);
            break;
        default:
            return -2;
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
