// Rotary table builder for the rotary prefill instance.
//
// meganeura attention.wgsl leaves the rotation of queries and keys to hooks
// with no formula; the rotation read into them is the rotate-half rotary
// embedding, whose pair e (elements e and e + d/2) turns at position p by
// p * theta^(-2e/d). Entry (p, e) of the table is (cos, sin) of that angle.
// Angles reach thousands of radians at long positions, where a float angle
// would already be off by about 1e-3, so each entry is computed in double
// precision and rounded once to float.

#include <hip/hip_runtime.h>

#include "ta03_internal.h"

namespace ta03 {
namespace {

__global__ void rope_table_kernel(float2* __restrict__ cs, long long n, int half, int head_dim,
                                  double theta) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const long long p = i / half;
    const int e = (int)(i - p * half);
    const double inv_freq = pow(theta, -2.0 * (double)e / (double)head_dim);
    double sn, cn;
    sincos((double)p * inv_freq, &sn, &cn);
    cs[i] = make_float2((float)cn, (float)sn);
}

}  // namespace

hipError_t launch_rope_table(float* cs, int rows, int head_dim, double theta, hipStream_t stream) {
    const int half = head_dim / 2;
    const long long n = (long long)rows * half;
    if (n <= 0) return hipSuccess;
    const long long blocks = (n + 255) / 256;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<float2*>(cs), n, half, head_dim, theta);
    return hipGetLastError();
}

}  // namespace ta03
