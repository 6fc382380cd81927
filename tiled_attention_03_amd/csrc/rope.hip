// Rotary table builder for the rotary prefill instances, and the rotation
// of whole rows by it (keys turned once, for the instance that turns only
// the queries).
//
// meganeura attention.wgsl leaves the rotation of queries and keys to hooks
// with no formula; the rotation read into them is the rotate-half rotary
// embedding, whose pair e (elements e and e + d/2) turns at position p by
// p * theta^(-2e/d). Entry (p, e) of the table is (cos, sin) of that angle.
// Angles reach thousands of radians at long positions, where a float angle
// would already be off by about 1e-3, so each entry is computed in double
// precision and rounded once to float.

#include <hip/hip_runtime.h>

#include <algorithm>

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

// Rows turned by the table, once: y[r][h d + e], y[r][h d + e + d/2] from
// the pair (x[r][h d + e], x[r][h d + e + d/2]) at position pos0 + r, the
// same rotate-half form as the prefill's rotary instances. One thread per
// four pairs of one (row, head): two 16-byte loads of x and two of the table,
// two 16-byte stores (memory-bound); a grid of at most kApplyBlocks blocks
// strides over larger inputs. Each thread reads every element it writes, and
// no other, so y may be x itself.
constexpr long long kApplyBlocks = 1 << 16;

__global__ void rope_apply_kernel(const float* x, long long xs, float* y,
                                  long long ys, int heads, int half, int pos0,
                                  const float* __restrict__ cs, long long n) {
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x) {
        const int groups = half / 4;  // four-pair groups per head
        const long long rh = i / groups;
        const int c = (int)(i - rh * groups);
        const long long r = rh / heads;
        const int h = (int)(rh - r * heads);
        const float* xr = x + r * xs + (long long)h * 2 * half + 4 * c;
        const float4 lo = *reinterpret_cast<const float4*>(xr);
        const float4 hi = *reinterpret_cast<const float4*>(xr + half);
        const float* t = cs + (pos0 + r) * 2 * half + 8 * c;  // (cos, sin) of pairs 4c .. 4c + 3
        const float4 c0 = *reinterpret_cast<const float4*>(t);
        const float4 c1 = *reinterpret_cast<const float4*>(t + 4);
        float4 nlo, nhi;
        nlo.x = lo.x * c0.x - hi.x * c0.y;
        nhi.x = hi.x * c0.x + lo.x * c0.y;
        nlo.y = lo.y * c0.z - hi.y * c0.w;
        nhi.y = hi.y * c0.z + lo.y * c0.w;
        nlo.z = lo.z * c1.x - hi.z * c1.y;
        nhi.z = hi.z * c1.x + lo.z * c1.y;
        nlo.w = lo.w * c1.z - hi.w * c1.w;
        nhi.w = hi.w * c1.z + lo.w * c1.w;
        float* yr = y + r * ys + (long long)h * 2 * half + 4 * c;
        *reinterpret_cast<float4*>(yr) = nlo;
        *reinterpret_cast<float4*>(yr + half) = nhi;
    }
}

}  // namespace

hipError_t launch_rope_apply(const float* x, long long x_stride, float* y, long long y_stride,
                             int rows, int heads, int head_dim, int pos0, const float* cs,
                             hipStream_t stream) {
    const int half = head_dim / 2;
    const long long n = (long long)rows * heads * (half / 4);
    if (n <= 0) return hipSuccess;
    const long long blocks = std::min((n + 255) / 256, kApplyBlocks);
    hipLaunchKernelGGL(rope_apply_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       x_stride, y, y_stride, heads, half, pos0, cs, n);
    return hipGetLastError();
}

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
