// Single-token decode over a KV cache, split along the cache axis.
//
// What it computes is meganeura cached_attention.wgsl (main): one query row
// of num_heads heads attends to cache rows [0, kv_pos] with kv_pos read from
// device memory, GQA map kv_head = head / group, online softmax. The window
// is clamped to the cache length as cera attention_prefill.wgsl clamps its
// causal window.
//
// The page runs one workgroup per head over every cache row in sequence, and
// every head of a GQA group reads the same K/V rows again. Here the path is
// bandwidth-bound, so it is organised around reading each K/V byte once with
// the whole chip busy:
//   1. split kernel: grid (split, kv-head x head-block). A block reads kv_pos,
//      derives the cache length and its chunk on the device (so a recorded
//      launch stays valid as kv_pos grows), streams its chunk of K and V once
//      in 64-row sub-tiles (128-bit coalesced loads, one sub-tile ahead in
//      registers, staged through LDS), and serves up to 4 query heads of the
//      group from each staged tile: wave w computes head w's scores (lane =
//      key), its tile max / sum with in-wave shuffles, and its P.V partial
//      (lane = two head-dim columns). It writes an unnormalised partial row
//      and its (max, sum) per head and split to the workspace.
//   2. merge kernel: per head, combine the active splits' partials with
//      log-sum-exp weights: M = max m_s, L = sum l_s 2^(m_s - M),
//      out = sum 2^(m_s - M) O_s / L -- the same rescale the online update
//      applies when a tile raises the running max.

#include <hip/hip_runtime.h>

#include "ta03_internal.h"

namespace ta03 {
namespace {

constexpr int kBlock = 256;
constexpr int kT = 64;           // keys per sub-tile
constexpr int kMaxHeads = 4;     // query heads per block
constexpr int kTargetBlocks = 1024;
constexpr float kNegBig = -1e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Args {
    int num_heads, num_kv_heads, head_dim, max_seq;
    int group, heads_per_blk, blks_per_kv, n_splits;
    float qscale;  // scale * log2(e)
};

// Cache length and chunking, derived identically by both kernels.
__device__ __forceinline__ void chunking(const uint32_t* kv_pos, const Args& a,
                                         int* kv_len, int* chunk, int* n_active) {
    const unsigned long long len = (unsigned long long)(*kv_pos) + 1ull;
    const int L = (int)(len < (unsigned long long)a.max_seq ? len : (unsigned long long)a.max_seq);
    int c = (L + a.n_splits - 1) / a.n_splits;
    c = (c + kT - 1) / kT * kT;
    *kv_len = L;
    *chunk = c;
    *n_active = (L + c - 1) / c;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

template <int D>
__global__ void __launch_bounds__(kBlock)
decode_split_kernel(const float* __restrict__ q, const float* __restrict__ k,
                    const float* __restrict__ v, const uint32_t* __restrict__ kv_pos,
                    float* __restrict__ ws, Args a) {
    constexpr int KS = D + 4;
    constexpr int F4_ROW = D / 4;
    constexpr int F4_THR = kT * F4_ROW / kBlock;  // 8 (D=128) or 4 (D=64)
    constexpr int DPL = D / 64;                   // head-dim columns per lane in P.V

    __shared__ __attribute__((aligned(16))) float Ks[kT * KS];
    __shared__ __attribute__((aligned(16))) float Vs[kT * D];
    __shared__ __attribute__((aligned(16))) float Qs[kMaxHeads * D];
    __shared__ float Ps[kMaxHeads * kT];

    int kv_len, chunk, n_active;
    chunking(kv_pos, a, &kv_len, &chunk, &n_active);
    const int split = blockIdx.x;
    if (split >= n_active) return;  // whole block: nothing to read

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kv_head = blockIdx.y / a.blks_per_kv;
    const int hsub = blockIdx.y % a.blks_per_kv;
    const int head0 = kv_head * a.group + hsub * a.heads_per_blk;
    const int nh = min(a.heads_per_blk, a.group - hsub * a.heads_per_blk);
    const int kvdim = a.num_kv_heads * D;
    const int c0 = split * chunk;
    const int c1 = min(c0 + chunk, kv_len);

    for (int i = tid; i < nh * D; i += kBlock) Qs[i] = q[(size_t)head0 * D + i] * a.qscale;

    const float* kbase = k + kv_head * D;
    const float* vbase = v + kv_head * D;
    float4 kp[F4_THR], vp[F4_THR];
    auto gload = [&](int base) {
#pragma unroll
        for (int it = 0; it < F4_THR; ++it) {
            const int idx = tid + it * kBlock;
            const int r = idx / F4_ROW;
            const int c4 = idx % F4_ROW;
            const int key = base + r;
            if (key < c1) {
                const size_t off = (size_t)key * kvdim + 4 * c4;
                kp[it] = *reinterpret_cast<const float4*>(kbase + off);
                vp[it] = *reinterpret_cast<const float4*>(vbase + off);
            } else {
                kp[it] = make_float4(0.f, 0.f, 0.f, 0.f);
                vp[it] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    };

    const bool active = wave < nh;
    float m_run = kNegBig, l_run = 0.f;
    float acc[DPL];
#pragma unroll
    for (int c = 0; c < DPL; ++c) acc[c] = 0.f;

    gload(c0);
    for (int base = c0; base < c1; base += kT) {
        __syncthreads();
#pragma unroll
        for (int it = 0; it < F4_THR; ++it) {
            const int idx = tid + it * kBlock;
            const int r = idx / F4_ROW;
            const int c4 = idx % F4_ROW;
            *reinterpret_cast<float4*>(&Ks[r * KS + 4 * c4]) = kp[it];
            *reinterpret_cast<float4*>(&Vs[r * D + 4 * c4]) = vp[it];
        }
        __syncthreads();
        if (base + kT < c1) gload(base + kT);

        if (active) {
            // Scores: lane = key of the sub-tile, wave = head.
            const int key = base + lane;
            const float* qh = Qs + wave * D;
            const float* kr = Ks + lane * KS;
            float s = 0.f;
#pragma unroll
            for (int d = 0; d < D; d += 4) {
                const float4 kk = *reinterpret_cast<const float4*>(kr + d);
                const float4 qq = *reinterpret_cast<const float4*>(qh + d);
                s = fmaf(qq.x, kk.x, s);
                s = fmaf(qq.y, kk.y, s);
                s = fmaf(qq.z, kk.z, s);
                s = fmaf(qq.w, kk.w, s);
            }
            if (key >= c1) s = -INFINITY;
            const float m_new = fmaxf(m_run, wave_max(s));
            const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
            const float p = __builtin_amdgcn_exp2f(s - m_new);
            l_run = l_run * corr + wave_sum(p);
            m_run = m_new;
            Ps[wave * kT + lane] = p;
#pragma unroll
            for (int c = 0; c < DPL; ++c) acc[c] *= corr;
        }
        __syncthreads();
        if (active) {
            const float* pw = Ps + wave * kT;
#pragma unroll 8
            for (int r = 0; r < kT; ++r) {
                const float p = pw[r];
                if constexpr (DPL == 2) {
                    const float2 vv = *reinterpret_cast<const float2*>(Vs + r * D + 2 * lane);
                    acc[0] = fmaf(p, vv.x, acc[0]);
                    acc[1] = fmaf(p, vv.y, acc[1]);
                } else {
                    acc[0] = fmaf(p, Vs[r * D + lane], acc[0]);
                }
            }
        }
    }

    if (!active) return;
    const int head = head0 + wave;
    float* part = ws + ((size_t)head * a.n_splits + split) * (D + 2);
    if constexpr (DPL == 2) {
        *reinterpret_cast<float2*>(part + 2 * lane) = make_float2(acc[0], acc[1]);
    } else {
        part[lane] = acc[0];
    }
    if (lane == 0) {
        part[D] = m_run;
        part[D + 1] = l_run;
    }
}

template <int D>
__global__ void __launch_bounds__(D)
decode_merge_kernel(const uint32_t* __restrict__ kv_pos, const float* __restrict__ ws,
                    float* __restrict__ out, float* __restrict__ lse, Args a) {
    int kv_len, chunk, n_active;
    chunking(kv_pos, a, &kv_len, &chunk, &n_active);
    const int head = blockIdx.x;
    const int t = threadIdx.x;
    const float* base = ws + (size_t)head * a.n_splits * (D + 2);

    float M = kNegBig;
    for (int s = 0; s < n_active; ++s) M = fmaxf(M, base[(size_t)s * (D + 2) + D]);
    float L = 0.f, o = 0.f;
    for (int s = 0; s < n_active; ++s) {
        const float* p = base + (size_t)s * (D + 2);
        const float w = __builtin_amdgcn_exp2f(p[D] - M);
        L = fmaf(p[D + 1], w, L);
        o = fmaf(p[t], w, o);
    }
    out[(size_t)head * D + t] = o / L;
    if (lse != nullptr && t == 0) {
        lse[2 * head] = M * kLn2;
        lse[2 * head + 1] = __logf(L);
    }
}

Args make_args(const DecodeShape& s, const DecodePlan& p) {
    Args a;
    a.num_heads = s.num_heads;
    a.num_kv_heads = s.num_kv_heads;
    a.head_dim = s.head_dim;
    a.max_seq = s.max_seq;
    a.group = p.group;
    a.heads_per_blk = p.heads_per_blk;
    a.blks_per_kv = p.blks_per_kv;
    a.n_splits = p.n_splits;
    a.qscale = s.scale * kLog2e;
    return a;
}

}  // namespace

DecodePlan decode_plan(const DecodeShape& s) {
    DecodePlan p;
    p.group = s.num_heads / s.num_kv_heads;
    p.heads_per_blk = p.group < kMaxHeads ? p.group : kMaxHeads;
    p.blks_per_kv = (p.group + p.heads_per_blk - 1) / p.heads_per_blk;
    const long long rows = (long long)s.num_kv_heads * p.blks_per_kv;
    long long n = (kTargetBlocks + rows - 1) / rows;
    const long long max_useful = (s.max_seq + kT - 1) / kT;
    if (n > max_useful) n = max_useful;
    if (n < 1) n = 1;
    p.n_splits = (int)n;
    p.ws_floats = (size_t)s.num_heads * (size_t)p.n_splits * (size_t)(s.head_dim + 2);
    return p;
}

hipError_t launch_decode(const float* q, const float* k, const float* v,
                         const uint32_t* kv_pos, float* out, float* lse,
                         const DecodeShape& s, const DecodePlan& p, float* ws,
                         hipStream_t stream) {
    const Args a = make_args(s, p);
    const dim3 grid1((unsigned)p.n_splits, (unsigned)(s.num_kv_heads * p.blks_per_kv));
    if (s.head_dim == 128) {
        hipLaunchKernelGGL(decode_split_kernel<128>, grid1, dim3(kBlock), 0, stream,
                           q, k, v, kv_pos, ws, a);
        hipLaunchKernelGGL(decode_merge_kernel<128>, dim3((unsigned)s.num_heads), dim3(128), 0,
                           stream, kv_pos, ws, out, lse, a);
    } else {
        hipLaunchKernelGGL(decode_split_kernel<64>, grid1, dim3(kBlock), 0, stream,
                           q, k, v, kv_pos, ws, a);
        hipLaunchKernelGGL(decode_merge_kernel<64>, dim3((unsigned)s.num_heads), dim3(64), 0,
                           stream, kv_pos, ws, out, lse, a);
    }
    return hipGetLastError();
}

}  // namespace ta03
