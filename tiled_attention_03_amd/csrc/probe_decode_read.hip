// Read ceiling of the decode's access pattern: measurement only, not part of
// the library's entry points (built into libta03_probe.so, which only the
// benchmark loads).
//
// The kernel reads exactly the bytes the decode kernel reads, in the same
// way: the decode's grid (the split count of its plan for this device, one
// block row per (kv head, head block)), 64-key units dealt round-robin to the
// active splits, the same per-lane K and V load shapes (16-byte loads, 64
// contiguous bytes of 16 key rows per K instruction, whole V rows per V
// instruction), two register sets per wave both in flight before the first
// wait and each refilled as soon as it is consumed, the last pair peeled. It
// does no attention arithmetic and no merge: each set is folded into one sum
// that is stored only when the caller passes a non-zero flag (the benchmark
// passes 0; the stores exist so the loads cannot be dropped). The cache
// length is a kernel argument (no device-side position read), or, when a
// kv_pos pointer is given, read from device memory first exactly as the
// decode reads it (min(*kv_pos + 1, max_seq)), so the two timings separate
// the cost of that round trip from the cost of the decode's arithmetic and
// merge.
//
// C entry point:
//   int ta03_probe_decode_read(const float* k_cache, const float* v_cache,
//                              const uint32_t* kv_pos, int kv_len,
//                              int num_heads, int num_kv_heads,
//                              int head_dim, int max_seq, int store,
//                              float* sink, size_t sink_floats,
//                              hipStream_t stream)
// kv_pos: NULL (use kv_len) or a device uint32 (kv_len is then ignored).
// k_cache, v_cache: [max_seq, num_kv_heads * head_dim] device f32, 16-byte
// aligned; sink: device floats, at least ta03_probe_decode_read_sink_floats()
// of the same sizes (written only when store != 0). Returns 0, or -2 for
// invalid sizes, -4 for a short sink, -5 for a failed launch.

#include <hip/hip_runtime.h>

#include "ta03_internal.h"

namespace ta03 {
namespace {

constexpr int kWaves = 4;
constexpr int kBlock = 64 * kWaves;
constexpr int kT = 16 * kWaves;   // keys per unit (16 per wave), as the decode
constexpr int kKW = kT / kWaves;  // keys per wave per unit

struct ProbeArgs {
    const uint32_t* kv_pos;  // nullptr: kv_len
    int num_kv_heads, kv_len, max_seq, n_splits, blks_per_kv, store;
};

template <int D>
__global__ void __launch_bounds__(kBlock)
decode_read_kernel(const float* __restrict__ k, const float* __restrict__ v,
                   float* __restrict__ sink, ProbeArgs a) {
    constexpr int QT = D / 16;    // K float4 loads per lane per set
    constexpr int LPR = D / 4;    // lanes per V row
    constexpr int KR = 64 / LPR;  // V rows per load instruction
    constexpr int VK = kKW / KR;  // V float4 loads per lane per set

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kv_head = blockIdx.y / a.blks_per_kv;
    const int j = lane & 3;
    const int sl = (lane >> 2) & 3;
    const int kg = lane >> 4;

    int c1 = a.kv_len;
    if (a.kv_pos != nullptr) {
        const unsigned long long len = (unsigned long long)(*a.kv_pos) + 1ull;
        c1 = (int)(len < (unsigned long long)a.max_seq ? len : (unsigned long long)a.max_seq);
    }
    const int n_units = (c1 + kT - 1) / kT;
    const int half = n_units / 2 > 1 ? n_units / 2 : 1;
    const int n_active = half < a.n_splits ? half : a.n_splits;
    const int split = blockIdx.x;
    if (split >= n_active) return;
    const int kvdim = a.num_kv_heads * D;
    const int n_mine = (n_units - split + n_active - 1) / n_active;
    const int n_pairs = (n_mine + 1) / 2;
    const float* kbase = k + kv_head * D;
    const float* vbase = v + kv_head * D;

    auto gload = [&](float4 (&kx)[QT], float4 (&vx)[VK], int u) {
        const int wbase = (split + u * n_active) * kT + wave * kKW;
        const long long key = min(wbase + 4 * kg + j, c1 - 1);
        const float* kp = kbase + (size_t)key * kvdim + 4 * sl;
#pragma unroll
        for (int t = 0; t < QT; ++t) kx[t] = *reinterpret_cast<const float4*>(kp + 16 * t);
#pragma unroll
        for (int t = 0; t < VK; ++t) {
            const long long vkey = min(wbase + t + VK * (lane / LPR), c1 - 1);
            vx[t] = *reinterpret_cast<const float4*>(vbase + (size_t)vkey * kvdim + 4 * (lane % LPR));
        }
    };
    float acc = 0.f;
    auto consume = [&](const float4 (&kx)[QT], const float4 (&vx)[VK]) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int t = 0; t < QT; ++t) s0 += (kx[t].x + kx[t].y) + (kx[t].z + kx[t].w);
#pragma unroll
        for (int t = 0; t < VK; ++t) s1 += (vx[t].x + vx[t].y) + (vx[t].z + vx[t].w);
        acc += s0 + s1;
    };

    float4 ka[QT], va[VK], kb[QT], vb[VK];
    gload(ka, va, 0);
    gload(kb, vb, 1);
    int ub = 0;
    for (int pr = 1; pr < n_pairs; ++pr, ub += 2) {
        consume(ka, va);
        gload(ka, va, ub + 2);
        consume(kb, vb);
        gload(kb, vb, ub + 3);
    }
    consume(ka, va);
    consume(kb, vb);
    if (a.store) sink[((size_t)blockIdx.y * gridDim.x + blockIdx.x) * kBlock + tid] = acc;
}

}  // namespace
}  // namespace ta03

extern "C" {

size_t ta03_probe_decode_read_sink_floats(int num_heads, int num_kv_heads, int head_dim,
                                          int max_seq) {
    if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0 || max_seq < 1 ||
        (head_dim != 64 && head_dim != 128))
        return 0;
    ta03::DecodeShape s{num_heads, num_kv_heads, head_dim, max_seq, 1.0f};
    const ta03::DecodePlan p = ta03::decode_plan(s, ta03::device_cu_count());
    return (size_t)p.n_splits * (size_t)num_kv_heads * p.blks_per_kv * ta03::kBlock;
}

int ta03_probe_decode_read(const float* k_cache, const float* v_cache, const uint32_t* kv_pos,
                           int kv_len, int num_heads, int num_kv_heads, int head_dim, int max_seq,
                           int store, float* sink, size_t sink_floats, hipStream_t stream) {
    if (num_heads < 1 || num_kv_heads < 1 || num_heads % num_kv_heads != 0 || max_seq < 1 ||
        (kv_pos == nullptr && (kv_len < 1 || kv_len > max_seq)) || (head_dim != 64 && head_dim != 128) ||
        k_cache == nullptr || v_cache == nullptr || sink == nullptr)
        return -2;
    ta03::DecodeShape s{num_heads, num_kv_heads, head_dim, max_seq, 1.0f};
    const ta03::DecodePlan p = ta03::decode_plan(s, ta03::device_cu_count());
    const size_t need = (size_t)p.n_splits * (size_t)num_kv_heads * p.blks_per_kv * ta03::kBlock;
    if (sink_floats < need) return -4;
    ta03::ProbeArgs a{kv_pos, num_kv_heads, kv_len, max_seq, p.n_splits, p.blks_per_kv, store};
    const dim3 grid((unsigned)p.n_splits, (unsigned)(num_kv_heads * p.blks_per_kv));
    if (head_dim == 128) {
        hipLaunchKernelGGL(ta03::decode_read_kernel<128>, grid, dim3(ta03::kBlock), 0, stream,
                           k_cache, v_cache, sink, a);
    } else {
        hipLaunchKernelGGL(ta03::decode_read_kernel<64>, grid, dim3(ta03::kBlock), 0, stream,
                           k_cache, v_cache, sink, a);
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
