// Single-token decode over a KV cache, split along the cache axis.
//
// What it computes is meganeura cached_attention.wgsl (main): one query row
// of num_heads heads attends to cache rows [0, kv_pos] with kv_pos read from
// device memory, GQA map kv_head = head / group, online softmax. The window
// is clamped to the cache length as cera attention_prefill.wgsl clamps its
// causal window.
//
// The page runs one workgroup per head over every cache row in sequence, and
// each head of a GQA group re-reads the same K/V rows. This path is bound by
// HBM bandwidth, so it is built to read each K/V byte once with the chip
// full of requests:
//   * grid (split, kv head x head block); a block reads kv_pos, derives the
//     cache length and its chunk on the device (a recorded launch stays valid
//     as kv_pos grows) and serves up to 4 query heads of one GQA group;
//   * inside a block the 4 waves are independent: wave w owns keys
//     [16w, 16w+16) of every 64-key sub-tile, with its own online-softmax
//     state per head;
//   * K rows go HBM -> registers directly in the score layout: lane (key,
//     quarter) holds interleaved 16-byte pieces of its key (each load
//     instruction covers 64 contiguous bytes of 16 rows) and forms 4-head
//     dot products against Q broadcast from LDS; two DPP quad steps finish
//     them, and max and sum over the wave's 16 keys use DPP mirrors and the
//     row / half-wave swaps (no LDS permutes on the path). Staging K
//     through LDS measured markedly slower here;
//   * V rows go HBM -> registers directly in the P.V layout (lane = 4
//     head-dim columns of one key, 128-bit coalesced);
//   * two register sets per wave, both in flight before the first wait and
//     each refilled as soon as it has been consumed; Q is loaded ahead of
//     them (vector loads complete in issue order);
//   * the 4 waves combine with log-sum-exp weights through LDS and the block
//     publishes one partial (unnormalised row, max, sum) per head with
//     device-scope atomic stores;
//   * the last block of each (kv head, head block) to finish -- found with an
//     atomic ticket taken by one thread once the block's partial stores are
//     complete --
//     merges the group's partials: M = max m_s, L = sum l_s 2^(m_s - M),
//     out = sum 2^(m_s - M) O_s / L, the rescale the online update applies
//     when the running max grows; its loads over the splits are independent
//     and issued together. It then resets the ticket for the next call. One
//     launch per call: on this stack a kernel launch alone costs about as much
//     as streaming 20 MB, and the ticket replaces a second launch.
// Scores are in log2 units (log2(e) folded into the pre-scaled Q; exp2).

#include <hip/hip_runtime.h>

#include "ta03_internal.h"

namespace ta03 {
namespace {

#ifndef TA03_DECODE_WAVES
#define TA03_DECODE_WAVES 4
#endif
constexpr int kWaves = TA03_DECODE_WAVES;
constexpr int kBlock = 64 * kWaves;
constexpr int kT = 16 * kWaves;   // keys per sub-tile (16 per wave)
constexpr int kKW = kT / kWaves;  // keys per wave per sub-tile
constexpr int kG = 4;             // query heads per block
static_assert(kWaves >= kG, "the merge serves one head per wave");
#ifndef TA03_DECODE_TARGET_BLOCKS
#define TA03_DECODE_TARGET_BLOCKS 256
#endif
constexpr int kTargetBlocks = TA03_DECODE_TARGET_BLOCKS;
#ifndef TA03_DECODE_MIN_SUB
#define TA03_DECODE_MIN_SUB 2
#endif
constexpr int kMinChunk = TA03_DECODE_MIN_SUB * kT;  // keys per block at least
constexpr float kNegBig = -1e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Args {
    int num_heads, num_kv_heads, max_seq;
    int group, heads_per_blk, blks_per_kv, n_splits;
    float qscale;  // scale * log2(e)
    size_t cnt_offset;  // floats from ws to the ticket counters
    // Paged cache (table == nullptr: one dense cache). Token t lives in row
    // t % page_size of page table[t / page_size]; page_size is a multiple of
    // 16, so a wave's 16-key slice never straddles two pages.
    const int* table;
    int page_size, num_pages;
};

// Cache length and chunking, derived identically by every block.
__device__ __forceinline__ void chunking(const uint32_t* kv_pos, const Args& a,
                                         int* kv_len, int* chunk, int* n_active) {
    const unsigned long long len = (unsigned long long)(*kv_pos) + 1ull;
    const int L = (int)(len < (unsigned long long)a.max_seq ? len : (unsigned long long)a.max_seq);
    int c = (L + a.n_splits - 1) / a.n_splits;
    c = (c + kT - 1) / kT * kT;
    c = c < kMinChunk ? kMinChunk : c;  // both ping-pong sub-tiles of a wave in flight
    *kv_len = L;
    *chunk = c;
    *n_active = (L + c - 1) / c;
}

// Cross-lane steps that do not go through the LDS permute unit: DPP moves
// inside a row of 16 lanes, and the gfx950 row / half-wave swaps
// (v_permlane16_swap, v_permlane32_swap with both operands x hand each lane
// the pair {x[l], x[l ^ 16]} resp. {x[l % 32], x[l % 32 + 32]}, lower lane
// first, so both partners combine them in the same order).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kRowMirror = 0x140;     // lane i <- 15 - i within a row of 16
constexpr int kRowHalfMirror = 0x141; // lane i <- 7 - i within each half-row

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL,
                                                      0xF, 0xF, false));
}
__device__ __forceinline__ float pair_sum16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float pair_max16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float pair_max32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// Sum and max over the 32 lanes of each half-wave (quad steps, half-row and
// row mirrors, then the row swap); every lane of a half ends with the same
// value.
__device__ __forceinline__ float sum32(float x) {
    x += dpp<kQuadXor1>(x);
    x += dpp<kQuadXor2>(x);
    x += dpp<kRowHalfMirror>(x);
    x += dpp<kRowMirror>(x);
    return pair_sum16(x);
}
__device__ __forceinline__ float max32(float x) {
    x = fmaxf(x, dpp<kQuadXor1>(x));
    x = fmaxf(x, dpp<kQuadXor2>(x));
    x = fmaxf(x, dpp<kRowHalfMirror>(x));
    x = fmaxf(x, dpp<kRowMirror>(x));
    return pair_max16(x);
}

// Split partials cross work-groups (and L2s): written and read with 64-bit
// device-scope atomic accesses (p 8-byte aligned), which go to the
// coherence point.
__device__ __forceinline__ void store_pair(float* p, float lo, float hi) {
    const unsigned long long u =
        ((unsigned long long)__float_as_uint(hi) << 32) | (unsigned long long)__float_as_uint(lo);
    __hip_atomic_store(reinterpret_cast<unsigned long long*>(p), u, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_pair(const float* p) {
    const unsigned long long u =
        __hip_atomic_load(reinterpret_cast<unsigned long long*>(const_cast<float*>(p)),
                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((unsigned)u), __uint_as_float((unsigned)(u >> 32)));
}

// LDS written by this wave's lanes becomes readable by its other lanes: DS
// instructions of one wave execute in order, so waiting for the wave's own
// LDS operations (lgkmcnt = 0; vector memory counters untouched) suffices.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_wave_barrier();
}

template <int D>
__global__ void __launch_bounds__(kBlock)
decode_kernel(const float* __restrict__ q, const float* __restrict__ k,
              const float* __restrict__ v, const uint32_t* __restrict__ kv_pos,
              float* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws,
              Args a) {
    constexpr int QI = D / 16;    // 16-float pieces per K row: K float4 per lane per sub-tile
    constexpr int LPR = D / 4;    // lanes per V row in P.V (one float4 each)
    constexpr int KR = 64 / LPR;  // key groups per wave in P.V
    constexpr int VK = kKW / KR;  // V rows per lane per sub-tile

    __shared__ __attribute__((aligned(16))) float Qs[kG * D];
    __shared__ __attribute__((aligned(16))) float Ps[kWaves][kKW * kG];
    __shared__ __attribute__((aligned(16))) float Ow[kWaves][kG * D];
    __shared__ float Mw[kWaves][kG], Lw[kWaves][kG];
    __shared__ int last_flag;
    extern __shared__ int tbl[];  // this block's slice of the page table (paged cache)

    const int tid = threadIdx.x;
    const int grp = blockIdx.y;  // kv_head * blks_per_kv + hsub
    const int kv_head = grp / a.blks_per_kv;
    const int hsub = grp % a.blks_per_kv;
    const int head0 = kv_head * a.group + hsub * a.heads_per_blk;
    const int nh = min(a.heads_per_blk, a.group - hsub * a.heads_per_blk);

    // Q is loaded first: it does not depend on kv_pos, and vector loads
    // complete in issue order, so waiting for Q further down does not wait
    // for the K/V loads issued after it.
    constexpr int QPT = (kG * D + kBlock - 1) / kBlock;  // Q floats per thread
    float qreg[QPT];
#pragma unroll
    for (int j = 0; j < QPT; ++j) {
        const int i = tid + j * kBlock;
        const int h = i / D;
        qreg[j] = (i < kG * D && h < nh) ? q[(size_t)(head0 + h) * D + (i % D)] : 0.f;
    }

    int kv_len, chunk, n_active;
    chunking(kv_pos, a, &kv_len, &chunk, &n_active);
    const int split = blockIdx.x;
    if (split >= n_active) return;  // whole block: nothing of this cache to read

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kvdim = a.num_kv_heads * D;
    const int c0 = split * chunk;
    const int c1 = min(c0 + chunk, kv_len);

    const float* kbase = k + kv_head * D;
    const float* vbase = v + kv_head * D;

    // Per-lane roles.
    const int kk = lane >> 2;   // scores: key within the wave's 16
    const int qq = lane & 3;    // scores: which 16-byte piece of each 64 bytes
    const int dq = lane % LPR;  // P.V: head-dim float4 index
    const int kr = lane / LPR;  // P.V: key group

    // Paged cache: stage this chunk's table entries in LDS, each clamped to
    // a valid page so that no table content can send a load out of bounds.
    const bool paged = a.table != nullptr;
    const int b0 = paged ? c0 / a.page_size : 0;
    if (paged) {
        const int nb = (c1 - 1) / a.page_size - b0 + 1;
        for (int i = tid; i < nb; i += kBlock)
            tbl[i] = min(max(a.table[b0 + i], 0), a.num_pages - 1);
        __syncthreads();
    }

    // K arrives straight in the score layout: lane (kk, qq) holds the pieces
    // [16 i + 4 qq, +4) of its key for i < QI (each load instruction covers
    // 64 contiguous bytes of 16 rows). V arrives in the P.V layout. Rows past
    // the chunk end are read as the chunk's last row (in bounds, no branch
    // around the load); their scores are masked and their weight is 0. In a
    // paged cache every key of the wave's slice (after that clamp) lies in the
    // page of min(slice start, c1 - 1): one row offset per slice.
    auto gload = [&](float4 (&kx)[QI], float4 (&vx)[VK], int base) {
        const int wbase = base + wave * kKW;
        long long shift = 0;  // physical row - token index
        if (paged) {
            const int blk = min(wbase, c1 - 1) / a.page_size;
            shift = (long long)(tbl[blk - b0] - blk) * a.page_size;
        }
        const long long key = min(wbase + kk, c1 - 1) + shift;
        const float* kp = kbase + (size_t)key * kvdim + 4 * qq;
#pragma unroll
        for (int i = 0; i < QI; ++i) kx[i] = *reinterpret_cast<const float4*>(kp + 16 * i);
#pragma unroll
        for (int i = 0; i < VK; ++i) {
            const long long vkey = min(wbase + kr * VK + i, c1 - 1) + shift;
            vx[i] = *reinterpret_cast<const float4*>(vbase + (size_t)vkey * kvdim + 4 * dq);
        }
    };

    // Both register sets in flight before anything waits. Loads are never
    // behind a branch (rows are clamped into the chunk), so the compiler's
    // wait counts stay exact: waiting for one set never waits for the other.
    float4 ka[QI], va[VK], kb[QI], vb[VK];
    gload(ka, va, c0);
    gload(kb, vb, c0 + kT);

#pragma unroll
    for (int j = 0; j < QPT; ++j) {
        const int i = tid + j * kBlock;
        if (i < kG * D) Qs[i] = qreg[j] * a.qscale;
    }
    __syncthreads();

    float m_run[kG], l_run[kG];
    float4 acc[kG];
#pragma unroll
    for (int h = 0; h < kG; ++h) {
        m_run[h] = kNegBig;
        l_run[h] = 0.f;
        acc[h] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float* ps = Ps[wave];

    auto process = [&](const float4 (&kx)[QI], const float4 (&vx)[VK], int base) {
        // Scores for key kk, 4 heads, over this lane's pieces; a quad
        // shuffle completes the dot products.
        float s[kG];
#pragma unroll
        for (int h = 0; h < kG; ++h) s[h] = 0.f;
#pragma unroll
        for (int i = 0; i < QI; ++i) {
#pragma unroll
            for (int h = 0; h < kG; ++h) {
                const float4 qx = *reinterpret_cast<const float4*>(Qs + h * D + 16 * i + 4 * qq);
                s[h] = fmaf(qx.x, kx[i].x, s[h]);
                s[h] = fmaf(qx.y, kx[i].y, s[h]);
                s[h] = fmaf(qx.z, kx[i].z, s[h]);
                s[h] = fmaf(qx.w, kx[i].w, s[h]);
            }
        }
        const bool valid = base + wave * kKW + kk < c1;
        float p[kG], corr[kG];
#pragma unroll
        for (int h = 0; h < kG; ++h) {
            s[h] += dpp<kQuadXor1>(s[h]);
            s[h] += dpp<kQuadXor2>(s[h]);
            // From here each value is the same on the 4 lanes of its key's
            // quad: the half-row mirror pairs neighbouring keys, the row
            // mirror pairs key pairs, the swaps pair rows and half-waves, so
            // each key enters the max and the sum once.
            const float x = valid ? s[h] : -INFINITY;
            float mx = fmaxf(x, dpp<kRowHalfMirror>(x));
            mx = fmaxf(mx, dpp<kRowMirror>(mx));
            mx = pair_max32(pair_max16(mx));
            const float m_new = fmaxf(m_run[h], mx);
            corr[h] = __builtin_amdgcn_exp2f(m_run[h] - m_new);
            p[h] = __builtin_amdgcn_exp2f(x - m_new);
            float sm = p[h] + dpp<kRowHalfMirror>(p[h]);
            sm += dpp<kRowMirror>(sm);
            sm = pair_sum32(pair_sum16(sm));
            l_run[h] = l_run[h] * corr[h] + sm;
            m_run[h] = m_new;
        }
        if (qq == 0)
            *reinterpret_cast<float4*>(ps + kk * kG) = make_float4(p[0], p[1], p[2], p[3]);
        wave_lds_sync();

        // O += P V over the wave's keys kr*VK .. kr*VK+VK-1, 4 columns per lane.
#pragma unroll
        for (int h = 0; h < kG; ++h) {
            acc[h].x *= corr[h];
            acc[h].y *= corr[h];
            acc[h].z *= corr[h];
            acc[h].w *= corr[h];
        }
#pragma unroll
        for (int i = 0; i < VK; ++i) {
            const float4 pk = *reinterpret_cast<const float4*>(ps + (kr * VK + i) * kG);
            const float pv[kG] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
            for (int h = 0; h < kG; ++h) {
                acc[h].x = fmaf(pv[h], vx[i].x, acc[h].x);
                acc[h].y = fmaf(pv[h], vx[i].y, acc[h].y);
                acc[h].z = fmaf(pv[h], vx[i].z, acc[h].z);
                acc[h].w = fmaf(pv[h], vx[i].w, acc[h].w);
            }
        }
        wave_lds_sync();  // P reads done before the next sub-tile rewrites it
    };

    // Sub-tiles go in pairs, one per register set, each set refilled as soon
    // as it has been consumed, so two sub-tiles per wave stay in flight. The
    // last pair is peeled off (no refills): every iteration of the loop then
    // has the same loads in flight, and nothing is requested that is not
    // used. A sub-tile wholly past the chunk end (an odd count) reads the
    // chunk's last row and contributes nothing: its scores are masked, so its
    // weights are 0 and the running max is kept.
    const int n_pairs = (c1 - c0 + 2 * kT - 1) / (2 * kT);
    int base = c0;
    for (int pr = 1; pr < n_pairs; ++pr, base += 2 * kT) {
        process(ka, va, base);
        gload(ka, va, base + 2 * kT);
        process(kb, vb, base + kT);
        gload(kb, vb, base + 3 * kT);
    }
    process(ka, va, base);
    process(kb, vb, base + kT);

    // Sum the key groups of the wave (same running max within a wave).
#pragma unroll
    for (int h = 0; h < kG; ++h) {
        if constexpr (LPR == 16) {  // key groups in lane bits 4 and 5
            acc[h].x = pair_sum16(acc[h].x);
            acc[h].y = pair_sum16(acc[h].y);
            acc[h].z = pair_sum16(acc[h].z);
            acc[h].w = pair_sum16(acc[h].w);
        }
        static_assert(LPR == 16 || LPR == 32, "head_dim 64 or 128");
        acc[h].x = pair_sum32(acc[h].x);
        acc[h].y = pair_sum32(acc[h].y);
        acc[h].z = pair_sum32(acc[h].z);
        acc[h].w = pair_sum32(acc[h].w);
    }
    if (kr == 0) {
#pragma unroll
        for (int h = 0; h < kG; ++h)
            *reinterpret_cast<float4*>(&Ow[wave][h * D + 4 * dq]) = acc[h];
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < kG; ++h) {
            Mw[wave][h] = m_run[h];
            Lw[wave][h] = l_run[h];
        }
    }
    __syncthreads();

    // Block partial per head: combine the 4 waves with log-sum-exp weights.
    const size_t row = D + 2;
    if (n_active == 1) {
        // One split covers the cache: this block's partial is the result.
        for (int i = tid; i < nh * D; i += kBlock) {
            const int h = i / D, d = i % D;
            float M = Mw[0][h];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, Mw[w][h]);
            float o = 0.f, L = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float wt = __builtin_amdgcn_exp2f(Mw[w][h] - M);
                o = fmaf(Ow[w][h * D + d], wt, o);
                L = fmaf(Lw[w][h], wt, L);
            }
            out[(size_t)(head0 + h) * D + d] = o / L;
            if (lse != nullptr && d == 0) {
                lse[2 * (head0 + h)] = M * kLn2;
                lse[2 * (head0 + h) + 1] = __logf(L);
            }
        }
        return;
    }
    // Two columns per thread, published with 64-bit stores (rows are D + 2
    // floats, so every pair starts 8-byte aligned).
    for (int i = tid; i < nh * D / 2; i += kBlock) {
        const int h = 2 * i / D, d = 2 * i % D;
        float M = Mw[0][h];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, Mw[w][h]);
        float o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float wt = __builtin_amdgcn_exp2f(Mw[w][h] - M);
            o0 = fmaf(Ow[w][h * D + d], wt, o0);
            o1 = fmaf(Ow[w][h * D + d + 1], wt, o1);
        }
        float* part = ws + ((size_t)(head0 + h) * a.n_splits + split) * row;
        store_pair(part + d, o0, o1);
        if (d == 0) {
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) L = fmaf(Lw[w][h], __builtin_amdgcn_exp2f(Mw[w][h] - M), L);
            store_pair(part + D, M, L);
        }
    }

    // Ticket. The partial stores above are device-coherent (agent-scope
    // atomic stores write through to the coherence point); each wave waits
    // for their completion (vmcnt = 0) before the block barrier, so when
    // thread 0's atomic increment is performed every partial of this block
    // is visible to any agent-scope load. The last block reads the partials
    // with agent-scope atomic loads, which are served from the coherence
    // point. No L2-wide write-back or invalidate is needed (a release/acquire
    // ticket would issue one per block, which costs more than the merge).
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are complete
    __syncthreads();
    unsigned int* cnt = reinterpret_cast<unsigned int*>(ws + a.cnt_offset) + blockIdx.y;
    if (tid == 0) {
        const unsigned int t = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
        last_flag = t == (unsigned int)(n_active - 1);
    }
    __syncthreads();
    if (!last_flag) return;

    // Merge: wave h serves head head0 + h, each lane D/64 columns. Splits go
    // in batches of 32: lane j (and j + 32) loads the (max, sum) pair of
    // split j of the batch, every lane loads its columns of all 32 partial
    // rows (33 loads, one round trip), the batch max and the weights
    // w_j = 2^(m_j - M) come from cross-lane steps, and each w_j reaches the
    // column sums through a lane read. Across batches the running (M, L, o)
    // is rescaled as in the online update. Indices past the last split are
    // clamped to it (no load sits behind a branch) and their weight is 0.
    if (wave < nh) {
        constexpr int DPL = D / 64;
        constexpr int NB = 32;
        const int head = head0 + wave;
        const float* hb = ws + (size_t)head * a.n_splits * row;
        const int lj = lane & (NB - 1);
        float M = kNegBig, L = 0.f, o[DPL];
#pragma unroll
        for (int c = 0; c < DPL; ++c) o[c] = 0.f;
        for (int s0 = 0; s0 < n_active; s0 += NB) {
            const bool live = s0 + lj < n_active;
            const float2 ml = load_pair(hb + (size_t)min(s0 + lj, n_active - 1) * row + D);
            float ov[NB][DPL];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const float* p = hb + (size_t)min(s0 + j, n_active - 1) * row + lane * DPL;
                if constexpr (DPL == 2) {
                    const float2 x = load_pair(p);
                    ov[j][0] = x.x;
                    ov[j][1] = x.y;
                } else {
                    ov[j][0] = __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            const float mj = live ? ml.x : kNegBig;
            const float bm = fmaxf(M, max32(mj));
            const float r = __builtin_amdgcn_exp2f(M - bm);
            M = bm;
            const float wj = live ? __builtin_amdgcn_exp2f(mj - M) : 0.f;
            L = fmaf(L, r, sum32(ml.y * wj));
#pragma unroll
            for (int c = 0; c < DPL; ++c) o[c] *= r;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), j));
#pragma unroll
                for (int c = 0; c < DPL; ++c) o[c] = fmaf(ov[j][c], w, o[c]);
            }
        }
        const float inv = 1.0f / L;
#pragma unroll
        for (int c = 0; c < DPL; ++c) out[(size_t)head * D + lane * DPL + c] = o[c] * inv;
        if (lse != nullptr && lane == 0) {
            lse[2 * head] = M * kLn2;
            lse[2 * head + 1] = __logf(L);
        }
    }
    if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void zero_counters_kernel(unsigned int* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace

DecodePlan decode_plan(const DecodeShape& s) {
    DecodePlan p;
    p.group = s.num_heads / s.num_kv_heads;
    p.heads_per_blk = p.group < kG ? p.group : kG;
    p.blks_per_kv = (p.group + p.heads_per_blk - 1) / p.heads_per_blk;
    const long long rows = (long long)s.num_kv_heads * p.blks_per_kv;
    long long n = (kTargetBlocks + rows - 1) / rows;
    const long long max_useful = (s.max_seq + kT - 1) / kT;
    if (n > max_useful) n = max_useful;
    if (n < 1) n = 1;
    p.n_splits = (int)n;
    const size_t part = (size_t)s.num_heads * (size_t)p.n_splits * (size_t)(s.head_dim + 2);
    p.cnt_offset = (part + 3) / 4 * 4;  // counters start 16-byte aligned
    p.n_counters = (size_t)rows;
    p.ws_floats = p.cnt_offset + (p.n_counters + 3) / 4 * 4;
    return p;
}

hipError_t launch_decode_ws_init(float* ws, const DecodePlan& p, hipStream_t stream) {
    unsigned int* c = reinterpret_cast<unsigned int*>(ws + p.cnt_offset);
    const int n = (int)p.n_counters;
    hipLaunchKernelGGL(zero_counters_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, c, n);
    return hipGetLastError();
}

size_t decode_table_lds_bytes(const DecodeShape& s, const DecodePlan& p, int page_size) {
    // The largest chunk any kv_pos can give (the cache full), as chunking()
    // computes it, and the table entries a chunk can touch.
    long long c = ((long long)s.max_seq + p.n_splits - 1) / p.n_splits;
    c = (c + kT - 1) / kT * kT;
    if (c < kMinChunk) c = kMinChunk;
    return (size_t)(c / page_size + 2) * sizeof(int);
}

hipError_t launch_decode(const float* q, const float* k, const float* v,
                         const uint32_t* kv_pos, float* out, float* lse,
                         const DecodeShape& s, const DecodePlan& p, float* ws,
                         hipStream_t stream, const int* table, int page_size, int num_pages) {
    Args a;
    a.num_heads = s.num_heads;
    a.num_kv_heads = s.num_kv_heads;
    a.max_seq = s.max_seq;
    a.group = p.group;
    a.heads_per_blk = p.heads_per_blk;
    a.blks_per_kv = p.blks_per_kv;
    a.n_splits = p.n_splits;
    a.qscale = s.scale * kLog2e;
    a.cnt_offset = p.cnt_offset;
    a.table = table;
    a.page_size = page_size;
    a.num_pages = num_pages;
    const size_t lds = table != nullptr ? decode_table_lds_bytes(s, p, page_size) : 0;
    const dim3 grid((unsigned)p.n_splits, (unsigned)(s.num_kv_heads * p.blks_per_kv));
    if (s.head_dim == 128) {
        hipLaunchKernelGGL(decode_kernel<128>, grid, dim3(kBlock), lds, stream, q, k, v, kv_pos,
                           out, lse, ws, a);
    } else {
        hipLaunchKernelGGL(decode_kernel<64>, grid, dim3(kBlock), lds, stream, q, k, v, kv_pos,
                           out, lse, ws, a);
    }
    return hipGetLastError();
}

}  // namespace ta03
