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
// full of requests and as little work as possible between a load's arrival
// and its refill:
//   * the cache is cut into units of 64 keys dealt round-robin to the
//     splits (split s takes units s, s + n, s + 2n, ... of the n active
//     splits), so at any moment the chip streams neighbouring rows rather
//     than rows 1 MiB apart; a block reads kv_pos and derives the cache
//     length and its units on the device (a recorded launch stays valid as
//     kv_pos grows) and serves up to 4 query heads of one GQA group;
//   * inside a block the 4 waves are independent: wave w owns keys
//     [16w, 16w+16) of every unit, with its own online-softmax state;
//   * both products run on the matrix cores as v_mfma_f32_4x4x1_16b_f32
//     (16 independent 4x4 blocks, so the 4 heads of a group fill every
//     column): S = K Q^T with K rows straight from HBM as the A operand
//     (each load instruction covers 64 contiguous bytes of 16 rows) and Q
//     in registers as the B operand, four head-dim slices in four blocks
//     summed by two DPP row rotations; then O^T += V^T P with V rows
//     straight from HBM as the A operand (whole rows per instruction) and P
//     as the B operand -- each lane already holds the weights of its head
//     (column), and one row-pair swap hands it the keys its V rows hold.
//     The vector ALU keeps only the softmax of one head per lane;
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

#include <mutex>

#include "ta03_internal.h"

// Scratch of the allocation-free decode entry point (attn_decode_noalloc):
// one copy per device, held until the process ends. Host code never names
// it directly: the array's name on the host is a stand-in, not a device
// address, so its device address is looked up once per device
// (hipGetSymbolAddress) and that pointer is what the kernels get. Layout: a
// fixed counter region of kNoallocCounterWords words (one ticket slot per
// (kv head, head block), zero-filled once per device, left at zero by every
// call), then the split partials.
static __device__ __align__(256) float scratch[ta03::kNoallocScratchFloats];

namespace ta03 {
namespace {

#ifndef TA03_DECODE_WAVES
#define TA03_DECODE_WAVES 4
#endif
constexpr int kWaves = TA03_DECODE_WAVES;
constexpr int kBlock = 64 * kWaves;
constexpr int kT = 16 * kWaves;   // keys per unit (16 per wave)
constexpr int kKW = kT / kWaves;  // keys per wave per unit
constexpr int kG = 4;             // query heads per block
static_assert(kWaves >= kG, "the merge serves one head per wave");
// The completion counters sit 256 bytes apart: side by side in one line, the
// atomics of all 256 blocks serialised on it (the last ticket of a call came
// ~1.4 us after its block's stores; 17.2 -> 16.6 us at an 8192-row cache).
constexpr int kCntStride = 64;  // words between ticket counters
constexpr float kNegBig = -1e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Args {
    int num_heads, num_kv_heads, max_seq;
    int group, heads_per_blk, blks_per_kv, n_splits;
    float qscale;  // scale * log2(e)
    size_t part_offset;  // floats from ws to the split partials (the counters come first)
    // Paged cache (table == nullptr: one dense cache). Token t lives in row
    // t % page_size of page table[t / page_size]; page_size is a multiple of
    // 16, so a wave's 16-key slice never straddles two pages.
    const int* table;
    int page_size, num_pages;
};

// Cache length, unit count and active splits, derived identically by every
// block.
__device__ __forceinline__ void chunking(const uint32_t* kv_pos, const Args& a,
                                         int* kv_len, int* n_units, int* n_active) {
    const unsigned long long len = (unsigned long long)(*kv_pos) + 1ull;
    const int L = (int)(len < (unsigned long long)a.max_seq ? len : (unsigned long long)a.max_seq);
    *kv_len = L;
    *n_units = (L + kT - 1) / kT;
    // Two units per active split at least (both register sets of a wave
    // carry data), at most n_splits splits; split s takes units s,
    // s + n_active, s + 2 n_active, ...
    const int half = *n_units / 2 > 1 ? *n_units / 2 : 1;
    *n_active = half < a.n_splits ? half : a.n_splits;
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
constexpr int kRowRor4 = 0x124;       // lane i <- lane (i - 4) mod 16 within a row
constexpr int kRowRor8 = 0x128;       // lane i <- lane (i - 8) mod 16 within a row

typedef float v4f __attribute__((ext_vector_type(4)));

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

template <int D>
__global__ void __launch_bounds__(kBlock)
decode_kernel(const float* __restrict__ q, const float* __restrict__ k,
              const float* __restrict__ v, const uint32_t* __restrict__ kv_pos,
              float* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws,
              Args a) {
    constexpr int QT = D / 16;    // K float4 loads per lane per set (16 dims per load row)
    constexpr int LPR = D / 4;    // lanes per V row (one float4 each)
    constexpr int KR = 64 / LPR;  // V rows per load instruction
    constexpr int VK = kKW / KR;  // V float4 loads per lane per set
    static_assert(LPR == 16 || LPR == 32, "head_dim 64 or 128");

    __shared__ __attribute__((aligned(16))) float Ow[kWaves][kG * D];
    __shared__ float Mw[kWaves][kG], Lw[kWaves][kG];
    __shared__ int last_flag;
    extern __shared__ int tbl[];  // this block's page-table entries (paged cache)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = blockIdx.y;  // kv_head * blks_per_kv + hsub
    const int kv_head = grp / a.blks_per_kv;
    const int hsub = grp % a.blks_per_kv;
    const int head0 = kv_head * a.group + hsub * a.heads_per_blk;
    const int nh = min(a.heads_per_blk, a.group - hsub * a.heads_per_blk);

    // Lane roles. Matrix blocks are lanes 4b..4b+3; column j = lane % 4 is
    // the query head head0 + j throughout. Scores: block b = 4 kg + sl holds
    // keys 4 kg .. 4 kg + 3 (rows) over the head-dim slice sl.
    const int j = lane & 3;
    const int sl = (lane >> 2) & 3;
    const int kg = lane >> 4;

    // Q first (it does not depend on kv_pos): lane (sl, j) keeps head j's
    // elements 16 t + 4 sl + c, pre-scaled, as the B operand of the score
    // products. Heads past the block's count are zero.
    float4 qr[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const float* qp = q + (size_t)(head0 + j) * D + 16 * t + 4 * sl;
        qr[t] = j < nh ? *reinterpret_cast<const float4*>(qp) : make_float4(0.f, 0.f, 0.f, 0.f);
    }

    int kv_len, n_units, n_active;
    chunking(kv_pos, a, &kv_len, &n_units, &n_active);
    const int split = blockIdx.x;
    if (split >= n_active) return;  // whole block: nothing of this cache to read

    const int kvdim = a.num_kv_heads * D;
    const int c1 = kv_len;
    const int n_mine = (n_units - split + n_active - 1) / n_active;  // units of this block
    const int n_pairs = (n_mine + 1) / 2;

    const float* kbase = k + kv_head * D;
    const float* vbase = v + kv_head * D;

    const bool paged = a.table != nullptr;
    if (paged) {
        // Entry u * kWaves + w: the page of wave w's 16-key slice of the
        // block's unit u (slices past the cache read its last row, as the
        // loads do), clamped to a valid page.
        for (int i = tid; i < 2 * n_pairs * kWaves; i += kBlock) {
            const int tok = min((split + (i / kWaves) * n_active) * kT + (i % kWaves) * kKW, c1 - 1);
            tbl[i] = min(max(a.table[tok / a.page_size], 0), a.num_pages - 1);
        }
        __syncthreads();
    }

    // K arrives as the A operand of the score products: lane (kg, sl, i)
    // holds key 4 kg + i, elements [16 t + 4 sl, +4) (each load instruction
    // covers 64 contiguous bytes of 16 rows). V arrives as the A operand of
    // the P.V products: lane l holds elements [4 (l % LPR), +4) of key
    // t + (kKW / KR)(l / LPR) (each instruction KR whole rows). Rows past the
    // cache are read as its last row (in bounds, no branch around the
    // load); their scores are masked and their weight is 0.
    auto gload = [&](float4 (&kx)[QT], float4 (&vx)[VK], int u) {
        const int wbase = (split + u * n_active) * kT + wave * kKW;
        long long shift = 0;  // physical row - token index
        if (paged) {
            const int blk = min(wbase, c1 - 1) / a.page_size;
            shift = (long long)(tbl[u * kWaves + wave] - blk) * a.page_size;
        }
        const long long key = min(wbase + 4 * kg + j, c1 - 1) + shift;
        const float* kp = kbase + (size_t)key * kvdim + 4 * sl;
#pragma unroll
        for (int t = 0; t < QT; ++t) kx[t] = *reinterpret_cast<const float4*>(kp + 16 * t);
#pragma unroll
        for (int t = 0; t < VK; ++t) {
            const long long vkey = min(wbase + t + VK * (lane / LPR), c1 - 1) + shift;
            vx[t] = *reinterpret_cast<const float4*>(vbase + (size_t)vkey * kvdim + 4 * (lane % LPR));
        }
    };

    float4 ka[QT], va[VK], kb[QT], vb[VK];
    gload(ka, va, 0);
    gload(kb, vb, 1);
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        qr[t].x *= a.qscale;
        qr[t].y *= a.qscale;
        qr[t].z *= a.qscale;
        qr[t].w *= a.qscale;
    }

    // Online-softmax state of head j (the same in every lane of column j)
    // and the unnormalised output: oc[c] register i = element
    // 16 (b % (LPR / 4)) + 4 i + c of head j, b = lane / 4, summed over the
    // key groups of the lane's V rows.
    float m_run = kNegBig, l_run = 0.f;
    v4f oc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) oc[c] = v4f{0.f, 0.f, 0.f, 0.f};

    auto process = [&](const float4 (&kx)[QT], const float4 (&vx)[VK], int u) {
        const int wbase = (split + u * n_active) * kT + wave * kKW;
        // S (keys x heads) on the matrix cores, two accumulators in turn.
        v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < QT; ++t) {
            s0 = __builtin_amdgcn_mfma_f32_4x4x1f32(kx[t].x, qr[t].x, s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_4x4x1f32(kx[t].y, qr[t].y, s1, 0, 0, 0);
            s0 = __builtin_amdgcn_mfma_f32_4x4x1f32(kx[t].z, qr[t].z, s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_4x4x1f32(kx[t].w, qr[t].w, s1, 0, 0, 0);
        }
        // Sum the four head-dim slices (lanes 4 apart in each row of 16):
        // register r of lane (kg, sl, j) is then the score of key 4 kg + r
        // for head j.
        float x[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float sc = s0[r] + s1[r];
            sc += dpp<kRowRor4>(sc);
            sc += dpp<kRowRor8>(sc);
            x[r] = wbase + 4 * kg + r < c1 ? sc : -INFINITY;
        }
        float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
        mx = pair_max32(pair_max16(mx));
        const float m_new = fmaxf(m_run, mx);
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(x[r] - m_new);
        const float sm = pair_sum32(pair_sum16((p[0] + p[1]) + (p[2] + p[3])));
        l_run = l_run * corr + sm;
        m_run = m_new;

        // P as the B operand: the weight of head j for the key that the
        // lane's V rows hold in load t (key t + VK (lane / LPR)).
        float pb[VK];
        if constexpr (LPR == 32) {
            // Keys t + 8 h for the half h: the row pair's even row holds
            // keys 8 h + r, its odd row 8 h + 4 + r.
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const auto e = __builtin_amdgcn_permlane16_swap(__float_as_uint(p[r]),
                                                                __float_as_uint(p[r]), false, false);
                pb[r] = __uint_as_float(e[0]);
                pb[4 + r] = __uint_as_float(e[1]);
            }
        } else {
            // Keys t + 4 kg: the lane's own registers.
#pragma unroll
            for (int r = 0; r < 4; ++r) pb[r] = p[r];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) oc[c] *= corr;
#pragma unroll
        for (int t = 0; t < VK; ++t) {
            oc[0] = __builtin_amdgcn_mfma_f32_4x4x1f32(vx[t].x, pb[t], oc[0], 0, 0, 0);
            oc[1] = __builtin_amdgcn_mfma_f32_4x4x1f32(vx[t].y, pb[t], oc[1], 0, 0, 0);
            oc[2] = __builtin_amdgcn_mfma_f32_4x4x1f32(vx[t].z, pb[t], oc[2], 0, 0, 0);
            oc[3] = __builtin_amdgcn_mfma_f32_4x4x1f32(vx[t].w, pb[t], oc[3], 0, 0, 0);
        }
    };

    // Units go in pairs, one per register set, each set refilled as soon as
    // it has been consumed, so two units per wave stay in flight. The last
    // pair is peeled off (no refills). A unit past the block's count (an odd
    // count) reads the cache's last row and contributes nothing: its scores
    // are masked, so its weights are 0 and the running max is kept.
    int ub = 0;
    for (int pr = 1; pr < n_pairs; ++pr, ub += 2) {
        process(ka, va, ub);
        gload(ka, va, ub + 2);
        process(kb, vb, ub + 1);
        gload(kb, vb, ub + 3);
    }
    process(ka, va, ub);
    process(kb, vb, ub + 1);

    // Sum the key groups of the wave's V rows (lane bits 4-5 for head_dim
    // 64, bit 5 for 128); every running max of the wave is the same.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float o = oc[c][r];
            if constexpr (LPR == 16) o = pair_sum16(o);
            oc[c][r] = pair_sum32(o);
        }
    }
    if (lane < LPR) {
        const int b = lane >> 2;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            *reinterpret_cast<float4*>(&Ow[wave][j * D + 16 * b + 4 * r]) =
                make_float4(oc[0][r], oc[1][r], oc[2][r], oc[3][r]);
    }
    if (lane < kG) {
        Mw[wave][j] = m_run;
        Lw[wave][j] = l_run;
    }
    __syncthreads();

    // Block partial per head: combine the 4 waves with log-sum-exp weights.
    const size_t row = D + 4;
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
    // Two columns per thread, published with 64-bit stores. A partial row is
    // D + 4 floats (the output row, then max and sum, then two pad floats), so
    // rows start 16-byte aligned for the merge's 128-bit loads.
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
        float* part = ws + a.part_offset + ((size_t)(head0 + h) * a.n_splits + split) * row;
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
    unsigned int* cnt = reinterpret_cast<unsigned int*>(ws) + (size_t)blockIdx.y * kCntStride;
    if (tid == 0) {
        const unsigned int t = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
        last_flag = t == (unsigned int)(n_active - 1);
    }
    __syncthreads();
    if (!last_flag) return;

    // Merge: wave h serves head head0 + h. Splits go in batches of 32: lane
    // j (and j + 32) loads the (max, sum) pair of split j of the batch; the
    // partial rows come in 16-byte loads, lane l taking columns
    // 4 (l % (D/4)) .. + 3 of split slot l / (D/4), so one instruction covers
    // 64 / (D/4) splits (17 or 9 loads per lane per batch, one round trip;
    // 64-bit loads of 2 columns per split took 33). The batch max and the
    // weights w_j = 2^(m_j - M) come from cross-lane steps, each w_j reaches
    // the lanes of its slot through lane reads, and the slots are summed at
    // the end by half-row / half-wave swaps. Across batches the running
    // (M, L, o) is rescaled as in the online update. Indices past the last
    // split are clamped to it (no load sits behind a branch) and their
    // weight is 0. The partial loads are buffer loads with the sc1 policy:
    // coherent with the other blocks' agent-scope stores (a line this XCD's
    // L2 kept from an earlier call is not used), like the agent-scope atomic
    // loads of the (max, sum) pairs.
    if (wave < nh) {
        constexpr int LPS = D / 4;     // lanes per split row (one float4 each)
        constexpr int SPI = 64 / LPS;  // splits per load instruction
        constexpr int NB = 32;
        const int head = head0 + wave;
        const float* hb = ws + a.part_offset + (size_t)head * a.n_splits * row;
        const int lj = lane & (NB - 1);
        const int sub = lane / LPS;
        const int c4 = 4 * (lane % LPS);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(hb), 0, (int)(a.n_splits * row * 4), 0x00020000);
        float M = kNegBig, L = 0.f;
        float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int s0 = 0; s0 < n_active; s0 += NB) {
            const bool live = s0 + lj < n_active;
            const float2 ml = load_pair(hb + (size_t)min(s0 + lj, n_active - 1) * row + D);
            float4 ov[NB / SPI];
#pragma unroll
            for (int i = 0; i < NB / SPI; ++i) {
                const int s = min(s0 + i * SPI + sub, n_active - 1);
                const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, (s * (int)row + c4) * 4, 0, 16);
                ov[i] = make_float4(__int_as_float(x[0]), __int_as_float(x[1]), __int_as_float(x[2]),
                                    __int_as_float(x[3]));
            }
            const float mj = live ? ml.x : kNegBig;
            const float bm = fmaxf(M, max32(mj));
            const float r = __builtin_amdgcn_exp2f(M - bm);
            M = bm;
            const float wj = live ? __builtin_amdgcn_exp2f(mj - M) : 0.f;
            L = fmaf(L, r, sum32(ml.y * wj));
            o.x *= r; o.y *= r; o.z *= r; o.w *= r;
#pragma unroll
            for (int i = 0; i < NB / SPI; ++i) {
                float w = 0.f;
#pragma unroll
                for (int q2 = 0; q2 < SPI; ++q2) {
                    const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), i * SPI + q2));
                    w = sub == q2 ? wq : w;
                }
                o.x = fmaf(ov[i].x, w, o.x);
                o.y = fmaf(ov[i].y, w, o.y);
                o.z = fmaf(ov[i].z, w, o.z);
                o.w = fmaf(ov[i].w, w, o.w);
            }
        }
        // sum over the SPI split slots (lane groups LPS apart)
        if constexpr (SPI == 4) {
            o.x = pair_sum16(o.x); o.y = pair_sum16(o.y); o.z = pair_sum16(o.z); o.w = pair_sum16(o.w);
        }
        o.x = pair_sum32(o.x); o.y = pair_sum32(o.y); o.z = pair_sum32(o.z); o.w = pair_sum32(o.w);
        const float inv = 1.0f / L;
        if (lane < LPS)
            *reinterpret_cast<float4*>(out + (size_t)head * D + c4) =
                make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
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

DecodePlan decode_plan(const DecodeShape& s, int target_blocks) {
    DecodePlan p;
    p.group = s.num_heads / s.num_kv_heads;
    p.heads_per_blk = p.group < kG ? p.group : kG;
    p.blks_per_kv = (p.group + p.heads_per_blk - 1) / p.heads_per_blk;
    const long long rows = (long long)s.num_kv_heads * p.blks_per_kv;
    // About one block per compute unit.
    long long n = (target_blocks + rows - 1) / rows;
    const long long max_useful = (s.max_seq + kT - 1) / kT;
    if (n > max_useful) n = max_useful;
    if (n < 1) n = 1;
    p.n_splits = (int)n;
    // The counters first (their region depends on the head counts only, so
    // a zero fill needs no split count), then the partials.
    p.n_counters = (size_t)rows * kCntStride;
    p.part_offset = p.n_counters;
    const size_t part = (size_t)s.num_heads * (size_t)p.n_splits * (size_t)(s.head_dim + 4);
    p.ws_floats = p.part_offset + (part + kCntStride - 1) / kCntStride * kCntStride;
    return p;
}

hipError_t launch_decode_ws_init(float* ws, const DecodePlan& p, hipStream_t stream) {
    unsigned int* c = reinterpret_cast<unsigned int*>(ws);
    const int n = (int)p.n_counters;
    hipLaunchKernelGGL(zero_counters_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, c, n);
    return hipGetLastError();
}

namespace {
std::mutex g_scratch_mu;
float* g_scratch_ptr[64];  // per device: device address of `scratch`, zero-filled counters
}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, float** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        // The counters must start at zero: one fill kernel on the caller's
        // stream, ahead of the first decode there (no memset node).
        const int n = (int)kNoallocCounterWords;
        hipLaunchKernelGGL(zero_counters_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           stream, static_cast<unsigned int*>(p), n);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

size_t decode_table_lds_bytes(const DecodeShape& s, const DecodePlan& p, int page_size) {
    // One entry per wave slice of each unit a block can take (the cache
    // full), the unit count rounded up to the pairs the loop runs.
    (void)page_size;
    // A block takes at most ceil(units / n_splits) units, or 3 when fewer
    // splits are active than n_splits.
    const long long units = ((long long)s.max_seq + kT - 1) / kT;
    long long cnt = (units + p.n_splits - 1) / p.n_splits;
    if (cnt < 3) cnt = 3;
    cnt = (cnt + 1) / 2 * 2;
    return (size_t)(cnt * kWaves) * sizeof(int);
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
    a.part_offset = p.part_offset;
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
