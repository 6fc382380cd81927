// Prefill attention forward on gfx950 f32 matrix cores.
//
// Computes, for every query row i and head h (kv head = h / group),
//   out[i,h] = sum_j softmax_j(scale * <q_i, k_j>) v_j   over j < w_i,
//   lse[i,h] = (max_j s_ij, log sum_j exp(s_ij - max))
// in one pass with online softmax: a running max and sum per row, the output
// accumulator rescaled by exp(old max - new max) as each key tile arrives
// (meganeura attention.wgsl, main: the online update; cera
// attention_prefill.wgsl, main: the per-tile max / correction / sum update).
// Windows: causal w_i = min(start_pos + i + 1, kv_len), otherwise kv_len
// (attention.wgsl header; attention_prefill.wgsl main).
//
// Work decomposition (one 256-thread block = 4 waves of 64 lanes):
//   * a wave owns 32 query rows of one head; the four waves of a block are
//     the query heads of one GQA group on the same rows (or, for small
//     groups, neighbouring 32-row strips of one head), so the block shares
//     every K/V tile it stages;
//   * K/V tiles of 32 keys go HBM -> registers (128-bit, coalesced, one tile
//     ahead) -> LDS; K rows are padded by 4 floats so the transposed 128-bit
//     reads are bank-conflict free;
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x2_f32: each lane then holds one query column and 16
//     of the tile's 32 keys, so the row max and row sum are in-lane plus one
//     exchange with the other half-wave;
//   * O^T += V^T P^T reuses the score registers directly as the B operand:
//     the k-step t of the product pairs the two keys that the accumulator
//     layout put in register t of the two half-waves (the sum over keys does
//     not care about their order), so P never leaves registers;
//   * exp is exp2 with log2(e) folded into the pre-scaled Q;
//   * causal: key tiles past a block's last window are never loaded, tiles
//     inside every row's window skip the mask, and blocks are issued
//     heaviest-first.

#include <hip/hip_runtime.h>

#include "ta03_internal.h"

namespace ta03 {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlock = 256;  // 4 waves
constexpr int kBM = 32;      // query rows per wave
constexpr int kBN = 32;      // keys per tile
constexpr float kNegBig = -1e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row (key) index held by accumulator register r in half-wave hh of a 32x32
// MFMA result: rows 8*(r/4) + 4*hh + r%4.
__device__ __forceinline__ int acc_row(int r, int hh) {
    return 8 * (r >> 2) + 4 * hh + (r & 3);
}

struct Args {
    int q_seq, kv_len, num_heads, num_kv_heads, group;
    int causal, start_pos;
    float qscale;  // scale * log2(e)
    int hg;        // heads per block
    int rs;        // 32-row strips per block
    int n_head_blocks, n_row_blocks;
};

template <int D>
__global__ void __launch_bounds__(kBlock, 2)
prefill_kernel(const float* __restrict__ q, const float* __restrict__ k,
               const float* __restrict__ v, float* __restrict__ out,
               float* __restrict__ lse, Args a) {
    constexpr int KS = D + 4;               // padded K row (floats)
    constexpr int NB = D / 32;              // 32-row blocks of O^T
    constexpr int F4_ROW = D / 4;           // float4 per K/V row
    constexpr int F4_THR = kBN * F4_ROW / kBlock;  // float4 per thread per tile
    static_assert(F4_THR >= 1, "tile too small for the block");

    __shared__ __attribute__((aligned(16))) float Ks[kBN * KS];
    __shared__ __attribute__((aligned(16))) float Vs[kBN * D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31;
    const int hh = lane >> 5;

    const int bid = blockIdx.x;
    const int head_block = bid % a.n_head_blocks;
    const int seq = bid / a.n_head_blocks;
    const int rb = a.causal ? (a.n_row_blocks - 1 - seq) : seq;  // heaviest first

    const int head = head_block * a.hg + wave % a.hg;
    const int strip = wave / a.hg;
    const int row0 = (rb * a.rs + strip) * kBM;
    const int kv_head = head / a.group;
    const int qdim = a.num_heads * D;
    const int kvdim = a.num_kv_heads * D;

    // Keys the block must stage: up to the last row's window.
    const int blk_rows_hi = min((rb + 1) * a.rs * kBM, a.q_seq);
    const int w_block = a.causal ? min(a.start_pos + blk_rows_hi, a.kv_len) : a.kv_len;
    const bool wave_live = row0 < a.q_seq;
    const int w_wave_max = !wave_live ? 0
        : (a.causal ? min(a.start_pos + min(row0 + kBM, a.q_seq), a.kv_len) : a.kv_len);
    const int w_wave_min = a.causal ? min(a.start_pos + row0 + 1, a.kv_len) : a.kv_len;
    const int row = row0 + j;
    const int w_row = a.causal ? min(a.start_pos + row + 1, a.kv_len) : a.kv_len;

    // Q^T operand: lane (j, hh) holds q[row][8*g + 4*hh + c] for k-step 4*g+c.
    float qr[D / 2];
    {
        const bool ok = row < a.q_seq;
        const float* qp = q + (size_t)(ok ? row : 0) * qdim + head * D + 4 * hh;
#pragma unroll
        for (int g = 0; g < D / 8; ++g) {
            float4 x = ok ? *reinterpret_cast<const float4*>(qp + 8 * g)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
            qr[4 * g + 0] = x.x * a.qscale;
            qr[4 * g + 1] = x.y * a.qscale;
            qr[4 * g + 2] = x.z * a.qscale;
            qr[4 * g + 3] = x.w * a.qscale;
        }
    }

    f32x16 o[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
    float m_run = kNegBig;  // log2 units
    float l_run = 0.f;

    const int n_tiles = (w_block + kBN - 1) / kBN;
    float4 kp[F4_THR], vp[F4_THR];
    const float* kbase = k + kv_head * D;
    const float* vbase = v + kv_head * D;

    auto gload = [&](int t) {
        const int kv0 = t * kBN;
#pragma unroll
        for (int it = 0; it < F4_THR; ++it) {
            const int idx = tid + it * kBlock;
            const int r = idx / F4_ROW;
            const int c4 = idx % F4_ROW;
            const int key = kv0 + r;
            if (key < w_block) {
                const size_t off = (size_t)key * kvdim + 4 * c4;
                kp[it] = *reinterpret_cast<const float4*>(kbase + off);
                vp[it] = *reinterpret_cast<const float4*>(vbase + off);
            } else {
                kp[it] = make_float4(0.f, 0.f, 0.f, 0.f);
                vp[it] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    };

    if (n_tiles > 0) gload(0);

    for (int t = 0; t < n_tiles; ++t) {
        __syncthreads();  // the previous tile's readers are done with LDS
#pragma unroll
        for (int it = 0; it < F4_THR; ++it) {
            const int idx = tid + it * kBlock;
            const int r = idx / F4_ROW;
            const int c4 = idx % F4_ROW;
            *reinterpret_cast<float4*>(&Ks[r * KS + 4 * c4]) = kp[it];
            *reinterpret_cast<float4*>(&Vs[r * D + 4 * c4]) = vp[it];
        }
        __syncthreads();
        if (t + 1 < n_tiles) gload(t + 1);  // in flight while this tile computes

        const int kv0 = t * kBN;
        if (kv0 >= w_wave_max) continue;  // wave-uniform: past every row's window

        // S^T = K Q^T for this tile (already in log2 units).
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        const float* kr = Ks + j * KS + 4 * hh;
#pragma unroll
        for (int g = 0; g < D / 8; ++g) {
            const float4 kk = *reinterpret_cast<const float4*>(kr + 8 * g);
            s = mfma32(kk.x, qr[4 * g + 0], s);
            s = mfma32(kk.y, qr[4 * g + 1], s);
            s = mfma32(kk.z, qr[4 * g + 2], s);
            s = mfma32(kk.w, qr[4 * g + 3], s);
        }

        if (kv0 + kBN > w_wave_min) {  // some key of the tile is outside some window
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (kv0 + acc_row(r, hh) >= w_row) s[r] = -INFINITY;
        }

        // Online softmax for query column j.
        float mx = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = __builtin_amdgcn_exp2f(s[r] - m_new);
            ls += s[r];
        }
        ls += __shfl_xor(ls, 32);
        l_run = l_run * corr + ls;
        m_run = m_new;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] *= corr;

        // O^T += V^T P^T: k-step t pairs keys acc_row(t, 0) and acc_row(t, 1).
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
            const float* vr = Vs + acc_row(tt, hh) * D + NB * j;
            if constexpr (NB == 4) {
                const float4 vv = *reinterpret_cast<const float4*>(vr);
                o[0] = mfma32(vv.x, s[tt], o[0]);
                o[1] = mfma32(vv.y, s[tt], o[1]);
                o[2] = mfma32(vv.z, s[tt], o[2]);
                o[3] = mfma32(vv.w, s[tt], o[3]);
            } else {
                const float2 vv = *reinterpret_cast<const float2*>(vr);
                o[0] = mfma32(vv.x, s[tt], o[0]);
                o[1] = mfma32(vv.y, s[tt], o[1]);
            }
        }
    }

    if (!wave_live || row >= a.q_seq) return;

    // Epilogue: O^T block b, register r holds head-dim NB*acc_row(r, hh) + b.
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float* orow = out + (size_t)row * qdim + head * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = acc_row(r, hh);
        if constexpr (NB == 4) {
            *reinterpret_cast<float4*>(orow + 4 * i) =
                make_float4(o[0][r] * inv, o[1][r] * inv, o[2][r] * inv, o[3][r] * inv);
        } else {
            *reinterpret_cast<float2*>(orow + 2 * i) = make_float2(o[0][r] * inv, o[1][r] * inv);
        }
    }
    if (lse != nullptr && hh == 0) {
        float2 pr;
        if (l_run > 0.f) {
            pr = make_float2(m_run * kLn2, __logf(l_run));
        } else {
            pr = make_float2(kNegBig, kNegBig);
        }
        *reinterpret_cast<float2*>(lse + ((size_t)row * a.num_heads + head) * 2) = pr;
    }
}

int gcd_int(int x, int y) {
    while (y) {
        const int t = x % y;
        x = y;
        y = t;
    }
    return x;
}

}  // namespace

hipError_t launch_prefill(const float* q, const float* k, const float* v, float* out,
                          float* lse, const PrefillShape& s, hipStream_t stream) {
    Args a;
    a.q_seq = s.q_seq;
    a.kv_len = s.kv_len;
    a.num_heads = s.num_heads;
    a.num_kv_heads = s.num_kv_heads;
    a.group = s.num_heads / s.num_kv_heads;
    a.causal = s.causal;
    a.start_pos = s.start_pos;
    a.qscale = s.scale * kLog2e;
    a.hg = gcd_int(a.group, 4);
    a.rs = 4 / a.hg;
    a.n_head_blocks = s.num_heads / a.hg;
    a.n_row_blocks = (s.q_seq + a.rs * kBM - 1) / (a.rs * kBM);
    const long long grid = (long long)a.n_head_blocks * a.n_row_blocks;
    if (grid <= 0) return hipSuccess;
    if (s.head_dim == 128) {
        hipLaunchKernelGGL(prefill_kernel<128>, dim3((unsigned)grid), dim3(kBlock), 0, stream,
                           q, k, v, out, lse, a);
    } else {
        hipLaunchKernelGGL(prefill_kernel<64>, dim3((unsigned)grid), dim3(kBlock), 0, stream,
                           q, k, v, out, lse, a);
    }
    return hipGetLastError();
}

}  // namespace ta03
