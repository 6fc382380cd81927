// Prefill attention forward for launches with few query rows: 16-row waves
// on v_mfma_f32_16x16x4_f32, operands straight from memory into registers.
//
// Same computation as prefill.hip (meganeura attention.wgsl, main: the
// online update; cera attention_prefill.wgsl, main: windows continued from
// start_pos) and the same outputs. The 32-row kernel shares K/V tiles through
// LDS between the waves of a block; with few query rows (short or cross
// sequences, a continuation batch) its blocks are too few and LDS caps them at
// one per CU. This kernel trades that sharing for parallelism:
//   * a wave owns 16 query rows of one head; a block of 8 waves is, in some
//     mix, query heads of a GQA group, row strips of one head, and up to 8
//     splits of the key range, merged through LDS at the end;
//   * no K/V tiles in LDS: each 16-key tile goes HBM/L2 -> registers straight
//     into the operand layouts, one tile ahead of its use (waves of a block
//     that read the same keys meet in the L1 cache);
//   * S^T = K Q^T: lane (j, g) of a 16x16x4 product supplies key/query j and
//     k index g; k-step 4c + e with index g carries head-dim element
//     16c + 4g + e (the k order of a dot product is free), so each 16-byte
//     load instruction c of a key tile reads 64 contiguous bytes of each of
//     its 16 key rows (one half cache line per row; the order g*D/4 + s,
//     64 bytes apart per lane, touched two lines per row and measured ~1%
//     slower on the cross 512x2048 workload);
//   * O^T += V^T P^T: k-step t with index g pairs key 4g + t, which is
//     exactly register t of the score result in that lane, so P never leaves
//     registers; O^T block b row m is head-dim (D/16)*m + b, so a lane reads
//     D/16 contiguous floats of one V row per k-step;
//   * row max and sum: in-lane over 4 keys plus two lane-pair exchanges
//     (v_permlane16_swap, v_permlane32_swap); exp is exp2 with log2(e)
//     folded into the scaled Q.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ta03_internal.h"

namespace ta03 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kBlock = 64 * kWaves;
constexpr int kRows = 16;  // query rows per wave
constexpr int kKeys = 16;  // keys per tile
constexpr int kWavesPerCU = 8;  // two waves per SIMD
constexpr float kNegBig = -1e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRefSlack = 8.0f;  // log2 units: weights stay <= 256 between reference moves

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// All-reduce over lane pairs with one vector instruction (no LDS round trip):
// v_permlane16_swap / v_permlane32_swap with both operands x hand each lane
// the pair {x[l], x[l ^ 16]} resp. {x[l % 32], x[l % 32 + 32]} (lower lane
// first, so both partners combine them in the same order).
__device__ __forceinline__ float pair_max16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum16(float x) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float pair_max32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

__device__ __forceinline__ float comp(const float4& x, int i) {
    return i == 0 ? x.x : (i == 1 ? x.y : (i == 2 ? x.z : x.w));
}

struct Args16 {
    int q_seq, kv_len, num_heads, group;
    int causal, start_pos;
    float qscale;  // scale * log2(e)
    long long q_stride, k_stride, v_stride, out_stride;
    int hg, rs, ks;  // block: heads x row strips x key splits = 8 waves
    int n_head_blocks, n_row_blocks;
};

template <int D>
struct Tile {
    float4 kx[D / 16];  // K[key j][16c + 4g .. +4) in kx[c]
    float4 vx[D / 16];  // V[key 4g + t][(D/16)*j .. +D/16), t-major
};

template <int D>
__global__ void __launch_bounds__(kBlock, D == 64 ? 2 : 1)
prefill16_kernel(const float* __restrict__ q, const float* __restrict__ k,
                 const float* __restrict__ v, float* __restrict__ out,
                 float* __restrict__ lse, Args16 a) {
    constexpr int KS = D / 4;   // k-steps of the score product
    constexpr int NB = D / 16;  // 16-row blocks of O^T
    extern __shared__ __attribute__((aligned(16))) float smem[];  // key-split partials

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;
    const int g = lane >> 4;

    const int bid = blockIdx.x;
    const int head_block = bid % a.n_head_blocks;
    const int seq = bid / a.n_head_blocks;
    const int rb = a.causal ? (a.n_row_blocks - 1 - seq) : seq;  // heaviest first
    const int kvs = wave % a.ks;
    const int rest = wave / a.ks;
    const int head = head_block * a.hg + rest % a.hg;
    const int strip = rest / a.hg;
    const int row0 = (rb * a.rs + strip) * kRows;
    const int kv_head = head / a.group;

    const int row = row0 + j;
    const bool ok = row < a.q_seq;
    const bool wave_live = row0 < a.q_seq;
    const int w_row = a.causal ? min(a.start_pos + row + 1, a.kv_len) : a.kv_len;
    const int w_max = !wave_live ? 0
        : (a.causal ? min(a.start_pos + min(row0 + kRows, a.q_seq), a.kv_len) : a.kv_len);

    const int n_tiles = (w_max + kKeys - 1) / kKeys;
    const int nt = (n_tiles + a.ks - 1) / a.ks;
    const int t_begin = kvs * nt;
    const int t_end = min(t_begin + nt, n_tiles);

    // Q^T operand: lane (j, g) holds q[row][16c + 4g + e] * scale*log2(e)
    // in register 4c + e (k-step 4c + e).
    float qr[KS];
    {
        const float* qp = q + (size_t)(ok ? row : 0) * a.q_stride + head * D + 4 * g;
#pragma unroll
        for (int c = 0; c < KS / 4; ++c) {
            const float4 x = ok ? *reinterpret_cast<const float4*>(qp + 16 * c)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            qr[4 * c + 0] = x.x * a.qscale;
            qr[4 * c + 1] = x.y * a.qscale;
            qr[4 * c + 2] = x.z * a.qscale;
            qr[4 * c + 3] = x.w * a.qscale;
        }
    }

    f32x4 o[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) o[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Online softmax against a reference max (log2 units), as in the 32-row
    // kernel: the score products start from -m_ref, so they give s - m_ref
    // and p = exp2 of the result, and the reference (with O and the sum)
    // moves only when some lane's score passes its row's reference by more
    // than kRefSlack, or a row sees its first keys: one wave-wide vote per
    // tile. A row's 16 keys of a tile sit in four lanes; each lane keeps its
    // own running max above the reference (rel) and its own partial sum, and
    // the row's are formed across the four lanes only when the reference
    // moves and once after the last tile. Before a row has a reference,
    // m_ref is 0, thr is -inf and rel is -inf.
    float m_ref = 0.f;
    float thr = -INFINITY;  // kRefSlack once the row has a reference
    float rel = -INFINITY;
    float l_part = 0.f;
    f32x4 negm = f32x4{0.f, 0.f, 0.f, 0.f};

    const float* kbase = k + kv_head * D;
    const float* vbase = v + kv_head * D;
    // Key tiles are read through buffer resources whose base is the tile's
    // first row and whose size covers the rows before the wave's last window
    // (scalar work per tile): each lane's byte offsets are the same for every
    // tile, so a tile's loads cost no vector instructions for addresses, and
    // rows past the window read as zero (their scores are masked and their
    // weight is 0). K: row j, elements 16c + 4g (c in the instruction
    // offset); V: row 4g + tt, elements NB j.
    const unsigned kvo = (unsigned)(j * a.k_stride + 4 * g) * 4u;
    unsigned vvo[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) vvo[tt] = (unsigned)((4 * g + tt) * a.v_stride + NB * j) * 4u;
    auto load = [&](Tile<D>& T, int t) {
        const int kv0 = t * kKeys;
        const int rows = min(kKeys, w_max - kv0);
        const auto rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(kbase + (size_t)kv0 * a.k_stride), 0, rows * (int)a.k_stride * 4,
            kBufferFlags);
        const auto rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(vbase + (size_t)kv0 * a.v_stride), 0, rows * (int)a.v_stride * 4,
            kBufferFlags);
#pragma unroll
        for (int c = 0; c < KS / 4; ++c) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rk, kvo + 64u * c, 0, 0);
            T.kx[c] = make_float4(__int_as_float(x[0]), __int_as_float(x[1]), __int_as_float(x[2]),
                                  __int_as_float(x[3]));
        }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int c = 0; c < NB / 4; ++c) {
                const auto x = __builtin_amdgcn_raw_buffer_load_b128(rv, vvo[tt] + 16u * c, 0, 0);
                T.vx[tt * (NB / 4) + c] = make_float4(__int_as_float(x[0]), __int_as_float(x[1]),
                                                      __int_as_float(x[2]), __int_as_float(x[3]));
            }
        }
    };

    auto compute = [&](const Tile<D>& T, int t, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int kv0 = t * kKeys;
        // S^T - m_ref: row 4g + r is key kv0 + 4g + r, column j the query.
        f32x4 s = negm;
#pragma unroll
        for (int st = 0; st < KS; ++st) s = mfma16(comp(T.kx[st / 4], st % 4), qr[st], s);
        // The window mask as a select (a branch here would put a block edge
        // between the last product and the first vector read of its result,
        // where the wait the matrix unit's result needs was found missing in
        // the generated code); tiles inside every row's window run a version
        // without it.
        if constexpr (MASKED) {
#pragma unroll
            for (int r = 0; r < 4; ++r) s[r] = kv0 + 4 * g + r < w_row ? s[r] : -INFINITY;
        }
        const float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        rel = fmaxf(rel, mx);
        if (__builtin_amdgcn_ballot_w64(mx > thr) != 0ull) {
            // Every row takes its running max as the new reference. A row
            // with a reference had one lane at rel = 0 after its last move, so
            // its shift is >= 0 and the correction <= 1; a row without one
            // has O and the sum still 0.
            const float rrow = pair_max32(pair_max16(rel));
            const bool seen = rrow > -INFINITY;
            const float shift = seen ? rrow : 0.f;
            const float corr = thr > -INFINITY ? __builtin_amdgcn_exp2f(-shift) : 0.f;
#pragma unroll
            for (int b = 0; b < NB; ++b) o[b] *= corr;
            l_part *= corr;
#pragma unroll
            for (int r = 0; r < 4; ++r) s[r] -= shift;
            m_ref += shift;
            rel -= shift;
            thr = thr > -INFINITY || seen ? kRefSlack : -INFINITY;
            negm = f32x4{-m_ref, -m_ref, -m_ref, -m_ref};
        }
        // The tile's sum first, then one add to the lane's running sum.
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] = __builtin_amdgcn_exp2f(s[r]);
        l_part += (s[0] + s[1]) + (s[2] + s[3]);
        __builtin_amdgcn_s_setprio(1);
        // O^T += V^T P^T: k-step tt pairs key 4g + tt with register tt. At
        // raised wave priority, so the SIMD's other wave fills the gaps with
        // its softmax (as in the 32-row kernel; ~0.5% on the cross workload).
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int b = 0; b < NB; ++b)
                o[b] = mfma16(comp(T.vx[tt * (NB / 4) + b / 4], b % 4), s[tt], o[b]);
        __builtin_amdgcn_s_setprio(0);
    };

    // Two register tiles, the next one in flight while the current one is
    // consumed; loads never sit behind a branch inside a loop, so each wait
    // covers exactly the tile it needs. The tiles inside every row's window
    // (those before w_min) go first, in a loop without mask code; the rest
    // follow with the mask. Each loop body is straight-line from the score
    // products to the softmax.
    const int w_min = a.causal ? min(a.start_pos + row0 + 1, a.kv_len) : a.kv_len;
    const int t_int = w_min / kKeys;  // tiles before it need no mask
    const std::false_type plain;
    const std::true_type masked;
    if (t_begin < t_end) {
        Tile<D> A, B;
        load(A, t_begin);
        int t = t_begin;
        for (; t + 2 < t_end && t + 1 < t_int; t += 2) {
            load(B, t + 1);
            compute(A, t, plain);
            load(A, t + 2);
            compute(B, t + 1, plain);
        }
        for (; t + 2 < t_end; t += 2) {
            load(B, t + 1);
            compute(A, t, masked);
            load(A, t + 2);
            compute(B, t + 1, masked);
        }
        if (t + 1 < t_end) {
            load(B, t + 1);
            compute(A, t, masked);
            compute(B, t + 1, masked);
        } else {
            compute(A, t, masked);
        }
    }

    // The row's (max, sum) pair from its four lanes' parts: max = m_ref +
    // the lanes' max above the reference, the sum and O rescaled to it
    // (selects, no branch: O holds matrix-core results).
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
    float m_run, l_run;
    {
        const float rrow = pair_max32(pair_max16(rel));
        const float lrow = pair_sum32(pair_sum16(l_part));
        const bool seen = rrow > -INFINITY;
        const float f = seen ? __builtin_amdgcn_exp2f(-rrow) : 0.f;
        m_run = seen ? m_ref + rrow : kNegBig;
        l_run = lrow * f;
#pragma unroll
        for (int b = 0; b < NB; ++b) o[b] *= f;
    }

    if (a.ks > 1) {
        // Key splits 1.. publish (m, l, O) through LDS in register order,
        // split 0 rescales and adds.
        // Per lane, contiguous: (m, l, -, -), then O block b (4 + 4 NB floats,
        // an odd number of 16-byte chunks: conflict-free 128-bit accesses).
        constexpr int PART = 4 + 4 * NB;
        float4* part = reinterpret_cast<float4*>(smem) + ((size_t)wave * 64 + lane) * (PART / 4);
        if (kvs > 0) {
            part[0] = make_float4(m_run, l_run, 0.f, 0.f);
#pragma unroll
            for (int b = 0; b < NB; ++b) part[1 + b] = make_float4(o[b][0], o[b][1], o[b][2], o[b][3]);
        }
        __syncthreads();
        if (kvs > 0) return;
        for (int p = 1; p < a.ks; ++p) {
            const float4* pp =
                reinterpret_cast<const float4*>(smem) + ((size_t)(wave + p) * 64 + lane) * (PART / 4);
            const float4 ml = pp[0];
            const float M = fmaxf(m_run, ml.x);
            const float f0 = __builtin_amdgcn_exp2f(m_run - M);
            const float f1 = __builtin_amdgcn_exp2f(ml.x - M);
            l_run = l_run * f0 + ml.y * f1;
            m_run = M;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float4 x = pp[1 + b];
                o[b][0] = o[b][0] * f0 + x.x * f1;
                o[b][1] = o[b][1] * f0 + x.y * f1;
                o[b][2] = o[b][2] * f0 + x.z * f1;
                o[b][3] = o[b][3] * f0 + x.w * f1;
            }
        }
    }

    if (!ok) return;
    // O^T block b, register r of lane (j, g): head-dim NB*(4g + r) + b.
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float* orow = out + (size_t)row * a.out_stride + head * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int c = 0; c < NB / 4; ++c) {
            *reinterpret_cast<float4*>(orow + NB * (4 * g + r) + 4 * c) =
                make_float4(o[4 * c + 0][r] * inv, o[4 * c + 1][r] * inv,
                            o[4 * c + 2][r] * inv, o[4 * c + 3][r] * inv);
        }
    }
    if (lse != nullptr && g == 0) {
        float2 pr;
        if (l_run > 0.f) {
            pr = make_float2(m_run * kLn2, __logf(l_run));
        } else {
            pr = make_float2(kNegBig, kNegBig);
        }
        *reinterpret_cast<float2*>(lse + ((size_t)row * a.num_heads + head) * 2) = pr;
    }
}

int gcd16(int x, int y) {
    while (y) {
        const int t = x % y;
        x = y;
        y = t;
    }
    return x;
}

template <int D>
hipError_t launch16(long long grid, size_t lds, hipStream_t stream, const float* q,
                    const float* k, const float* v, float* out, float* lse, const Args16& a) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(prefill16_kernel<D>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        kWaves * (4 + D / 4) * 64 * (int)sizeof(float));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((prefill16_kernel<D>), dim3((unsigned)grid), dim3(kBlock), lds, stream, q,
                       k, v, out, lse, a);
    return hipSuccess;
}

}  // namespace

hipError_t launch_prefill16(const float* q, const float* k, const float* v, float* out,
                            float* lse, const PrefillShape& s, hipStream_t stream) {
    Args16 a;
    a.q_seq = s.q_seq;
    a.kv_len = s.kv_len;
    a.num_heads = s.num_heads;
    a.group = s.num_heads / s.num_kv_heads;
    a.causal = s.causal;
    a.start_pos = s.start_pos;
    a.qscale = s.scale * kLog2e;
    a.q_stride = s.q_stride;
    a.k_stride = s.k_stride;
    a.v_stride = s.v_stride;
    a.out_stride = s.out_stride;

    // Key splits until the launch has about two waves per SIMD, each split
    // keeping at least two key tiles.
    const int strips = (s.q_seq + kRows - 1) / kRows;
    const long long base_waves = (long long)s.num_heads * strips;
    const int max_w = s.causal ? min(s.start_pos + s.q_seq, s.kv_len) : s.kv_len;
    const int key_tiles = (max_w + kKeys - 1) / kKeys;
    int ks = 1;
    const long long target_waves = (long long)kWavesPerCU * device_cu_count();
    while (ks < kWaves && base_waves * ks < target_waves && key_tiles >= 2 * ks * 2) ks *= 2;
    a.ks = ks;
    a.hg = gcd16(a.group, kWaves / ks);
    a.rs = kWaves / (ks * a.hg);
    a.n_head_blocks = s.num_heads / a.hg;
    a.n_row_blocks = (s.q_seq + a.rs * kRows - 1) / (a.rs * kRows);
    const long long grid = (long long)a.n_head_blocks * a.n_row_blocks;
    if (grid <= 0) return hipSuccess;
    const size_t lds = ks > 1 ? (size_t)kWaves * (4 + s.head_dim / 4) * 64 * sizeof(float) : 0;
    hipError_t e = s.head_dim == 128
        ? launch16<128>(grid, lds, stream, q, k, v, out, lse, a)
        : launch16<64>(grid, lds, stream, q, k, v, out, lse, a);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace ta03
