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
//   * a wave owns 32 query rows of one head and one share of the key range.
//     The 4 waves of a block are, in some mix, query heads of one GQA group
//     on the same rows (they share every staged K/V tile), neighbouring
//     32-row strips of one head (they share the tiles too), and key-range
//     splits of the same rows (used when the grid would otherwise leave CUs
//     idle; their partial rows are merged through LDS at the end, so no
//     workspace is needed);
//   * K/V tiles of 32 keys go HBM -> LDS directly (global_load_lds, 16 bytes
//     per lane, no staging registers), double-buffered with one barrier per
//     tile. Rows past the block's window are loaded as its last row (always
//     in bounds; their scores are masked and their weight is 0). Each K row's
//     16-byte chunks are XOR-swizzled by the row index so that the transposed
//     128-bit reads of the score product are bank-conflict free;
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
//     heaviest-first;
//   * rotary embedding (a separate template instance): meganeura
//     attention.wgsl turns each query and key element through hooks as it
//     loads them, without giving the rotation. Here it is the rotate-half
//     form, angle p * theta^(-2e/d) from a (cos, sin) table: the query is
//     turned in registers right after loading (element e and its partner
//     e + d/2 sit in the same lane of the operand layout); keys go HBM ->
//     registers -> turned -> LDS, one tile ahead of their use, while V keeps
//     the direct path. A third instance turns the queries only, for keys
//     already turned in memory (a rotated cache, or attn_rope_apply once per
//     call): its tile loop is the plain one.

#include <hip/hip_runtime.h>

#include <type_traits>

#include "ta03_internal.h"

namespace ta03 {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBlock = 256;  // 4 waves
constexpr int kWaves = 4;
constexpr int kBM = 32;      // query rows per wave
constexpr int kBN = 32;      // keys per tile
constexpr int kWavesPerCU = 8;  // two waves per SIMD
constexpr float kNegBig = -1e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRefSlack = 8.0f;  // log2 units: weights stay <= 256 between reference moves

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row (key) index held by accumulator register r in half-wave hh of a 32x32
// MFMA result: rows 8*(r/4) + 4*hh + r%4.
__device__ __forceinline__ int acc_row(int r, int hh) {
    return 8 * (r >> 2) + 4 * hh + (r & 3);
}

// All-reduce over the two half-waves with one vector instruction (no LDS
// round trip): v_permlane32_swap with both operands x hands each lane the
// pair {x[l % 32], x[l % 32 + 32]} (lower lane first, so both partners
// combine them in the same order).
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

__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's tile loads have landed
}

struct Args {
    const float* rope_cs;  // rotary (cos, sin) table [positions][D/2][2] (rotary instance)
    int q_seq, kv_len, num_heads, num_kv_heads, group;
    int causal, start_pos;
    float qscale;  // scale * log2(e)
    long long q_stride, k_stride, v_stride, out_stride;  // row strides (floats)
    int small_strides;  // 32 * 4 * max(k_stride, v_stride) < 2^31: 32-bit tile byte offsets
    int hg;        // heads per block
    int rs;        // 32-row strips per block
    int ks;        // key-range splits per block
    int n_head_blocks, n_row_blocks;
};

// Rotary modes of the kernel: none, queries and keys rotated as they are
// loaded, queries only (keys already rotated in memory).
constexpr int kRopeNone = 0, kRopeQK = 1, kRopeQ = 2;

// Rotary instance: most chunk-pair load instructions one wave issues per key
// tile (the host keeps the key splits low enough for this).
template <int D>
constexpr int rope_rmax() { return D == 128 ? 2 : 4; }

// Two blocks per CU while their LDS (KS * D * 512 bytes) allows it.
template <int D, int ROPE, int KS>
__global__ void __launch_bounds__(kBlock, KS * D <= 128 ? 2 : 1)
prefill_kernel(const float* __restrict__ q, const float* __restrict__ k,
               const float* __restrict__ v, float* __restrict__ out,
               float* __restrict__ lse, Args a) {
    // Rotary modes: keys rotated as they are loaded (ROPE == kRopeQK), or
    // queries only, the keys taken as given (kRopeQ).
    constexpr bool ROT_K = ROPE == kRopeQK;
    constexpr int NB = D / 32;                // 32-row blocks of O^T
    constexpr int CPR = D / 4;                // 16-byte chunks per K/V row
    constexpr int TILE_F = kBN * D;           // floats per K (or V) tile
    constexpr int TILE_CHUNKS = TILE_F / 4;   // 16-byte chunks per tile
    constexpr int LOADS = TILE_CHUNKS / 64;   // wave load instructions per tile
    constexpr int HC = CPR / 2;               // 16-byte chunks per half row
    constexpr int RP_INST = kBN * HC / 64;    // rotary: chunk-pair instructions per K tile
    constexpr int RMAX = rope_rmax<D>();
    // The two tile buffers ([key split][K tile | V tile] each) are separate
    // LDS objects, each named directly at every copy and read (the tile loop
    // is unrolled by two): the compiler then knows that the next tile's
    // copies do not write the buffer being read and does not make the reads
    // wait for them to land, which with offsets into one array it did.
    __shared__ __attribute__((aligned(16))) float lb0[KS * 2 * TILE_F];
    __shared__ __attribute__((aligned(16))) float lb1[KS * 2 * TILE_F];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31;
    const int hh = lane >> 5;

    const int bid = blockIdx.x;
    const int head_block = bid % a.n_head_blocks;
    const int seq = bid / a.n_head_blocks;
    const int rb = a.causal ? (a.n_row_blocks - 1 - seq) : seq;  // heaviest first

    // wave -> (key split, head, strip); waves sharing a key split share tiles
    const int kvs = wave % KS;
    const int rest = wave / KS;
    const int head = head_block * a.hg + rest % a.hg;
    const int strip = rest / a.hg;
    const int wg = wave / KS;              // index within its key split's group
    const int gw = kWaves / KS;            // waves per key split
    const int row0 = (rb * a.rs + strip) * kBM;
    const int kv_head = head / a.group;

    // Keys the block needs: up to the last row's window.
    const int blk_rows_hi = min((rb + 1) * a.rs * kBM, a.q_seq);
    const int w_block = a.causal ? min(a.start_pos + blk_rows_hi, a.kv_len) : a.kv_len;
    const bool wave_live = row0 < a.q_seq;
    const int w_wave_max = !wave_live ? 0
        : (a.causal ? min(a.start_pos + min(row0 + kBM, a.q_seq), a.kv_len) : a.kv_len);
    const int row = row0 + j;
    const int w_row = a.causal ? min(a.start_pos + row + 1, a.kv_len) : a.kv_len;
    // Smallest window of the wave's rows: tiles ending at or before it need no mask.
    const int w_wave_min = a.causal ? min(a.start_pos + row0 + 1, a.kv_len) : a.kv_len;

    // Tiles of this wave's key split.
    const int n_tiles_all = (w_block + kBN - 1) / kBN;
    const int nt = (n_tiles_all + KS - 1) / KS;
    const int t_begin = kvs * nt;
    const int t_end = min(t_begin + nt, n_tiles_all);

    // This key split's K | V tiles in the two buffers.
    float* my0 = lb0 + (size_t)kvs * 2 * TILE_F;
    float* my1 = lb1 + (size_t)kvs * 2 * TILE_F;

    // Q^T operand: lane (j, hh) holds q[row][8*g + 4*hh + c] for k-step 4*g+c.
    float qr[D / 2];
    {
        const bool ok = row < a.q_seq;
        const float* qp = q + (size_t)(ok ? row : 0) * a.q_stride + head * D + 4 * hh;
#pragma unroll
        for (int g = 0; g < D / 8; ++g) {
            float4 x = ok ? *reinterpret_cast<const float4*>(qp + 8 * g)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
            qr[4 * g + 0] = x.x * a.qscale;
            qr[4 * g + 1] = x.y * a.qscale;
            qr[4 * g + 2] = x.z * a.qscale;
            qr[4 * g + 3] = x.w * a.qscale;
        }
        if constexpr (ROPE != kRopeNone) {
            // Element e = 8g + 4hh + c (register 4g + c) pairs with e + D/2
            // (register 4(g + D/16) + c); the row sits at start_pos + row.
            if (ok) {
                const float* cs = a.rope_cs + (size_t)(a.start_pos + row) * D + 8 * hh;
#pragma unroll
                for (int g = 0; g < D / 16; ++g) {
                    const float4 c0 = *reinterpret_cast<const float4*>(cs + 16 * g);
                    const float4 c1 = *reinterpret_cast<const float4*>(cs + 16 * g + 4);
                    const float cw[4] = {c0.x, c0.z, c1.x, c1.z};
                    const float sw[4] = {c0.y, c0.w, c1.y, c1.w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const float x = qr[4 * g + c], y = qr[4 * (g + D / 16) + c];
                        qr[4 * g + c] = x * cw[c] - y * sw[c];
                        qr[4 * (g + D / 16) + c] = y * cw[c] + x * sw[c];
                    }
                }
            }
        }
    }

    f32x16 o[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[b][r] = 0.f;
    // Online softmax against a reference max (log2 units): the score
    // products start from -m_ref (the first product's accumulator input), so
    // they produce s - m_ref directly, and the reference moves only when a
    // row's max exceeds it by more than kRefSlack (p <= 2^kRefSlack in
    // between): most tiles then need neither a subtraction per score nor a
    // rescale of O. A query column's 32 keys of a tile sit in two lanes (one
    // per half-wave); each lane keeps its own running max above the reference
    // (rel) and its own partial sum, and the column's are formed across the
    // two lanes only when the reference moves and once at the end, where the
    // true (max, sum) pair is restored. Before a row has seen a key m_ref is
    // 0 and thr and rel are -inf. The instance that turns the keys,
    // whose registers are spoken for (with the reference's registers it
    // spilled 24 and took 17.5 instead of 16.2 ms on the 16K workload), keeps
    // the plain running max m_run and rescales whenever it moves.
    constexpr bool REF = !ROT_K;
    float m_run = kNegBig;
    float m_ref = 0.f;
    float rel = -INFINITY;
    float thr = -INFINITY;  // kRefSlack once the row has a reference
    float l_run = 0.f;      // this lane's partial sum until the end
    f32x16 negm;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[r] = 0.f;

    const float* kbase = k + kv_head * D;
    const float* vbase = v + kv_head * D;

    // Issue this wave's share of tile t's K and V into buffer buf. LDS slot s
    // (16 bytes) of a tile holds row s/CPR; for K its chunk position p holds
    // logical chunk p ^ (row % 16), for V the natural chunk.
    // Per-lane byte offsets inside a tile (row s / CPR, chunk s % CPR of the
    // wave's load slot s), the same for every tile. With 32-bit tile offsets
    // the copies go through buffer resources whose base is the tile's first
    // row and whose size ends at the block's window: a copy then costs no
    // vector instructions for its address, and rows past the window read as
    // zero (their scores are masked and their weight is 0). At most
    // LOADS / gw slots per wave: head_dim 128 runs at most 2 key splits
    // (gw >= 2), head_dim 64 at most 4 (gw >= 1). The instance that turns
    // the keys and larger strides take the general path below.
    constexpr int MAXI = D == 128 ? LOADS / 2 : LOADS;
    unsigned koff[MAXI], voff[MAXI];
#pragma unroll
    for (int u = 0; u < MAXI; ++u) {
        const unsigned s = (unsigned)((wg + u * gw) * 64 + lane);
        const unsigned r = s / CPR, c = s % CPR;
        koff[u] = (r * (unsigned)a.k_stride + 4u * (c ^ (r & 15u))) * 4u;
        voff[u] = (r * (unsigned)a.v_stride + 4u * c) * 4u;
    }
    // (Offsets reach the load builtins through named locals: an array
    // element written as a builtin argument made the host pass of the
    // compiler drop the kernel stubs without a diagnostic.)
    // Load u of this wave's share of tile t (buffer path), issued between the
    // score products of the current tile so the copies do not hold up the
    // wave's issue.
    auto issue_u = [&](int t, float* kd, int u) __attribute__((always_inline)) {
        const int inst = wg + u * gw;
        if (inst < LOADS) {
            const int kv0 = t * kBN;
            const int rows = min(kBN, w_block - kv0);
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(kbase + (size_t)kv0 * a.k_stride), 0, rows * (int)a.k_stride * 4,
                kBufferFlags);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(vbase + (size_t)kv0 * a.v_stride), 0, rows * (int)a.v_stride * 4,
                kBufferFlags);
            const unsigned ko = koff[u], vo = voff[u];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kd + inst * 256), 16, ko, 0, 0,
                                                     0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(kd + TILE_F + inst * 256), 16, vo,
                                                     0, 0, 0);
        }
    };
    auto issue_tile = [&](int t, float* kd) __attribute__((always_inline)) {
        float* vd = kd + TILE_F;
        const int kv0 = t * kBN;
        if (a.small_strides) {  // (turning the keys: V only, K goes through registers)
            const int rows = min(kBN, w_block - kv0);
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(kbase + (size_t)kv0 * a.k_stride), 0, rows * (int)a.k_stride * 4,
                kBufferFlags);
            const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(vbase + (size_t)kv0 * a.v_stride), 0, rows * (int)a.v_stride * 4,
                kBufferFlags);
#pragma unroll
            for (int u = 0; u < MAXI; ++u) {
                const int inst = wg + u * gw;
                if (inst < LOADS) {
                    const unsigned ko = koff[u], vo = voff[u];
                    if constexpr (!ROT_K) {
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(kd + inst * 256), 16,
                                                                 ko, 0, 0, 0);
                    }
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vd + inst * 256), 16, vo,
                                                             0, 0, 0);
                }
            }
            return;
        }
#pragma unroll 1
        for (int inst = wg; inst < LOADS; inst += gw) {
            const int s = inst * 64 + lane;
            const int r = s / CPR, p = s % CPR;
            const int key = min(kv0 + r, w_block - 1);
            if constexpr (!ROT_K) {
                const float* kg = kbase + (size_t)key * a.k_stride + 4 * (p ^ (r & 15));
                __builtin_amdgcn_global_load_lds(kg, (lds_void*)(kd + inst * 256), 16, 0, 0);
            }
            const float* vg = vbase + (size_t)key * a.v_stride + 4 * p;
            __builtin_amdgcn_global_load_lds(vg, (lds_void*)(vd + inst * 256), 16, 0, 0);
        }
    };

    // Rotary keys: lane work item s of a tile is (row s / HC, chunk pair
    // (c, c + HC), c = s % HC), i.e. elements 4c..4c+3 and their partners
    // D/2 further on, with the (cos, sin) of pairs 4c..4c+3 at the row's
    // position. With 32-bit tile offsets the rows come through buffer
    // resources as the copies above do (rows past the window read as zero:
    // their rotated keys are zero and masked); otherwise rows past the
    // block's window are read as its last row.
    float4 rk[ROT_K ? RMAX : 1][2], rc[ROT_K ? RMAX : 1][2];
    unsigned rko[ROT_K ? RMAX : 1], rco[ROT_K ? RMAX : 1];
    if constexpr (ROT_K) {
#pragma unroll
        for (int u = 0; u < RMAX; ++u) {
            const int s = (wg + u * gw) * 64 + lane;
            const int r = s / HC, c = s % HC;
            rko[u] = (unsigned)(r * (int)a.k_stride + 4 * c) * 4u;
            rco[u] = (unsigned)(r * D + 8 * c) * 4u;
        }
    }
    auto load_k_rot = [&](int t) {
        const int kv0 = t * kBN;
        if (a.small_strides) {
            const int rows = min(kBN, w_block - kv0);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(kbase + (size_t)kv0 * a.k_stride), 0, rows * (int)a.k_stride * 4,
                kBufferFlags);
            const __amdgpu_buffer_rsrc_t rt = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(a.rope_cs + (size_t)kv0 * D), 0, rows * D * 4, kBufferFlags);
#pragma unroll
            for (int u = 0; u < RMAX; ++u) {
                const int inst = wg + u * gw;
                if (inst < RP_INST) {
                    const unsigned ko = rko[u], co = rco[u];
                    const auto x0 = __builtin_amdgcn_raw_buffer_load_b128(rs, ko, 0, 0);
                    const auto x1 = __builtin_amdgcn_raw_buffer_load_b128(rs, ko + 2u * D, 0, 0);
                    const auto y0 = __builtin_amdgcn_raw_buffer_load_b128(rt, co, 0, 0);
                    const auto y1 = __builtin_amdgcn_raw_buffer_load_b128(rt, co + 16u, 0, 0);
                    rk[u][0] = make_float4(__int_as_float(x0[0]), __int_as_float(x0[1]),
                                           __int_as_float(x0[2]), __int_as_float(x0[3]));
                    rk[u][1] = make_float4(__int_as_float(x1[0]), __int_as_float(x1[1]),
                                           __int_as_float(x1[2]), __int_as_float(x1[3]));
                    rc[u][0] = make_float4(__int_as_float(y0[0]), __int_as_float(y0[1]),
                                           __int_as_float(y0[2]), __int_as_float(y0[3]));
                    rc[u][1] = make_float4(__int_as_float(y1[0]), __int_as_float(y1[1]),
                                           __int_as_float(y1[2]), __int_as_float(y1[3]));
                }
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < RMAX; ++u) {
            const int inst = wg + u * gw;
            if (inst < RP_INST) {
                const int s = inst * 64 + lane;
                const int r = s / HC, c = s % HC;
                const int key = min(kv0 + r, w_block - 1);
                const float* kg = kbase + (size_t)key * a.k_stride + 4 * c;
                rk[u][0] = *reinterpret_cast<const float4*>(kg);
                rk[u][1] = *reinterpret_cast<const float4*>(kg + D / 2);
                const float* cg = a.rope_cs + (size_t)key * D + 8 * c;
                rc[u][0] = *reinterpret_cast<const float4*>(cg);
                rc[u][1] = *reinterpret_cast<const float4*>(cg + 4);
            }
        }
    };
    auto store_k_rot = [&](float* kd) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < RMAX; ++u) {
            const int inst = wg + u * gw;
            if (inst < RP_INST) {
                const int s = inst * 64 + lane;
                const int r = s / HC, c = s % HC;
                const float4 lo = rk[u][0], hi = rk[u][1];
                const float4 c0 = rc[u][0], c1 = rc[u][1];
                float4 nlo, nhi;
                nlo.x = lo.x * c0.x - hi.x * c0.y;
                nhi.x = hi.x * c0.x + lo.x * c0.y;
                nlo.y = lo.y * c0.z - hi.y * c0.w;
                nhi.y = hi.y * c0.z + lo.y * c0.w;
                nlo.z = lo.z * c1.x - hi.z * c1.y;
                nhi.z = hi.z * c1.x + lo.z * c1.y;
                nlo.w = lo.w * c1.z - hi.w * c1.w;
                nhi.w = hi.w * c1.z + lo.w * c1.w;
                // Logical chunk c of row r lives at position c ^ (r % 16).
                *reinterpret_cast<float4*>(kd + r * D + 4 * (c ^ (r & 15))) = nlo;
                *reinterpret_cast<float4*>(kd + r * D + 4 * ((c + HC) ^ (r & 15))) = nhi;
            }
        }
    };

    if (t_begin < t_end) {
        issue_tile(t_begin, my0);
        if constexpr (ROT_K) {
            load_k_rot(t_begin);
            wait_vmem();
            store_k_rot(my0);
        }
    }

    // Byte offset in a K tile of the score operand's 16-byte read for
    // k-steps g and g + 8: row j, chunk (2g + hh) ^ (j % 16).
    unsigned kro[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) kro[g] = (unsigned)(j * D + 4 * ((2 * g + hh) ^ (j & 15))) * 4u;
    // One tile: Kb is the buffer holding tile it (this split's K | V tiles kvo
    // floats in), wb this split's part of the buffer tile it + 1 is copied into.
    auto step = [&](int it, const float* Kb, float* wb, auto masked_tag)
        __attribute__((always_inline)) {
        const int t = t_begin + it;
        const bool have = t < t_end;
        wait_vmem();
        // Tile t landed for every wave; buffer (it+1)&1 is free. A key split
        // served by one wave loads and reads only its own buffers, so its
        // wait suffices and the waves of the block run decoupled (full
        // 1024x1024, four splits: 30.5 -> 29.3 us).
        if (gw > 1) __syncthreads();
        const bool next = have && t + 1 < t_end;
        const int kv0 = t * kBN;
        const bool work = have && kv0 < w_wave_max;
        // the next tile's copies go between this tile's score products when
        // it lies inside the block's window (else, and without work, here)
        const bool spread = !ROT_K && next && work && a.small_strides;
        if (next && !spread) {
            issue_tile(t + 1, wb);
            if constexpr (ROT_K) load_k_rot(t + 1);
        }
        // Tiles inside every row's window (the leading ones, most of them)
        // run a version without mask code; the others apply the window as a
        // select (see the loops below).
        constexpr bool MASKED = decltype(masked_tag)::value;
        if (work) {  // wave-uniform
            // This split's K | V tiles start kvo floats into the buffer Kb;
            // the reads index Kb itself (through a split pointer the compiler
            // lost track of which buffer they read and waited for the next
            // tile's copies before them).
            const int kvo = kvs * 2 * TILE_F;

            // S^T - m_ref = K Q^T - m_ref for this tile (log2 units; the
            // instance that turns the keys: S^T).
            f32x16 s;
            if constexpr (REF) {
                s = negm;
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = 0.f;
            }
            const float4* kb4 = reinterpret_cast<const float4*>(Kb);
#pragma unroll
            for (int g = 0; g < D / 8; ++g) {
                // chunk (2g + hh) ^ (j % 16) of row j: k-steps 16 apart in g
                // are 256 bytes apart, an instruction offset
                const unsigned o = kro[g % 8];
                float4 kk;
                if constexpr (ROT_K) {  // (this instance's registers prefer the pointer form)
                    kk = *reinterpret_cast<const float4*>(
                        reinterpret_cast<const char*>(Kb + kvo) + o + 256 * (g / 8));
                } else {
                    kk = kb4[(unsigned)(4 * kvo + o + 256 * (g / 8)) / 16u];
                }
                s = mfma32(kk.x, qr[4 * g + 0], s);
                s = mfma32(kk.y, qr[4 * g + 1], s);
                if (g < MAXI && spread) issue_u(t + 1, wb, g);
                s = mfma32(kk.z, qr[4 * g + 2], s);
                s = mfma32(kk.w, qr[4 * g + 3], s);
            }

            // The window mask as a select (a branch here would put a block
            // edge between the last score product and the first vector read
            // of its result, where the wait the matrix unit's result needs was
            // once found missing in generated code).
            if constexpr (MASKED) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    s[r] = kv0 + acc_row(r, hh) < w_row ? s[r] : -INFINITY;
            }

            // Online softmax for query column j, against the reference.
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
          if constexpr (REF) {
            // This lane's tile max - m_ref (-inf: none of its keys in the window).
            rel = fmaxf(rel, mx);
            // Move the reference (one wave-wide vote) when a lane's max passed
            // its row's by more than the slack, or a row sees its first keys:
            // every row of the wave takes its true max as the new reference,
            // and O, the sum and this tile's scores follow. A row with a
            // reference had one lane at rel = 0 after its last move, so its
            // shift is >= 0; a row without one has O and the sum still 0.
            if (__builtin_amdgcn_ballot_w64(mx > thr) != 0ull) {
                const float rrow = pair_max32(rel);
                const bool seen = rrow > -INFINITY;
                const float shift = seen ? rrow : 0.f;
                const float corr = thr > -INFINITY ? __builtin_amdgcn_exp2f(-shift) : 0.f;
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[b][r] *= corr;
                l_run *= corr;
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] -= shift;
                m_ref += shift;
                rel -= shift;
                thr = thr > -INFINITY || seen ? kRefSlack : -INFINITY;
#pragma unroll
                for (int r = 0; r < 16; ++r) negm[r] = -m_ref;
            }
            // The tile's sum first, then one add to the lane's running sum
            // (thousands of single weights added to one running sum would
            // round more).
            float ls = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = __builtin_amdgcn_exp2f(s[r]);
                ls += s[r];
            }
            l_run += ls;
          } else {
            mx = pair_max32(mx);  // tile max (-inf: no key of the tile in the window)
            const float m_new = fmaxf(m_run, mx);
            const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
            float ls = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = __builtin_amdgcn_exp2f(s[r] - m_new);
                ls += s[r];
            }
            l_run = l_run * corr + ls;  // this lane's part; the pair's summed at the end
            m_run = m_new;
            // Rescale only if some row's max moved: one wave-wide vote
            // instead of 16*NB multiplies.
            if (__builtin_amdgcn_ballot_w64(corr != 1.0f) != 0ull) {
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[b][r] *= corr;
            }
          }

            // The P.V section runs at raised wave priority so the SIMD's other
            // wave fills its gaps with softmax work (raising it around the
            // score products as well measured slightly slower).
            __builtin_amdgcn_s_setprio(1);
            // O^T += V^T P^T: k-step t pairs keys acc_row(t, 0) and acc_row(t, 1).
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) {
                // (Indexed from the tile's base: with the address formed as
                // a float pointer plus offsets, the compiler lost track of which
                // LDS buffer these reads use and waited for the next tile's
                // copies before them.)
                const int vi = acc_row(tt, hh) * (D / NB) + j;  // in NB-float units
                if constexpr (NB == 4) {
                    const float4 vv = ROT_K
                        ? *reinterpret_cast<const float4*>(Kb + kvo + TILE_F + 4 * vi)
                        : reinterpret_cast<const float4*>(Kb)[(kvo + TILE_F) / 4 + vi];
                    o[0] = mfma32(vv.x, s[tt], o[0]);
                    o[1] = mfma32(vv.y, s[tt], o[1]);
                    o[2] = mfma32(vv.z, s[tt], o[2]);
                    o[3] = mfma32(vv.w, s[tt], o[3]);
                } else {
                    const float2 vv = ROT_K
                        ? *reinterpret_cast<const float2*>(Kb + kvo + TILE_F + 2 * vi)
                        : reinterpret_cast<const float2*>(Kb)[(kvo + TILE_F) / 2 + vi];
                    o[0] = mfma32(vv.x, s[tt], o[0]);
                    o[1] = mfma32(vv.y, s[tt], o[1]);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
        if constexpr (ROT_K) {
            if (next) {  // next tile's keys: turned and written after this tile's math
                wait_vmem();
                store_k_rot(wb);
            }
        }
    };
    // Two loops over the tiles (tile it in buffer it & 1): first the tiles
    // that lie inside every row's window, without mask code, then the rest
    // with the mask. Each loop body is straight-line from the score products
    // to the softmax (no block edge between a product and the vector reads
    // of its result), and the loops run one after the other, so the
    // unmasked version adds no registers to the masked one.
    const int n_int = max(0, min(nt, w_wave_min / kBN - t_begin));
    int it = 0;
    for (; it + 1 < n_int; it += 2) {
        step(it, lb0, my1, std::false_type{});
        step(it + 1, lb1, my0, std::false_type{});
    }
    for (; it < nt; it += 2) {
        step(it, lb0, my1, std::true_type{});
        if (it + 1 < nt) step(it + 1, lb1, my0, std::true_type{});
    }

    // The true (max, sum) pair from the two lanes' parts: max = m_ref + the
    // lanes' max above the reference, sum and O scaled to it (rows that saw
    // no key keep l = 0 and the sentinel max). Selects, no branch: O holds
    // matrix-core results.
    if constexpr (REF) {
        asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
        const float rrow = pair_max32(rel);
        const float lrow = pair_sum32(l_run);
        const bool seen = rrow > -INFINITY;
        const float f = seen ? __builtin_amdgcn_exp2f(-rrow) : 0.f;
        m_run = seen ? m_ref + rrow : kNegBig;
        l_run = lrow * f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[b][r] *= f;
    } else {
        l_run = pair_sum32(l_run);
    }

    if constexpr (KS > 1) {
        // Merge the key splits of the same (head, rows): splits 1.. publish
        // (m, l, O) through LDS in register order, split 0 rescales and adds.
        __syncthreads();  // every wave is done with the tile buffers
        // Per lane, contiguous: (m, l, -, -), then O block b registers 0..15
        // (4 + 16 NB floats: a lane stride of an odd number of 16-byte
        // chunks, so the 128-bit accesses are bank-conflict free).
        constexpr int PART = 4 + NB * 16;
        // Splits 1.. of each (head, strip) group take consecutive slots of
        // the first tile buffer: group rest, split kvs -> rest * (ks - 1) + kvs - 1.
        static_assert((kWaves / KS) * (KS - 1) * PART * 64 <= (KS > 1 ? KS * 2 * TILE_F : 1 << 30),
                      "merge slots fit the first tile buffer");
        float4* part = reinterpret_cast<float4*>(lb0) +
                       ((size_t)(rest * (KS - 1) + kvs - 1) * 64 + lane) * (PART / 4);
        if (kvs > 0) {
            part[0] = make_float4(m_run, l_run, 0.f, 0.f);
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    part[1 + 4 * b + r] = make_float4(o[b][4 * r], o[b][4 * r + 1], o[b][4 * r + 2],
                                                      o[b][4 * r + 3]);
        }
        __syncthreads();
        if (kvs > 0) return;
        for (int p = 1; p < KS; ++p) {
            const float4* pp = reinterpret_cast<const float4*>(lb0) +
                               ((size_t)(rest * (KS - 1) + p - 1) * 64 + lane) * (PART / 4);
            const float4 ml = pp[0];
            const float M = fmaxf(m_run, ml.x);
            const float f0 = __builtin_amdgcn_exp2f(m_run - M);
            const float f1 = __builtin_amdgcn_exp2f(ml.x - M);
            l_run = l_run * f0 + ml.y * f1;
            m_run = M;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float4 x = pp[1 + 4 * b + r];
                    o[b][4 * r + 0] = o[b][4 * r + 0] * f0 + x.x * f1;
                    o[b][4 * r + 1] = o[b][4 * r + 1] * f0 + x.y * f1;
                    o[b][4 * r + 2] = o[b][4 * r + 2] * f0 + x.z * f1;
                    o[b][4 * r + 3] = o[b][4 * r + 3] * f0 + x.w * f1;
                }
        }
    }

    if (!wave_live || row >= a.q_seq) return;

    // Epilogue: O^T block b, register r holds head-dim NB*acc_row(r, hh) + b.
    const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
    float* orow = out + (size_t)row * a.out_stride + head * D;
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

// One instance per key-split count (its LDS is static: KS x 2 buffers x
// (K, V) tiles).
template <int D, int ROPE, int KS>
hipError_t launch_ks(long long grid, hipStream_t stream, const float* q, const float* k,
                     const float* v, float* out, float* lse, const Args& a) {
    hipLaunchKernelGGL((prefill_kernel<D, ROPE, KS>), dim3((unsigned)grid), dim3(kBlock), 0,
                       stream, q, k, v, out, lse, a);
    return hipSuccess;
}

template <int D, int ROPE>
hipError_t launch_instance(long long grid, hipStream_t stream, const float* q, const float* k,
                           const float* v, float* out, float* lse, const Args& a) {
    if constexpr (D == 128 && ROPE == kRopeQK) {
        return launch_ks<D, ROPE, 1>(grid, stream, q, k, v, out, lse, a);
    } else if constexpr (D == 128) {
        return a.ks == 1 ? launch_ks<D, ROPE, 1>(grid, stream, q, k, v, out, lse, a)
                         : launch_ks<D, ROPE, 2>(grid, stream, q, k, v, out, lse, a);
    } else {
        return a.ks == 1   ? launch_ks<D, ROPE, 1>(grid, stream, q, k, v, out, lse, a)
               : a.ks == 2 ? launch_ks<D, ROPE, 2>(grid, stream, q, k, v, out, lse, a)
                           : launch_ks<D, ROPE, 4>(grid, stream, q, k, v, out, lse, a);
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
    a.rope_cs = s.rope_cs;
    a.q_seq = s.q_seq;
    a.kv_len = s.kv_len;
    a.num_heads = s.num_heads;
    a.num_kv_heads = s.num_kv_heads;
    a.group = s.num_heads / s.num_kv_heads;
    a.causal = s.causal;
    a.start_pos = s.start_pos;
    a.qscale = s.scale * kLog2e;
    a.q_stride = s.q_stride;
    a.k_stride = s.k_stride;
    a.v_stride = s.v_stride;
    a.out_stride = s.out_stride;
    {
        const long long big = s.k_stride > s.v_stride ? s.k_stride : s.v_stride;
        a.small_strides = 32 * 4 * big < (1ll << 31) ? 1 : 0;
    }

    // Block shape: heads of one GQA group x row strips x key splits = 4 waves.
    // Key splits only when one wave per (32 rows, head) leaves the chip short
    // of two waves per SIMD, and only over enough key tiles to share.
    const int strips = (s.q_seq + kBM - 1) / kBM;
    const long long base_waves = (long long)s.num_heads * strips;
    const int max_w = s.causal ? min(s.start_pos + s.q_seq, s.kv_len) : s.kv_len;
    const int key_tiles = (max_w + kBN - 1) / kBN;
    // 2 buffers x (K, V) per split in 160 KB; the instance that turns the
    // keys also holds the next key tile in registers, at most rope_rmax
    // instructions a wave.
    const bool rope = s.rope_cs != nullptr;
    const int rmode = !rope ? kRopeNone : s.rope_keys ? kRopeQK : kRopeQ;
    const int max_ks = s.head_dim == 128 ? (rmode == kRopeQK ? 1 : 2) : 4;
    int ks = 1;
    const int cus = device_cu_count();
    const long long target_waves = (long long)kWavesPerCU * cus;
    while (ks < max_ks && base_waves * ks < target_waves && key_tiles >= 4 * ks * 2) ks *= 2;
    a.ks = ks;
    a.hg = gcd_int(a.group, kWaves / ks);
    a.rs = kWaves / (ks * a.hg);
    a.n_head_blocks = s.num_heads / a.hg;
    a.n_row_blocks = (s.q_seq + a.rs * kBM - 1) / (a.rs * kBM);
    const long long grid = (long long)a.n_head_blocks * a.n_row_blocks;
    if (grid <= 0) return hipSuccess;
    if (!rope) {
        // Fewer blocks than compute units: the 16-row kernel, which needs no
        // shared tiles, spreads the work over more waves. At one block per
        // compute unit it still wins when the heads do not share K/V (group
        // 1: full 1024^2 22.9 vs 24.2 us), and loses when a GQA group would
        // share each tile through LDS (continuation 512 rows, group 4:
        // 149.5 vs 138.6 us). A testing override can force either kernel on
        // any shape the 16-row kernel takes.
        const int force = override_prefill_rows();
        const bool auto16 = grid < cus || (grid <= cus && a.group == 1);
        const bool use16 = (force != 0 ? force == 16 : auto16) && prefill16_fits(s);
        if (use16) return launch_prefill16(q, k, v, out, lse, s, stream);
    }
    hipError_t e;
    if (s.head_dim == 128) {
        e = rmode == kRopeQK ? launch_instance<128, kRopeQK>(grid, stream, q, k, v, out, lse, a)
            : rmode == kRopeQ ? launch_instance<128, kRopeQ>(grid, stream, q, k, v, out, lse, a)
                              : launch_instance<128, kRopeNone>(grid, stream, q, k, v, out, lse, a);
    } else {
        e = rmode == kRopeQK ? launch_instance<64, kRopeQK>(grid, stream, q, k, v, out, lse, a)
            : rmode == kRopeQ ? launch_instance<64, kRopeQ>(grid, stream, q, k, v, out, lse, a)
                              : launch_instance<64, kRopeNone>(grid, stream, q, k, v, out, lse, a);
    }
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace ta03
