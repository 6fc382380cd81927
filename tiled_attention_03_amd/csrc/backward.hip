// Attention backward on gfx950 f32 matrix cores.
//
// meganeura attention.wgsl writes, beside the output, the pair (row max m,
// log of the running sum l) "for backward"; the pages give no backward. This
// is the gradient of the forward's definition for a loss with dL/dout =
// dout, built on that pair: with s = scale <q_i, k_j> and the forward's
// (m_i, log l_i),
//   P_ij  = exp(s_ij - m_i - log l_i)      (the softmax, recomputed exactly)
//   dP_ij = <dout_i, v_j>,   D_i = <dout_i, out_i>
//   dS_ij = P_ij (dP_ij - D_i)
//   dq_i  = scale sum_j dS_ij k_j
//   dk_j  = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dout_i
// summed over the query heads of each KV head for dk, dv (GQA).
//
// No atomics anywhere (run-to-run bitwise deterministic). Two paths:
//   * stored path (workspace for every 16 x 16 dS tile): row-vector kernel
//     (D_i and the exponent offset of each row's pair); dk/dv
//     kernel that also writes the dS tiles it forms; dq = scale * dS K as one
//     product over the stored tiles. The matrix work is the algorithmic five
//     products (S, dP, dV, dK, dQ);
//   * recompute path (minimal workspace, or calls too short for the stored
//     path to pay): dq kernel (query-parallel, the forward's decomposition):
//     a wave owns 32 query rows of one head, holds Q^T (pre-scaled to log2
//     units) and dout^T as MFMA B operands in registers, and streams K/V
//     tiles of 32 keys through LDS (HBM -> LDS directly, double-buffered,
//     XOR-swizzled). Per tile: S^T = K Q^T and dP^T = V dout^T (keys x rows),
//     P^T and dS^T elementwise in the accumulator registers, dq^T += K^T dS^T
//     with dS^T reused in place as the B operand (the forward's P.V
//     pairing); it also writes the row vectors for the second kernel. Then the dk/dv
//     kernel. S and dP are formed in both kernels (seven products).
// The dk/dv kernel (key-parallel) in both paths: a wave owns 16 keys of one
// KV head, holds K and V as B operands, and walks the 16-row query tiles of
// every head of its group that can see its keys (causal: rows from
// key - start_pos on), Q and dout tiles streamed through LDS with their
// rows' exponent offsets and D. Per tile: S = Q K^T and dP = dout V^T (rows x keys), then
// dv^T += dout^T P and dk^T += Q^T dS with P and dS in place.

#include <hip/hip_runtime.h>

#include "ta03_internal.h"

namespace ta03 {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kBlock = 256;  // 4 waves
constexpr int kWaves = 4;
constexpr int kBM = 32;      // query rows per wave (dq) / per tile (dk, dv)
constexpr int kBN = 32;      // keys per tile (dq) / per wave (dk, dv)
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWavesPerCU = 8;  // two waves per SIMD

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row index held by accumulator register r in half-wave hh of a 32x32 MFMA
// result: 8*(r/4) + 4*hh + r%4.
__device__ __forceinline__ int acc_row(int r, int hh) {
    return 8 * (r >> 2) + 4 * hh + (r & 3);
}

__device__ __forceinline__ void wait_vmem() {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}

// Offset (floats) in a swizzled LDS row of the NB floats starting at logical
// column NB*j: 16-byte chunk c of row r is stored at position c ^ (r % 16).
template <int NB>
__device__ __forceinline__ int swz_cols(int j, int r) {
    if constexpr (NB == 4) {
        return 4 * (j ^ (r & 15));
    } else {
        return 4 * ((j >> 1) ^ (r & 15)) + 2 * (j & 1);
    }
}

struct BwdArgs {
    int q_seq, kv_len, num_heads, num_kv_heads, group;
    int causal, start_pos;
    float qscale;  // scale * log2(e)
    float scale;
    int hg, rs, ks, n_head_blocks, n_row_blocks;  // dq kernel block shape (ks: key splits)
    DsLayout ds;                              // stored dS tiles (when kept)
    // Window of the stored-dS launches (every query tile in one window when
    // every tile fits): query tiles win.off + j * win.stride, j < win.count.
    // Tile (h, local j, kt) sits at h * ds_tph + ds_win_tiles_before(j) + kt,
    // ds_tph being the window's tiles per head.
    DsWindow win;
    long long ds_tph;
    int accumulate;  // dk/dv kernel: add to dk, dv (windows after the first)
    int dq_hg, dq_rs, dq_rt, dq_n_head_blocks, dq_n_row_blocks;  // dq-from-dS block shape
    // dq from dS: 0, or the compute units of a grid that is resident all at
    // once, whose blocks are then dealt in rounds of that many, heaviest
    // first in even rounds and lightest first in odd ones.
    int dq_round;
};

// Issue this wave's share (inst = first, first + step, ...) of a 32-row, D-wide
// tile starting at row row0 of a matrix with row stride ld (ld * 128 < 2^31)
// into LDS, XOR-swizzled, through a buffer resource that ends at row row_hi:
// rows past it read as zero.
template <int D>
__device__ __forceinline__ void issue_rows(const float* base, long long ld, int row0, int row_hi,
                                           float* dst, int first, int step, int lane) {
    constexpr int CPR = D / 4;
    constexpr int LOADS = kBN * D / 4 / 64;
    const int rows = min(kBN, row_hi - row0);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(base + (size_t)row0 * ld), 0, rows * (int)ld * 4, kBufferFlags);
#pragma unroll 1
    for (int inst = first; inst < LOADS; inst += step) {
        const int s = inst * 64 + lane;
        const int r = s / CPR, p = s % CPR;
        const unsigned off = (unsigned)(r * (int)ld + 4 * (p ^ (r & 15))) * 4u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + inst * 256), 16, off, 0, 0,
                                                 0);
    }
}

template <int D>
__global__ void __launch_bounds__(kBlock, 2)
bwd_dq_kernel(const float* __restrict__ q, const float* __restrict__ k,
              const float* __restrict__ v, const float* __restrict__ o,
              const float* __restrict__ dout, const float* __restrict__ lse,
              float* __restrict__ dq, float* __restrict__ delta, BwdArgs a) {
    constexpr int NB = D / 32;
    constexpr int TILE_F = kBN * D;
    extern __shared__ __attribute__((aligned(16))) float smem[];  // [2][K tile | V tile]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 31;
    const int hh = lane >> 5;

    const int bid = blockIdx.x;
    const int head_block = bid % a.n_head_blocks;
    const int seq = bid / a.n_head_blocks;
    const int rb = a.causal ? (a.n_row_blocks - 1 - seq) : seq;  // heaviest first
    // wave -> (key split, head, strip); waves of one key split share its tiles
    const int kvs = wave % a.ks;
    const int rest = wave / a.ks;
    const int head = head_block * a.hg + rest % a.hg;
    const int strip = rest / a.hg;
    const int wg = wave / a.ks;       // index within its key split's group
    const int gw = kWaves / a.ks;     // waves per key split
    const int row0 = (rb * a.rs + strip) * kBM;
    const int kv_head = head / a.group;
    const int qd = a.num_heads * D;
    const int kvd = a.num_kv_heads * D;

    const int blk_rows_hi = min((rb + 1) * a.rs * kBM, a.q_seq);
    const int w_block = a.causal ? min(a.start_pos + blk_rows_hi, a.kv_len) : a.kv_len;
    const bool wave_live = row0 < a.q_seq;
    const int w_wave_max = !wave_live ? 0
        : (a.causal ? min(a.start_pos + min(row0 + kBM, a.q_seq), a.kv_len) : a.kv_len);
    const int w_wave_min = a.causal ? min(a.start_pos + row0 + 1, a.kv_len) : a.kv_len;
    const int row = row0 + j;
    const bool ok = row < a.q_seq;
    const int w_row = a.causal ? min(a.start_pos + row + 1, a.kv_len) : a.kv_len;
    const int n_tiles_all = (w_block + kBN - 1) / kBN;
    const int nt = (n_tiles_all + a.ks - 1) / a.ks;
    const int t_begin = kvs * nt;
    const int t_end = min(t_begin + nt, n_tiles_all);
    float* my_lds = smem + (size_t)kvs * 2 * 2 * TILE_F;  // this split's [2][K | V]

    // Q^T (log2 units) and dout^T operands: lane (j, hh) holds element
    // 8g + 4hh + c of row j in register 4g + c. D_j = <dout_j, out_j>.
    float qr[D / 2], gr[D / 2];
    float dlt, lse2;
    {
        const size_t off = (size_t)(ok ? row : 0) * qd + head * D + 4 * hh;
        float part = 0.f;
#pragma unroll
        for (int g = 0; g < D / 8; ++g) {
            const float4 x = ok ? *reinterpret_cast<const float4*>(q + off + 8 * g)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 y = ok ? *reinterpret_cast<const float4*>(dout + off + 8 * g)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            const float4 z = ok ? *reinterpret_cast<const float4*>(o + off + 8 * g)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
            qr[4 * g + 0] = x.x * a.qscale;
            qr[4 * g + 1] = x.y * a.qscale;
            qr[4 * g + 2] = x.z * a.qscale;
            qr[4 * g + 3] = x.w * a.qscale;
            gr[4 * g + 0] = y.x;
            gr[4 * g + 1] = y.y;
            gr[4 * g + 2] = y.z;
            gr[4 * g + 3] = y.w;
            part = fmaf(y.x, z.x, part);
            part = fmaf(y.y, z.y, part);
            part = fmaf(y.z, z.z, part);
            part = fmaf(y.w, z.w, part);
        }
        dlt = part + __shfl_xor(part, 32);
        lse2 = 0.f;
        if (ok) {
            const float2 ml = *reinterpret_cast<const float2*>(lse + ((size_t)row * a.num_heads + head) * 2);
            lse2 = (ml.x + ml.y) * kLog2e;
            if (hh == 0 && kvs == 0) {  // -D_i, then the exponent offset, for the dk/dv kernel
                const size_t pr = (size_t)row * a.num_heads + head;
                delta[pr] = -dlt;
                delta[(size_t)a.q_seq * a.num_heads + pr] = -lse2;
            }
        }
    }

    f32x16 acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;

    const float* kbase = k + kv_head * D;
    const float* vbase = v + kv_head * D;
    auto issue_tile = [&](int t, int buf) {
        float* kd = my_lds + (size_t)buf * 2 * TILE_F;
        issue_rows<D>(kbase, kvd, t * kBN, w_block, kd, wg, gw, lane);
        issue_rows<D>(vbase, kvd, t * kBN, w_block, kd + TILE_F, wg, gw, lane);
    };

    if (t_begin < t_end) issue_tile(t_begin, 0);
    for (int it = 0; it < nt; ++it) {
        const int t = t_begin + it;
        const bool have = t < t_end;
        wait_vmem();
        __syncthreads();  // tile t landed for every wave; buffer (it+1)&1 is free
        if (have && t + 1 < t_end) issue_tile(t + 1, (it + 1) & 1);
        const int kv0 = t * kBN;
        if (have && wave_live && kv0 < w_wave_max) {  // wave-uniform
            const float* Ks = my_lds + (size_t)(it & 1) * 2 * TILE_F;
            const float* Vs = Ks + TILE_F;
            // S^T = K Q^T and dP^T = V dout^T (row: key, column: query j).
            f32x16 s, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[r] = 0.f;
                dp[r] = 0.f;
            }
            const float* kr = Ks + j * D;
            const float* vr = Vs + j * D;
#pragma unroll
            for (int g = 0; g < D / 8; ++g) {
                const int c = (2 * g + hh) ^ (j & 15);
                const float4 kk = *reinterpret_cast<const float4*>(kr + 4 * c);
                const float4 vv = *reinterpret_cast<const float4*>(vr + 4 * c);
                s = mfma32(kk.x, qr[4 * g + 0], s);
                dp = mfma32(vv.x, gr[4 * g + 0], dp);
                s = mfma32(kk.y, qr[4 * g + 1], s);
                dp = mfma32(vv.y, gr[4 * g + 1], dp);
                s = mfma32(kk.z, qr[4 * g + 2], s);
                dp = mfma32(vv.z, gr[4 * g + 2], dp);
                s = mfma32(kk.w, qr[4 * g + 3], s);
                dp = mfma32(vv.w, gr[4 * g + 3], dp);
            }
            // dS^T in place of S^T; keys outside the row's window weigh 0.
            const bool need_mask = kv0 + kBN > w_wave_min;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const bool valid = !need_mask || kv0 + acc_row(r, hh) < w_row;
                const float p = valid ? __builtin_amdgcn_exp2f(s[r] - lse2) : 0.f;
                s[r] = p * (dp[r] - dlt);
            }
            // dq^T += K^T dS^T: k-step t pairs keys acc_row(t, 0) and
            // acc_row(t, 1); block b row m is head-dim NB*m + b.
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) {
                const int kr2 = acc_row(tt, hh);
                const float* kp = Ks + kr2 * D + swz_cols<NB>(j, kr2);
                if constexpr (NB == 4) {
                    const float4 kv = *reinterpret_cast<const float4*>(kp);
                    acc[0] = mfma32(kv.x, s[tt], acc[0]);
                    acc[1] = mfma32(kv.y, s[tt], acc[1]);
                    acc[2] = mfma32(kv.z, s[tt], acc[2]);
                    acc[3] = mfma32(kv.w, s[tt], acc[3]);
                } else {
                    const float2 kv = *reinterpret_cast<const float2*>(kp);
                    acc[0] = mfma32(kv.x, s[tt], acc[0]);
                    acc[1] = mfma32(kv.y, s[tt], acc[1]);
                }
            }
        }
    }

    if (a.ks > 1) {
        // Key splits 1.. publish their dq^T partial sums through LDS (the
        // tile buffers, free once every wave is past its last tile); split 0
        // adds them in split order.
        __syncthreads();
        constexpr int PART = NB * 16;  // floats per lane
        float* part = smem + (size_t)(wave * PART) * 64;
        if (kvs > 0) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) part[(b * 16 + r) * 64 + lane] = acc[b][r];
        }
        __syncthreads();
        if (kvs > 0) return;
        for (int p = 1; p < a.ks; ++p) {
            const float* pp = smem + (size_t)((wave + p) * PART) * 64;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][r] += pp[(b * 16 + r) * 64 + lane];
        }
    }

    if (!ok) return;
    float* drow = dq + (size_t)row * qd + head * D;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = acc_row(r, hh);
        if constexpr (NB == 4) {
            *reinterpret_cast<float4*>(drow + 4 * i) =
                make_float4(acc[0][r] * a.scale, acc[1][r] * a.scale, acc[2][r] * a.scale,
                            acc[3][r] * a.scale);
        } else {
            *reinterpret_cast<float2*>(drow + 2 * i) =
                make_float2(acc[0][r] * a.scale, acc[1][r] * a.scale);
        }
    }
}

// dk/dv with 16-key waves on v_mfma_f32_16x16x4_f32: per wave K, V (B
// operands) and the dk^T, dv^T accumulators take 32 registers each at
// head_dim 128 (half of the 32-key kernel), so two waves share a SIMD.
// Block: W = 4 waves x 16 keys of one KV head, two blocks per CU; query
// tiles of 16 rows (and their
// dout rows, (m, log l) and D) are staged in XOR-swizzled LDS, double-
// buffered. S = Q K^T: k-step s of lane group g carries head-dim g*D/4 + s
// (each lane reads d/4 contiguous floats of its query row); the result's
// register r of lane (j, g) is query 4g + r, key j, so in dv^T += dout^T P
// and dk^T += Q^T dS the k-step t of lane group g pairs query 4g + t with
// register t -- P and dS stay in registers. dk^T / dv^T block b row m is
// head-dim 64 (b / 4) + 4 m + b % 4, so the 16 lanes of a group read 256
// contiguous bytes of a Q / dout row (no bank conflicts).
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float comp4(const float4& x, int i) {
    return i == 0 ? x.x : (i == 1 ? x.y : (i == 2 ? x.z : x.w));
}

constexpr int k16Keys = 16;  // keys per wave
constexpr int k16Rows = 16;  // query rows per tile
// Query tiles per LDS stage of the dk/dv kernel: one block barrier per two
// tiles (46.5 -> 46.0 ms on the 16K causal backward; four per stage no longer
// fit two blocks per CU).
constexpr int kDkdvSub = 2;

template <int D, int W, bool STORE>
__global__ void __launch_bounds__(64 * W, 8 / W)  // 8 waves per CU: two per SIMD
bwd_dkdv16_kernel(const float* __restrict__ q, const float* __restrict__ k,
                  const float* __restrict__ v, const float* __restrict__ dout,
                  const float* __restrict__ rowv, float* __restrict__ dk,
                  float* __restrict__ dv, float* __restrict__ ds, BwdArgs a) {
    constexpr int KS = D / 4;   // k-steps of the score products
    constexpr int NB = D / 16;  // 16-row blocks of dk^T, dv^T
    constexpr int CPR = D / 4;  // 16-byte chunks per row
    constexpr int TILE_F = k16Rows * D;
    constexpr int LOADS = TILE_F / 4 / 64;  // wave instructions per tile (<= 8)
    // [2][SUB][Q tile | dout tile], then [2][SUB][128 floats: the rows' exponent
    // offsets -(m + log l) log2 e, then their -D_i, 16 rows four times each]
    constexpr int SUB = kDkdvSub;  // query tiles per stage (one barrier per stage)
    // Row r of a tile stores logical 16-byte chunk c at position c ^ swz(r).
    // A ds_read_b128 is served 16 lanes at a time over 64 four-byte banks (16
    // chunk positions per 256 bytes): in each half-wave the lane quads whose
    // index (lane >> 2) has even bit parity form one pass, the odd ones the
    // other. The score read (lane (j, g): row j, chunk g * KS / 4 + c) and the
    // dv / dk read (row 4g + t, chunk j + 16c) both hit 16 distinct positions
    // per pass with the masks below; r & 15 left both 2-way.
    auto swz = [](int r) { return D == 128 ? (r & 3) | ((r >> 1) & 4) : r & 11; };
    // The two stage buffers are separate LDS objects, each named directly at
    // every copy and read (the stage loop is unrolled by two): the compiler
    // then knows that the copies into one buffer do not touch the other, and
    // does not make the reads of the current stage wait for the next stage's
    // copies to land (with offsets into one array it did).
    __shared__ __attribute__((aligned(16))) float tl0[SUB * 2 * TILE_F];
    __shared__ __attribute__((aligned(16))) float tl1[SUB * 2 * TILE_F];
    __shared__ __attribute__((aligned(16))) float vc0[SUB * 128];
    __shared__ __attribute__((aligned(16))) float vc1[SUB * 128];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15;
    const int g = lane >> 4;

    const int bid = blockIdx.x;
    const int kv_head = bid % a.num_kv_heads;
    const int kb = bid / a.num_kv_heads;  // low keys first: the most rows see them
    const int blk_key0 = kb * W * k16Keys;
    const int key0 = blk_key0 + wave * k16Keys;
    const bool strip_live = key0 < a.kv_len;
    const int key = key0 + j;
    const int qd = a.num_heads * D;
    const int kvd = a.num_kv_heads * D;
    // Query row i weighs this lane's key iff i >= key - start_pos (causal),
    // i < q_seq and key < kv_len. With i = row0 + 4g + r of a tile that is
    // row0 + r + vbase in [0, vspan): one unsigned compare per score.
    const int ilo = a.causal ? max(0, key - a.start_pos) : 0;
    const unsigned vspan = (unsigned)max(0, (key < a.kv_len ? a.q_seq : 0) - ilo);
    const int vbase = 4 * g - ilo;

    // K (log2 units) and V of key j: element g*KS + s in register s.
    float kr[KS], vr[KS];
    {
        const size_t off = (size_t)min(key, a.kv_len - 1) * kvd + kv_head * D + g * KS;
#pragma unroll
        for (int c = 0; c < KS / 4; ++c) {
            const float4 x = *reinterpret_cast<const float4*>(k + off + 4 * c);
            const float4 y = *reinterpret_cast<const float4*>(v + off + 4 * c);
            kr[4 * c + 0] = x.x * a.qscale;
            kr[4 * c + 1] = x.y * a.qscale;
            kr[4 * c + 2] = x.z * a.qscale;
            kr[4 * c + 3] = x.w * a.qscale;
            vr[4 * c + 0] = y.x;
            vr[4 * c + 1] = y.y;
            vr[4 * c + 2] = y.z;
            vr[4 * c + 3] = y.w;
        }
        // Let K and V land here: a V register still in flight at the loop
        // made the compiler wait for every load (the stage copies too) at its
        // first use inside every stage.
        wait_vmem();
    }

    f32x4 dka[NB], dva[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        dka[b] = f32x4{0.f, 0.f, 0.f, 0.f};
        dva[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Query tiles of the window whose rows see some key of the block (causal:
    // rows from blk_key0 - start_pos on): local tiles j0 .. win.count - 1, query
    // tile win.off + j * win.stride.
    const int i_lo = a.causal ? max(0, blk_key0 - a.start_pos) : 0;
    const int qmin = i_lo / k16Rows;
    const int j0 = qmin <= a.win.off ? 0 : (qmin - a.win.off + a.win.stride - 1) / a.win.stride;
    const int n_qt = i_lo < a.q_seq && j0 < a.win.count ? a.win.count - j0 : 0;
    const int total = a.group * n_qt;
    // query tile of the block's tile step it (head it / n_qt)
    auto qt_of = [&](int it) { return a.win.off + (j0 + it % n_qt) * a.win.stride; };

    // Copies go through buffer resources whose base is the tile's first row
    // (of Q / dout at head h, of the row vectors) and whose size
    // ends at q_seq: every lane's byte offsets are the same for every tile
    // (computed once below), so a copy costs no vector instructions for its
    // address, and rows past q_seq read as zero (those rows are masked).
    // Tile load instruction inst = wave + W u: slot s = 64 inst + lane holds
    // row s / CPR, position s % CPR = logical chunk ^ swz(row).
    unsigned qoff[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int s_ = (wave + W * u) * 64 + lane;
        const int r = s_ / CPR, p = s_ % CPR;
        qoff[u] = (unsigned)(r * qd + 4 * (p ^ swz(r))) * 4u;
    }
    // Row vectors (rowv: -D_i per (row, head), then the exponent offsets):
    // lane l holds row l % 16.
    const unsigned doff = (unsigned)((lane & 15) * a.num_heads) * 4u;
    const size_t n_pairs = (size_t)a.q_seq * a.num_heads;
    auto issue_rows = [&](int it, int sub, float* tb, int u) __attribute__((always_inline)) {
        const int inst = wave + W * u;
        if (inst < LOADS) {
            const int h = kv_head * a.group + it / n_qt;
            const int row0 = qt_of(it) * k16Rows;
            const int rows = min(k16Rows, a.q_seq - row0);
            const size_t base = (size_t)row0 * qd + h * D;
            const auto rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(q + base), 0,
                                                              rows * qd * 4, kBufferFlags);
            const auto rg = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(dout + base), 0,
                                                              rows * qd * 4, kBufferFlags);
            float* qdst = tb + (size_t)sub * 2 * TILE_F;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (lds_void*)(qdst + inst * 256), 16,
                                                     qoff[u], 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rg, (lds_void*)(qdst + TILE_F + inst * 256),
                                                     16, qoff[u], 0, 0, 0);
        }
    };
    auto issue_vec = [&](int it, int sub, float* vb) __attribute__((always_inline)) {
        const int h = kv_head * a.group + it / n_qt;
        const int row0 = qt_of(it) * k16Rows;
        const int rows = min(k16Rows, a.q_seq - row0);
        const auto rl = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(rowv + n_pairs + (size_t)row0 * a.num_heads + h), 0,
            rows * a.num_heads * 4, kBufferFlags);
        const auto rd = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(rowv + (size_t)row0 * a.num_heads + h), 0, rows * a.num_heads * 4,
            kBufferFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (lds_void*)(vb + sub * 128), 4, doff, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_void*)(vb + sub * 128 + 64), 4, doff, 0, 0,
                                                 0);
    };
    auto issue1 = [&](int it, int sub, float* tb, float* vb) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 2; ++u) issue_rows(it, sub, tb, u);
        if (wave == W - 1) issue_vec(it, sub, vb);
    };
    // One piece of stage st's copies (for spreading them between products):
    // pieces 0..3 = Q / dout rows of sub-tile p >> 1, instruction p & 1;
    // pieces 4, 5 = the (m, log l) / D vectors of sub-tile p - 4.
    // The six pieces cover a stage only for two sub-tiles of at most two
    // load instructions per wave each; a change to either must change them.
    static_assert(SUB == 2 && LOADS <= 2 * W, "issue_piece covers every copy of a stage");
    auto issue_piece = [&](int st, float* tb, float* vb, int pc) __attribute__((always_inline)) {
        const int sub = pc < 4 ? pc >> 1 : pc - 4;
        const int it = st * SUB + sub;
        if (it >= total) return;
        if (pc < 4) {
            issue_rows(it, sub, tb, pc & 1);
        } else if (wave == W - 1) {
            issue_vec(it, sub, vb);
        }
    };
    auto issue = [&](int st, float* tb, float* vb) __attribute__((always_inline)) {
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub)
            if (st * SUB + sub < total) issue1(st * SUB + sub, sub, tb, vb);
    };

    const int n_st = (total + SUB - 1) / SUB;
    // dS tiles this wave stored in the previous stage, after that stage's
    // copies (four store instructions each).
    int stored_prev = 0;
    auto stage = [&](int st, const float* rt, const float* rv, float* wt, float* wv)
        __attribute__((always_inline)) {
        if constexpr (STORE) {
            // Vector-memory counts complete in issue order: this stage's
            // copies are done once at most the previous stage's dS stores
            // are in flight, which need not be complete here (nothing in this
            // kernel reads them). A bare barrier: __syncthreads' fences would
            // wait for every store too.
            if (stored_prev == 0)
                __builtin_amdgcn_s_waitcnt(0x0F70);
            else if (stored_prev == 1)
                __builtin_amdgcn_s_waitcnt(0x0F74);
            else
                __builtin_amdgcn_s_waitcnt(0x0F78);
            asm volatile("s_barrier" ::: "memory");
            stored_prev = 0;
        } else {
            wait_vmem();
            __syncthreads();  // stage st landed for every wave; the other buffer is free
        }
        // The next stage's copies go between the first sub-tile's score
        // products when this wave computes it, else here.
        const int rows_hi0 = min(qt_of(st * SUB) * k16Rows + k16Rows, a.q_seq);
        const int w_max0 = a.causal ? min(a.start_pos + rows_hi0, a.kv_len) : a.kv_len;
        const bool spread = st + 1 < n_st && strip_live && key0 < w_max0;
        if (st + 1 < n_st && !spread) issue(st + 1, wt, wv);
#pragma unroll
        for (int sub = 0; sub < SUB; ++sub) {
            const int it = st * SUB + sub;
            if (it >= total) break;
            const int row0 = qt_of(it) * k16Rows;
            const int rows_hi = min(row0 + k16Rows, a.q_seq);
            const int w_max = a.causal ? min(a.start_pos + rows_hi, a.kv_len) : a.kv_len;
            if (strip_live && key0 < w_max) {  // wave-uniform
                const float* Qs = rt + (size_t)sub * 2 * TILE_F;
                const float* Gs = Qs + TILE_F;
                const float* vd = rv + sub * 128;
                // S = Q K^T - (m + log l) (log2 units), dP - D = dout V^T - D:
                // register r of lane (j, g) is query row0 + 4g + r, key
                // key0 + j. The products start from the rows' -(m + log l) and
                // -D_i, so neither the exponent nor dS needs a subtraction.
                f32x4 s = *reinterpret_cast<const f32x4*>(vd + 4 * g);
                f32x4 dp = *reinterpret_cast<const f32x4*>(vd + 64 + 4 * g);
#pragma unroll
                for (int c = 0; c < KS / 4; ++c) {
                    const int pos = ((g * KS / 4 + c) ^ swz(j)) * 4;
                    const float4 qq = *reinterpret_cast<const float4*>(Qs + j * D + pos);
                    const float4 gg = *reinterpret_cast<const float4*>(Gs + j * D + pos);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s = mfma16(comp4(qq, e), kr[4 * c + e], s);
                        dp = mfma16(comp4(gg, e), vr[4 * c + e], dp);
                        // six pieces over the k-step groups (two per group at head_dim 64)
                        constexpr int PPG = KS / 4 >= 6 ? 1 : 2;
                        if (sub == 0 && spread && (e == 1 || (PPG == 2 && e == 3))) {
                            const int pc = c * PPG + (e == 3 ? 1 : 0);
                            if (pc < 6) issue_piece(st + 1, wt, wv, pc);
                        }
                    }
                }
                // P in s, dS in dp. The window test is a select (no branch between
                // the products and the first vector reads of their results).
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool valid = (unsigned)(row0 + r + vbase) < vspan;
                    const float p = valid ? __builtin_amdgcn_exp2f(s[r]) : 0.f;
                    s[r] = p;
                    dp[r] = p * dp[r];
                }
                if constexpr (STORE) {
                    // The 16 x 16 dS tile (query rows x keys, row-major) of this
                    // head, query tile and key tile; masked entries are 0. Four
                    // stores of 4 x 64 contiguous bytes, issued before the dv / dk
                    // products so they complete under them.
                    const int h = kv_head * a.group + it / n_qt;
                    const int jl = j0 + it % n_qt;
                    float* tile = ds + ((size_t)h * a.ds_tph + ds_win_tiles_before(a.ds, a.win, jl) +
                                        key0 / k16Keys) * (k16Rows * k16Keys);
#pragma unroll
                    for (int r = 0; r < 4; ++r) tile[(4 * g + r) * k16Keys + j] = dp[r];
                    ++stored_prev;
                }
                // dv^T += dout^T P, dk^T += Q^T dS: k-step t of lane group g is
                // query row 4g + t; lane (m, g) reads head-dims 4m .. 4m + 3 (and
                // 64 + 4m .. 64 + 4m + 3 at head_dim 128).
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int ir = 4 * g + t;
#pragma unroll
                    for (int c = 0; c < NB / 4; ++c) {
                        const int pos = ((j + 16 * c) ^ swz(ir)) * 4;
                        const float4 gg = *reinterpret_cast<const float4*>(Gs + ir * D + pos);
                        const float4 qq = *reinterpret_cast<const float4*>(Qs + ir * D + pos);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            dva[4 * c + e] = mfma16(comp4(gg, e), s[t], dva[4 * c + e]);
                            dka[4 * c + e] = mfma16(comp4(qq, e), dp[t], dka[4 * c + e]);
                        }
                    }
                }
            }
        }
    };
    if (total > 0) issue(0, tl0, vc0);
    for (int st = 0; st < n_st; st += 2) {
        stage(st, tl0, vc0, tl1, vc1);
        if (st + 1 < n_st) stage(st + 1, tl1, vc1, tl0, vc0);
    }

    if (!strip_live || key >= a.kv_len) return;
    // dk^T / dv^T block b, register r of lane (j, g): head-dim
    // 64 (b / 4) + 4 (4g + r) + b % 4.
    float* krow = dk + (size_t)key * kvd + kv_head * D;
    float* vrow = dv + (size_t)key * kvd + kv_head * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int c = 0; c < NB / 4; ++c) {
            const int d0 = 64 * c + 4 * (4 * g + r);
            float4 kx = make_float4(dka[4 * c + 0][r] * a.scale, dka[4 * c + 1][r] * a.scale,
                                    dka[4 * c + 2][r] * a.scale, dka[4 * c + 3][r] * a.scale);
            float4 vx = make_float4(dva[4 * c + 0][r], dva[4 * c + 1][r], dva[4 * c + 2][r],
                                    dva[4 * c + 3][r]);
            if (a.accumulate) {  // block-uniform: a later window adds to the earlier ones
                const float4 k0 = *reinterpret_cast<const float4*>(krow + d0);
                const float4 v0 = *reinterpret_cast<const float4*>(vrow + d0);
                kx = make_float4(k0.x + kx.x, k0.y + kx.y, k0.z + kx.z, k0.w + kx.w);
                vx = make_float4(v0.x + vx.x, v0.y + vx.y, v0.z + vx.z, v0.w + vx.w);
            }
            *reinterpret_cast<float4*>(krow + d0) = kx;
            *reinterpret_cast<float4*>(vrow + d0) = vx;
        }
    }
}

// ---------------------------------------------------------------------------
// Backward from stored dS (three launches): D_i first, then the 16-key dk/dv
// kernel, which also writes every 16 x 16 dS tile it forms, then dq as one
// product over the stored tiles, dq = scale * dS K, so no score or dP is
// formed twice. The tiles cost 1 KiB per 256 (row, key) pairs per head of
// workspace.

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL,
                                                      0xF, 0xF, false));
}

// The dk/dv kernel's row vectors per (row, head): -D_i with D_i =
// <dout_i, out_i> (16 lanes per pair, D/16 contiguous floats each, summed over
// the 16 lanes with DPP: quad xor 1, quad xor 2, half-row mirror, row mirror),
// and the exponent offset -(m + log l) log2 e of the row's stored pair. The
// dk/dv kernel starts its products from them.
template <int D>
__global__ void __launch_bounds__(256)
bwd_delta_kernel(const float* __restrict__ o, const float* __restrict__ dout,
                 const float* __restrict__ lse, float* __restrict__ rowv, long long n_pairs) {
    constexpr int PER = D / 16;
    const int tid = threadIdx.x;
    const long long pair = (long long)blockIdx.x * 16 + (tid >> 4);
    const int l16 = tid & 15;
    // q, out and dout rows are num_heads * D wide: pair (row, head) starts at pair * D.
    const long long pc = pair < n_pairs ? pair : n_pairs - 1;
    const float* op = o + pc * D + l16 * PER;
    const float* gp = dout + pc * D + l16 * PER;
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < PER / 4; ++c) {
        const float4 x = *reinterpret_cast<const float4*>(op + 4 * c);
        const float4 y = *reinterpret_cast<const float4*>(gp + 4 * c);
        acc = fmaf(x.x, y.x, acc);
        acc = fmaf(x.y, y.y, acc);
        acc = fmaf(x.z, y.z, acc);
        acc = fmaf(x.w, y.w, acc);
    }
    acc += dpp_f<0xB1>(acc);
    acc += dpp_f<0x4E>(acc);
    acc += dpp_f<0x141>(acc);
    acc += dpp_f<0x140>(acc);
    const float2 ml = *reinterpret_cast<const float2*>(lse + 2 * pc);
    if (l16 == 0 && pair < n_pairs) {
        rowv[pair] = -acc;
        rowv[n_pairs + pair] = (ml.x + ml.y) * -kLog2e;
    }
}

// dq from stored dS. A block is 4 KS waves: KS key splits of 4 waves, the 4
// waves being dq_hg query heads of one GQA group x dq_rs strips; a wave owns
// RT query tiles of 16 rows of one head, and each split streams its share of
// the 16-key K tiles of the block's KV head (up to the window of its last
// query tile) through LDS (HBM -> LDS directly). Per key tile and k-step t
// (keys 4g + t for lane group g), with v_mfma_f32_16x16x4_f32:
//   A: lane (j, g) gives dS[row j][key 4g + t] -- one 16-byte load of the
//      row-major tile per query tile covers all four k-steps;
//   B: lane (j, g) gives K[key 4g + t][d] for d = 64 (b / 4) + 4 j + b % 4 in
//      column block b (4 j + b at head_dim 64), so each lane reads one or two
//      16-byte runs of a K row and the 16 lanes of a group read 256
//      contiguous bytes (no bank conflicts);
//   result block b: register r of lane (j, g) is row 4g + r, column d, so a
//      row's four column blocks store as one float4 per lane.
// Key tiles past a query tile's window (and query tiles past the window's
// count) read as zero through the dS tiles' buffer resources. RT = 4 query tiles per wave
// (each K operand read serves 4 products), 1 where that would leave the grid
// short of blocks; then KS = 2 or 4 key splits where the grid is short even
// so: a window's dq launch otherwise lasts as long as one wave's walk over
// the keys of its last query tile, whatever the window's size. The splits'
// partial dq meet in LDS and are added in split order (deterministic).
// K tiles stream through a ring of four LDS buffers and each wave's dS tiles
// through a ring of four register sets, both issued three steps ahead: with
// one query tile per wave a step is only 32 products per wave, too short to
// cover a dS read from HBM issued one step ahead (with four, one step ahead
// measured the same). Vector-memory counts complete in issue order, so one
// wait for the current step's loads, with those of the next two steps left
// in flight, covers K and dS.
__host__ __device__ constexpr int waitcnt_vm(int n) {  // s_waitcnt vmcnt(n), other counters free
    return 0x0F70 | (n & 15) | ((n >> 4) << 14);
}

template <int D, int RT, int KS>
__global__ void __launch_bounds__(256 * KS, KS == 1 ? 2 : 1)
bwd_dq_ds_kernel(const float* __restrict__ k, const float* __restrict__ ds,
                 float* __restrict__ dq, BwdArgs a) {
    static_assert(KS == 1 || KS == 2 || KS == 4, "one, two or four key splits");
    static_assert(KS == 1 || RT == 1, "key splits with one query tile per wave");
    constexpr int NS = 4;  // ring slots: tiles issued NS - 1 steps ahead
    constexpr int NB = D / 16;
    constexpr int CPR = D / 4;
    constexpr int TILE_F = k16Keys * D;
    constexpr int LOADS = TILE_F / 4 / 64;  // wave instructions per K tile (8 or 4)
    constexpr int TF = k16Rows * k16Keys;   // floats per dS tile
    // Vector memory instructions a wave issues per step: its share of the K
    // tile copy and one dS load per query tile.
    constexpr int PER_STEP = LOADS / 4 + RT;
    static_assert((NS - 2) * PER_STEP < 64, "vmcnt range");
    // One LDS object per slot (each holding the slot of every split), named
    // directly at every copy and read, so the reads of one tile do not wait
    // for the copies of the others.
    __shared__ __attribute__((aligned(16))) float kb0[KS * TILE_F];
    __shared__ __attribute__((aligned(16))) float kb1[KS * TILE_F];
    __shared__ __attribute__((aligned(16))) float kb2[KS * TILE_F];
    __shared__ __attribute__((aligned(16))) float kb3[KS * TILE_F];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int split = KS == 1 ? 0 : wave >> 2;  // key split
    const int wq = KS == 1 ? wave : wave & 3;     // wave of the split: (head, strip)
    const int j = lane & 15;
    const int g = lane >> 4;

    int bid = blockIdx.x;
    if (a.dq_round > 0) {
        const int r = bid / a.dq_round, p = bid % a.dq_round;
        const int cnt = min(a.dq_round, (int)gridDim.x - r * a.dq_round);
        bid = r * a.dq_round + ((r & 1) ? cnt - 1 - p : p);
    }
    const int head_block = bid % a.dq_n_head_blocks;
    const int seq = bid / a.dq_n_head_blocks;
    const int rb = a.causal ? (a.dq_n_row_blocks - 1 - seq) : seq;  // heaviest first
    const int head = head_block * a.dq_hg + wq % a.dq_hg;
    const int strip = wq / a.dq_hg;
    const int kv_head = head / a.group;
    const int kvd = a.num_kv_heads * D;
    const int j_first = (rb * a.dq_rs + strip) * RT;  // this wave's first local query tile
    const int blk_j_last = min((rb + 1) * a.dq_rs * RT, a.win.count) - 1;
    const int n_blk = blk_j_last >= 0 ? ds_tiles_in(a.ds, a.win.off + blk_j_last * a.win.stride) : 0;
    // Split s walks key tiles s n_kt .. s n_kt + n_kt - 1 (every split the
    // same step count: the barriers are block-wide).
    const int n_kt = (n_blk + KS - 1) / KS;
    const int kt0 = split * n_kt;
    const int so = split * TILE_F;  // this split's slot in each buffer (floats)

    // The dS tiles of query tile rt go through a buffer resource whose base
    // is its first tile and whose size is its tile count (0 for a tile past
    // the window's count): key tiles past its window read as zero, so the
    // products need no select and the loads no clamp.
    __amdgpu_buffer_rsrc_t rds[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int jl = j_first + rt;
        const int jc = min(jl, a.win.count - 1);
        const int tcount = jl < a.win.count ? ds_tiles_in(a.ds, a.win.off + jc * a.win.stride) : 0;
        const long long tbase = (long long)head * a.ds_tph + ds_win_tiles_before(a.ds, a.win, jc);
        rds[rt] = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ds + (size_t)tbase * TF), 0,
                                                    tcount * TF * 4, kBufferFlags);
    }
    const unsigned dso = (unsigned)(16 * j + 4 * g) * 4u;  // the lane's float4 of a dS tile
    // K copies through a buffer resource whose base is the key tile's first
    // row of this KV head and whose size ends at kv_len (rows past it, and
    // the repeats past the last tile, read as zero): each lane's byte offsets
    // are fixed for the whole kernel. LOADS / 4 copies per wave (4 waves per
    // split), a count the compiler sees, so that it can count this wave's
    // loads in flight at every wait.
    unsigned koff[LOADS / 4];
#pragma unroll
    for (int i = 0; i < LOADS / 4; ++i) {
        const int s_ = (wq + 4 * i) * 64 + lane;
        koff[i] = (unsigned)((s_ / CPR) * kvd + 4 * (s_ % CPR)) * 4u;
    }

    // Step kt of this split: key tile kt0 + kt.
    auto issue = [&](int kt, float* dst, float4 (&x)[RT]) __attribute__((always_inline)) {
        const int t = kt0 + kt;
        // (Moved to a scalar register explicitly: the clamp otherwise became
        // a vector min-max, and the resource a loop over its lanes.)
        const int rows = __builtin_amdgcn_readfirstlane(min(k16Keys, max(a.kv_len - t * k16Keys, 0)));
        const auto rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(k + (size_t)t * k16Keys * kvd + kv_head * D), 0, rows * kvd * 4,
            kBufferFlags);
#pragma unroll
        for (int i = 0; i < LOADS / 4; ++i) {
            const unsigned ko = koff[i];
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (lds_void*)(dst + (so + (wq + 4 * i) * 256)), 16, ko, 0, 0, 0);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rds[rt], dso + (unsigned)t * (TF * 4),
                                                                 0, 0);
            x[rt] = make_float4(__int_as_float(v[0]), __int_as_float(v[1]), __int_as_float(v[2]),
                                __int_as_float(v[3]));
        }
    };

    f32x4 acc[RT][NB];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[rt][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Step kt reads K tile kt0 + kt from the split's slot of buffer Ks and its
    // dS tiles from cur, and first issues tile kt + NS - 1 into the buffers
    // tile kt - 1 used.
    auto step = [&](int kt, const float* Ks, float* kissue, const float4 (&cur)[RT],
                    float4 (&nxt)[RT]) __attribute__((always_inline)) {
        // Tile kt's loads complete while those of the next NS - 2 tiles stay
        // in flight (every step issues, past the last tile a clamped repeat,
        // so the count is fixed).
        __builtin_amdgcn_s_waitcnt(waitcnt_vm((NS - 2) * PER_STEP));
        // K tile kt landed for every wave; tile kt - 1's buffer is free. A
        // bare barrier: __syncthreads' fences would also wait for the copies
        // of the tiles ahead, which write LDS. The wait above covers this
        // wave's copies of tile kt, and every wave's reads of tile kt - 1
        // were consumed by its products before it arrived here; the clobber
        // keeps the compiler from moving memory accesses across.
        asm volatile("s_barrier" ::: "memory");
        issue(kt + NS - 1, kissue, nxt);
        float av[RT][4];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            av[rt][0] = cur[rt].x;
            av[rt][1] = cur[rt].y;
            av[rt][2] = cur[rt].z;
            av[rt][3] = cur[rt].w;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            // (Indexed from the buffer object itself: with the split's slot
            // as a separate pointer the compiler lost track of which buffer
            // these reads use and waited for every copy in flight.)
            const int kr = (so + (4 * g + t) * D + 4 * j) / 4;  // in float4 units
            float kb[NB];
#pragma unroll
            for (int h2 = 0; h2 < NB / 4; ++h2) {
                const float4 x = reinterpret_cast<const float4*>(Ks)[kr + 16 * h2];
                kb[4 * h2 + 0] = x.x;
                kb[4 * h2 + 1] = x.y;
                kb[4 * h2 + 2] = x.z;
                kb[4 * h2 + 3] = x.w;
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[rt][b] = mfma16(av[rt][t], kb[b], acc[rt][b]);
        }
    };

    float4 d0[RT], d1[RT], d2[RT], d3[RT];
    int kt = 0;
    if (n_kt > 0) {  // block-uniform
        // Issued in tile order, as the steps do (the waits count on it).
        issue(0, kb0, d0);
        asm volatile("" ::: "memory");
        issue(1, kb1, d1);
        asm volatile("" ::: "memory");
        issue(2, kb2, d2);
    }
    for (; kt + 4 <= n_kt; kt += 4) {
        step(kt, kb0, kb3, d0, d3);
        step(kt + 1, kb1, kb0, d1, d0);
        step(kt + 2, kb2, kb1, d2, d1);
        step(kt + 3, kb3, kb2, d3, d2);
    }
    if (kt < n_kt) step(kt, kb0, kb3, d0, d3);
    if (kt + 1 < n_kt) step(kt + 1, kb1, kb0, d1, d0);
    if (kt + 2 < n_kt) step(kt + 2, kb2, kb1, d2, d1);
    // The copies issued past the last tile land in LDS: wait for them before
    // the block can end and its LDS go to another block.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    // The last products' results are read below by vector ALU and LDS
    // instructions: keep the matrix-core result latency covered whatever
    // path led here.
    asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");

    if constexpr (KS > 1) {
        // Splits 1 .. KS - 1 leave their partial dq in the tile buffers (one
        // TILE_F region per wave: block b of lane l at float4 b 64 + l), and
        // split 0 adds them in split order. Region r is slot r % KS of
        // buffer r / KS (16 D floats = one K tile each).
        asm volatile("s_barrier" ::: "memory");  // every wave is done with the tiles
        auto region = [&](int r) -> float* {
            const int o = (r % KS) * TILE_F;
            return r < KS ? kb0 + o : r < 2 * KS ? kb1 + o : r < 3 * KS ? kb2 + o : kb3 + o;
        };
        if (split > 0) {
            float4* p = reinterpret_cast<float4*>(region((split - 1) * 4 + wq));
#pragma unroll
            for (int b = 0; b < NB; ++b)
                p[b * 64 + lane] = make_float4(acc[0][b][0], acc[0][b][1], acc[0][b][2], acc[0][b][3]);
        }
        __syncthreads();
        if (split > 0) return;
#pragma unroll 1
        for (int s = 1; s < KS; ++s) {
            const float4* p = reinterpret_cast<const float4*>(region((s - 1) * 4 + wq));
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float4 x = p[b * 64 + lane];
                acc[0][b][0] += x.x;
                acc[0][b][1] += x.y;
                acc[0][b][2] += x.z;
                acc[0][b][3] += x.w;
            }
        }
    }

    const int qd = a.num_heads * D;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int jl = j_first + rt;
        if (jl >= a.win.count) break;  // wave-uniform: past the window
        const int qt = a.win.off + jl * a.win.stride;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = qt * k16Rows + 4 * g + r;
            if (row >= a.q_seq) continue;
            float* dst = dq + (size_t)row * qd + head * D + 4 * j;
#pragma unroll
            for (int h2 = 0; h2 < NB / 4; ++h2) {
                *reinterpret_cast<float4*>(dst + 64 * h2) = make_float4(
                    acc[rt][4 * h2 + 0][r] * a.scale, acc[rt][4 * h2 + 1][r] * a.scale,
                    acc[rt][4 * h2 + 2][r] * a.scale, acc[rt][4 * h2 + 3][r] * a.scale);
            }
        }
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

template <int D, int W, bool STORE>
hipError_t launch_dkdv16(long long grid, size_t lds, hipStream_t stream, const float* q,
                         const float* k, const float* v, const float* dout, const float* rowv,
                         float* dk, float* dv, float* ds, const BwdArgs& a) {
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(bwd_dkdv16_kernel<D, W, STORE>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    if (grid > 0) {
        hipLaunchKernelGGL((bwd_dkdv16_kernel<D, W, STORE>), dim3((unsigned)grid), dim3(64 * W),
                           lds, stream, q, k, v, dout, rowv, dk, dv, ds, a);
    }
    return hipSuccess;
}

template <int D, bool STORE>
hipError_t launch_dkdv16_any(size_t lds, hipStream_t stream, const float* q, const float* k,
                             const float* v, const float* dout, const float* rowv, float* dk,
                             float* dv, float* ds, const BwdArgs& a) {
    // Blocks of 4 waves (64 keys), two per compute unit: while one block's
    // waves wait at a barrier the other block's share each SIMD (8-wave
    // blocks, one per CU, measured ~1 ms slower on the 16K causal pass).
    const long long blocks =
        (long long)a.num_kv_heads * ((a.kv_len + 4 * k16Keys - 1) / (4 * k16Keys));
    return launch_dkdv16<D, 4, STORE>(blocks, lds, stream, q, k, v, dout, rowv, dk, dv, ds, a);
}

// Blocks of one dq-from-dS instance that the device holds at once.
template <int D, int RT, int KS>
long long dq_resident_blocks(int cus) {
    static const int per_cu = [] {
        int n = 0;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(
                   &n, reinterpret_cast<const void*>(bwd_dq_ds_kernel<D, RT, KS>), 256 * KS, 0) ==
                       hipSuccess
                   ? n
                   : 0;
    }();
    return (long long)per_cu * cus;
}

// The stored-dS path over windows of query tiles (one window when the
// workspace holds every tile; else n windows, window w taking the query tiles
// w, w + n, w + 2n, ..., so that each spans every row and its dk/dv blocks
// keep the single launch's spread of work): D_i once; per window the dk/dv
// kernel over the window's rows, storing the window's dS tiles (dk, dv written
// by the first window, whose grid covers every key, and added to by the later
// ones, which cover the keys their rows see), then dq of the window's rows
// from them.
template <int D>
hipError_t launch_bwd_stored(const float* q, const float* k, const float* v, const float* o,
                             const float* dout, const float* lse, float* dq, float* dk,
                             float* dv, float* delta, float* ds, const BwdArgs& a0,
                             int n_win, int cus, hipStream_t stream) {
    const long long n_pairs = (long long)a0.q_seq * a0.num_heads;
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((n_pairs + 15) / 16)), dim3(256), 0,
                       stream, o, dout, lse, delta, n_pairs);
    const int n_qt = ds_query_tiles(a0.ds);
    for (int w = 0; w < n_win; ++w) {
        BwdArgs a = a0;
        a.win = ds_window(n_qt, n_win, w);
        a.ds_tph = ds_win_tiles_per_head(a.ds, a.win);
        a.accumulate = w > 0 ? 1 : 0;
        // Keys the window's rows see; the first window covers every key (it
        // writes dk, dv, zero for keys no row sees).
        int keys = a.kv_len;
        if (w > 0 && a.causal) {
            const int qt_last = a.win.off + (a.win.count - 1) * a.win.stride;
            const long long hi = (long long)a.start_pos + min((qt_last + 1) * k16Rows, a.q_seq);
            keys = (int)(hi < a.kv_len ? hi : a.kv_len);
        }
        const long long blocks =
            (long long)a.num_kv_heads * ((keys + 4 * k16Keys - 1) / (4 * k16Keys));
        const hipError_t e =
            launch_dkdv16<D, 4, true>(blocks, 0, stream, q, k, v, dout, delta, dk, dv, ds, a);
        if (e != hipSuccess) return e;
        // dq: 4 query tiles per wave while that still gives two blocks per
        // CU, else one (2 per wave measured slower on the 16K causal pass in 9
        // windows), with the keys split 4 or 2 ways inside each block where
        // the device then holds the whole grid at once. A grid the device
        // holds at once takes its blocks in snake order.
        const int tiles = a.win.count;
        const auto rows = [&](int rt) { return (tiles + a.dq_rs * rt - 1) / (a.dq_rs * rt); };
        a.dq_rt = (long long)a.dq_n_head_blocks * rows(4) >= 2 * cus ? 4 : 1;
        a.dq_n_row_blocks = rows(a.dq_rt);
        const long long grid = (long long)a.dq_n_head_blocks * a.dq_n_row_blocks;
        const dim3 g1((unsigned)grid);
        if (a.dq_rt == 4) {
            a.dq_round = grid <= dq_resident_blocks<D, 4, 1>(cus) ? cus : 0;
            hipLaunchKernelGGL((bwd_dq_ds_kernel<D, 4, 1>), g1, dim3(256), 0, stream, k, ds, dq, a);
        } else if (grid <= dq_resident_blocks<D, 1, 4>(cus)) {
            a.dq_round = cus;
            hipLaunchKernelGGL((bwd_dq_ds_kernel<D, 1, 4>), g1, dim3(1024), 0, stream, k, ds, dq, a);
        } else if (grid <= dq_resident_blocks<D, 1, 2>(cus)) {
            a.dq_round = cus;
            hipLaunchKernelGGL((bwd_dq_ds_kernel<D, 1, 2>), g1, dim3(512), 0, stream, k, ds, dq, a);
        } else {
            a.dq_round = grid <= dq_resident_blocks<D, 1, 1>(cus) ? cus : 0;
            hipLaunchKernelGGL((bwd_dq_ds_kernel<D, 1, 1>), g1, dim3(256), 0, stream, k, ds, dq, a);
        }
    }
    return hipSuccess;
}

template <int D>
hipError_t launch_bwd_instance(const float* q, const float* k, const float* v, const float* o,
                               const float* dout, const float* lse, float* dq, float* dk,
                               float* dv, float* delta, const BwdArgs& a, hipStream_t stream) {
    const size_t tile_bytes = (size_t)kBN * D * sizeof(float);
    const size_t lds_dq = (size_t)a.ks * 2 * 2 * tile_bytes;  // per key split: 2 x (K, V)
    static const hipError_t attr1 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(bwd_dq_kernel<D>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)((D == 128 ? 2 : 4) * 2 * 2 * tile_bytes));
    if (attr1 != hipSuccess) return attr1;
    const long long g1 = (long long)a.n_head_blocks * a.n_row_blocks;
    if (g1 > 0) {
        hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((unsigned)g1), dim3(kBlock), lds_dq, stream,
                           q, k, v, o, dout, lse, dq, delta, a);
    }
    // With no query rows the dk/dv blocks walk no tiles and write zeros.
    const size_t lds16 = 0;  // static LDS
    return launch_dkdv16_any<D, false>(lds16, stream, q, k, v, dout, delta, dk, dv, nullptr, a);
}

}  // namespace

int backward_windows(const DsLayout& l, long long capacity, int max_win) {
    // The fewest interleaved windows (window w of n: query tiles w + j n) each
    // holding at most `capacity` tiles per head; 0 when more than max_win would
    // be needed. No window count below total / capacity can fit.
    const int n_qt = ds_query_tiles(l);
    if (n_qt == 0 || capacity < ds_tiles_in(l, n_qt - 1)) return 0;  // the longest tile alone
    const long long total = ds_tiles_per_head(l);
    const long long lower = (total + capacity - 1) / capacity;
    if (lower > max_win) return 0;
    for (int n = (int)(lower < 1 ? 1 : lower); n <= max_win && n <= n_qt; ++n) {
        bool fits = true;
        for (int w = 0; w < n && fits; ++w)
            fits = ds_win_tiles_per_head(l, ds_window(n_qt, n, w)) <= capacity;
        if (fits) return n;
    }
    return 0;
}

hipError_t launch_backward(const float* q, const float* k, const float* v, const float* o,
                           const float* dout, const float* lse, float* dq, float* dk, float* dv,
                           float* delta, float* ds, long long ds_capacity, const PrefillShape& s,
                           hipStream_t stream) {
    BwdArgs a;
    a.q_seq = s.q_seq;
    a.kv_len = s.kv_len;
    a.num_heads = s.num_heads;
    a.num_kv_heads = s.num_kv_heads;
    a.group = s.num_heads / s.num_kv_heads;
    a.causal = s.causal;
    a.start_pos = s.start_pos;
    a.qscale = s.scale * kLog2e;
    a.scale = s.scale;
    // dq block: heads of a GQA group x row strips x key splits = 4 waves; key
    // splits (as the forward's) only while the launch is short of two waves
    // per SIMD and each split keeps several key tiles.
    const long long base_waves = (long long)s.num_heads * ((s.q_seq + kBM - 1) / kBM);
    const int max_w = s.causal ? min(s.start_pos + s.q_seq, s.kv_len) : s.kv_len;
    const int key_tiles = (max_w + kBN - 1) / kBN;
    const int max_ks = s.head_dim == 128 ? 2 : 4;  // 2 buffers x (K, V) per split in 160 KB
    int ks = 1;
    const int cus = device_cu_count();
    while (ks < max_ks && base_waves * ks < (long long)kWavesPerCU * cus &&
           key_tiles >= 4 * ks * 2)
        ks *= 2;
    a.ks = ks;
    a.hg = gcd_int(a.group, kWaves / ks);
    a.rs = kWaves / (ks * a.hg);
    a.n_head_blocks = s.num_heads / a.hg;
    a.n_row_blocks = (s.q_seq + a.rs * kBM - 1) / (a.rs * kBM);
    a.ds = DsLayout{s.causal, s.start_pos, s.q_seq, s.kv_len};
    const int n_qt = ds_query_tiles(a.ds);
    a.win = ds_window(n_qt, 1, 0);
    a.ds_tph = ds_tiles_per_head(a.ds);
    a.accumulate = 0;
    a.dq_hg = gcd_int(a.group, kWaves);
    a.dq_rs = kWaves / a.dq_hg;
    a.dq_n_head_blocks = s.num_heads / a.dq_hg;
    a.dq_rt = 1;
    a.dq_n_row_blocks = 0;
    a.dq_round = 0;
    // The stored path pays once the dq grid from the tiles fills the compute
    // units (one block of 4 waves per CU with 4 query tiles per wave);
    // shorter calls recompute. With fewer tiles than the call has, the stored
    // path runs in windows (at most kMaxBwdWindows when chosen by size). A testing
    // override forces either path (the stored one whenever a window of one
    // query tile fits).
    const int force = override_bwd_path();
    const auto dq_blocks = [&](int rt) {
        return (long long)a.dq_n_head_blocks * ((n_qt + a.dq_rs * rt - 1) / (a.dq_rs * rt));
    };
    const bool big = dq_blocks(dq_blocks(4) >= 2 * cus ? 4 : 1) >= cus;
    const bool use_ds = force != 0 ? force == 1 : big;
    hipError_t e;
    if (ds != nullptr && use_ds && s.q_seq > 0 && s.kv_len > 0) {
        const int n_win = backward_windows(a.ds, ds_capacity, force == 1 ? 4096 : kMaxBwdWindows);
        if (n_win > 0) {
            e = s.head_dim == 128
                ? launch_bwd_stored<128>(q, k, v, o, dout, lse, dq, dk, dv, delta, ds, a, n_win,
                                         cus, stream)
                : launch_bwd_stored<64>(q, k, v, o, dout, lse, dq, dk, dv, delta, ds, a, n_win,
                                        cus, stream);
            if (e != hipSuccess) return e;
            return hipGetLastError();
        }
    }
    if (s.head_dim == 128) {
        e = launch_bwd_instance<128>(q, k, v, o, dout, lse, dq, dk, dv, delta, a, stream);
    } else {
        e = launch_bwd_instance<64>(q, k, v, o, dout, lse, dq, dk, dv, delta, a, stream);
    }
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

}  // namespace ta03
