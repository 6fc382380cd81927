// Internal launch interface between the C ABI (ta03_api.cpp) and the HIP
// kernels. Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ta03 {

// Compute units of the current device, queried once per device
// (hipDeviceAttributeMultiprocessorCount) and cached; 256 if no device
// answers. The launch heuristics (key splits, kernel choice, split counts)
// size their grids with it.
int device_cu_count();

// Kernel-choice overrides set through attn_set_kernel_override (testing
// only: every shape can be run through each kernel). 0 = automatic.
//   prefill_rows: 16 or 32 forces the 16-row or the 32-row prefill kernel;
//   bwd_path: 1 stored dS (when the workspace holds every tile), 2 the
//   recompute path.
int override_prefill_rows();
int override_bwd_path();

// Fourth word of the raw buffer resources the kernels build
// (__builtin_amdgcn_make_buffer_rsrc): 32-bit data format, for untyped loads.
constexpr int kBufferFlags = 0x00020000;

struct PrefillShape {
    int q_seq, kv_len, num_heads, num_kv_heads, head_dim;
    int causal, start_pos;  // start_pos: causal position of row 0 of q/out
    float scale;
    long long q_stride, k_stride, v_stride, out_stride;  // row strides in floats
    // Rotary (cos, sin) table [positions][head_dim/2][2]; nullptr: no rotation.
    const float* rope_cs = nullptr;
    // With a table: rotate the keys as they are loaded (else they are taken
    // as given, already rotated, and only the queries turn).
    bool rope_keys = true;
};

struct DecodeShape {
    int num_heads, num_kv_heads, head_dim, max_seq;
    float scale;
};

// Split-KV plan of the decode path; a pure function of the sizes and the
// block count aimed at (the device's compute units), so that the workspace
// query and the launch agree on one device.
struct DecodePlan {
    int group;           // query heads per KV head
    int heads_per_blk;   // query heads one block serves (<= 4)
    int blks_per_kv;     // blocks per KV head along the head axis
    int n_splits;        // splits of the cache axis
    size_t n_counters;   // words of the counter region at the workspace start: one ticket
                         // per (kv head, head block), each in its own 256-byte slot
    size_t part_offset;  // floats from the workspace start to the split partials
    size_t ws_floats;    // workspace size in floats
};

DecodePlan decode_plan(const DecodeShape& s, int target_blocks);

hipError_t launch_prefill(const float* q, const float* k, const float* v, float* out,
                          float* lse, const PrefillShape& s, hipStream_t stream);

// 16-row variant for launches with few query rows (no rotation); chosen by
// launch_prefill when the 32-row kernel would launch fewer blocks than there
// are compute units, or forced by override_prefill_rows().
hipError_t launch_prefill16(const float* q, const float* k, const float* v, float* out,
                            float* lse, const PrefillShape& s, hipStream_t stream);
// The 16-row kernel addresses a key tile's rows with 32-bit byte offsets:
// K and V row strides below 2^25 floats.
inline bool prefill16_fits(const PrefillShape& s) {
    return s.k_stride < (1ll << 25) && s.v_stride < (1ll << 25);
}

// Attention backward (dense rows): dq [q_seq, H*d]; dk, dv [kv_len, Hkv*d];
// delta: 2*q_seq*H floats of scratch (per row and head: -D_i with
// D_i = <dout_i, out_i>, then the exponent offset -(m + log l) log2 e).
// Stored score gradients of the backward: dS in 16 x 16 tiles (query rows x
// keys, row-major, 1 KiB each), one run of tiles per head, and inside a head
// the tiles of query tile qt (rows [16 qt, 16 qt + 16)) for key tiles
// kt < tiles_in(qt) one after another. tiles_in(qt) covers the keys of the
// tile's last row window: causal min(start_pos + min(16 qt + 16, q_seq),
// kv_len), else kv_len. A causal call has start_pos + q_seq <= kv_len, so
// every query tile but the last holds qt + 1 + ceil(start_pos / 16) tiles
// and the tiles before qt sum in closed form. Host (workspace size) and
// device (addresses) use these same functions.
struct DsLayout {
    int causal, start_pos, q_seq, kv_len;
};
constexpr int kDsTile = 16;
__host__ __device__ inline int ds_query_tiles(const DsLayout& l) {
    return (l.q_seq + kDsTile - 1) / kDsTile;
}
__host__ __device__ inline int ds_tiles_in(const DsLayout& l, int qt) {
    if (!l.causal) return (l.kv_len + kDsTile - 1) / kDsTile;
    const int rows_hi = (qt + 1) * kDsTile < l.q_seq ? (qt + 1) * kDsTile : l.q_seq;
    long long w = (long long)l.start_pos + rows_hi;
    if (w > l.kv_len) w = l.kv_len;
    return (int)((w + kDsTile - 1) / kDsTile);
}
__host__ __device__ inline long long ds_tiles_before(const DsLayout& l, int qt) {
    if (!l.causal) return (long long)qt * ((l.kv_len + kDsTile - 1) / kDsTile);
    const long long c = (l.start_pos + kDsTile - 1) / kDsTile;
    return (long long)qt * (qt + 1) / 2 + c * qt;
}
__host__ __device__ inline long long ds_tiles_per_head(const DsLayout& l) {
    const int n = ds_query_tiles(l);
    return n == 0 ? 0 : ds_tiles_before(l, n - 1) + ds_tiles_in(l, n - 1);
}

// A window of the stored path: query tiles off + j * stride, j < count (the
// whole call: off 0, stride 1, count = all query tiles). Its tiles are laid
// out per head as in DsLayout over the window's own query tiles: those of
// local tile j after the tiles of local tiles 0 .. j - 1. Every local tile
// but the window's last lies before the call's last query tile, so in a
// causal call it holds qt + 1 + ceil(start_pos / 16) tiles and the sum has a
// closed form.
struct DsWindow {
    int off, stride, count;
};
__host__ __device__ inline long long ds_win_tiles_before(const DsLayout& l, const DsWindow& w,
                                                         int j) {  // j < count
    if (!l.causal) return (long long)j * ((l.kv_len + kDsTile - 1) / kDsTile);
    const long long c = (l.start_pos + kDsTile - 1) / kDsTile;
    return (long long)j * (w.off + 1 + c) + (long long)w.stride * j * (j - 1) / 2;
}
__host__ __device__ inline long long ds_win_tiles_per_head(const DsLayout& l, const DsWindow& w) {
    if (w.count == 0) return 0;
    const int last = w.count - 1;  // the window's last tile counts its own keys
    return ds_win_tiles_before(l, w, last) + ds_tiles_in(l, w.off + last * w.stride);
}
// Window w of n interleaved windows over n_qt query tiles (w < n <= n_qt).
__host__ __device__ inline DsWindow ds_window(int n_qt, int n, int w) {
    return DsWindow{w, n, (n_qt - w + n - 1) / n};
}

// ds == nullptr (or a capacity below the tiles of one query tile): dq
// recomputes the scores (two launches). Otherwise the dk/dv kernel stores dS
// tiles in `ds`, which holds ds_capacity tiles per head, and dq is computed
// from them: in one window when every tile fits, else in n windows of
// interleaved query tiles (window w: tiles w, w + n, w + 2n, ...), each laid
// out as DsWindow says.
hipError_t launch_backward(const float* q, const float* k, const float* v, const float* o,
                           const float* dout, const float* lse, float* dq, float* dk, float* dv,
                           float* delta, float* ds, long long ds_capacity, const PrefillShape& s,
                           hipStream_t stream);

// The fewest interleaved windows whose tiles each fit `capacity` tiles per
// head (1: every tile at once); 0 when none up to max_win do.
int backward_windows(const DsLayout& l, long long capacity, int max_win);
// Windows chosen by size: each window past the first costs a dk/dv and a dq
// launch (on the 16K causal pass ~0.1-0.35 ms up to 16 windows, ~0.6 ms
// beyond, where a window's dq lasts as long as its heaviest block; 32 windows
// take 52.6 ms against 57.6 ms recomputing the scores).
constexpr int kMaxBwdWindows = 32;

// Rotary table: entry (p, e) = (cos, sin) of p * theta^(-2e/head_dim).
hipError_t launch_rope_table(float* cs, int rows, int head_dim, double theta, hipStream_t stream);
hipError_t launch_rope_apply(const float* x, long long x_stride, float* y, long long y_stride,
                             int rows, int heads, int head_dim, int pos0, const float* cs,
                             hipStream_t stream);

hipError_t launch_decode_ws_init(float* ws, const DecodePlan& p, hipStream_t stream);

// Fixed-size device scratch of the allocation-free decode (4 MiB per device):
// a counter region of kNoallocCounterWords words (256 ticket slots of 64
// words), then at most kNoallocScratchFloats - kNoallocCounterWords floats of
// split partials.
constexpr size_t kNoallocScratchFloats = (size_t)1 << 20;
constexpr size_t kNoallocCounterWords = 256 * 64;
// The current device's scratch (its device address, looked up once per
// device; the first call also enqueues the zero fill of its counters on
// `stream`).
hipError_t noalloc_scratch(hipStream_t stream, float** ptr);

// Dynamic LDS a paged decode launch needs for its page-table slice.
size_t decode_table_lds_bytes(const DecodeShape& s, const DecodePlan& p, int page_size);

// table == nullptr: one dense cache of max_seq rows; otherwise k/v are page
// pools of num_pages pages of page_size rows and table maps token blocks to
// pages.
hipError_t launch_decode(const float* q, const float* k, const float* v,
                         const uint32_t* kv_pos, float* out, float* lse,
                         const DecodeShape& s, const DecodePlan& p, float* ws,
                         hipStream_t stream, const int* table = nullptr, int page_size = 0,
                         int num_pages = 0);

}  // namespace ta03
